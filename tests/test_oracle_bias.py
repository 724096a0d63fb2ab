"""Pins of the oracle's column-parallel bias (Z_i = bf16(GeLU(X·A_i + b1_i))),
on the CPU: a zero bias is the unbiased step, a zero input reduces the step
to the elementwise GeLU of the bias, an exact rational brute force on tiny
shapes, and the biased shards summing (plus the second bias, once) to the
unsharded block."""
from fractions import Fraction

import numpy as np
import pytest

import brute
import oracle
from workloads import bf16_bits_from_f32, make_bias, make_random


def _rel_maxdiff(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def test_zero_bias_is_the_unbiased_step():
    X, A, _ = make_random(24, 32, 64, seed=51, sigma=0.3)
    zero = np.zeros(64, dtype=np.uint16)
    assert np.array_equal(oracle.col_gelu_bias(X, A, zero), oracle.col_gelu(X, A))
    # -0.0 is a zero too
    nzero = np.full(64, 0x8000, dtype=np.uint16)
    assert np.array_equal(oracle.col_gelu_bias(X, A, nzero), oracle.col_gelu(X, A))


def test_zero_input_gives_the_gelu_of_the_bias():
    """X = 0: every row of Z_i is bf16(GeLU(b1_i)), each value against
    math.erfc and an exact round to the bf16 grid."""
    F = 48
    b = make_bias(F, seed=52, sigma=2.0)
    X = np.zeros((5, 16), dtype=np.uint16)
    _, A, _ = make_random(5, 16, F, seed=53, sigma=0.3)
    Z = oracle.bf16_decode(oracle.col_gelu_bias(X, A, b))
    for j in range(F):
        want = float(brute.bf16_round(Fraction(brute.gelu_float(float(brute.bf16_value(int(b[j])))))))
        assert np.all(Z[:, j] == want), f"column {j}: {Z[0, j]} != GeLU(b) = {want}"


@pytest.mark.parametrize("M,d,H,N,seed", [
    (3, 4, 16, 1, 60), (5, 8, 16, 2, 61), (7, 16, 16, 4, 62), (9, 5, 12, 3, 63), (1, 16, 16, 4, 64),
])
def test_biased_step_matches_brute_force(M, d, H, N, seed):
    X, A, B = make_random(M, d, H, seed, sigma=0.5)
    b1 = make_bias(H, seed, sigma=1.0)
    for rank in range(N):
        Zb, Yb = brute.shard_bias_exact(X, A, b1, B, N, rank)
        lo, hi = rank * (H // N), (rank + 1) * (H // N)
        Z = oracle.bf16_decode(oracle.col_gelu_bias(X, A[:, lo:hi], b1[lo:hi]))
        Zb_f = np.array([[float(v) for v in row] for row in Zb])
        assert np.array_equal(Z, Zb_f), f"rank {rank}: Z differs from the brute force"
        Y = oracle.mlp_shard_bias(X, A, b1, B, N, rank)
        Yb_f = np.array([[float(v) for v in row] for row in Yb])
        assert _rel_maxdiff(Y, Yb_f) <= 1e-13, f"rank {rank}: Y differs from the brute force"


@pytest.mark.parametrize("M,d,N,seed", [(32, 64, 2, 70), (17, 32, 8, 71), (5, 24, 3, 72)])
def test_biased_shards_sum_to_the_unsharded_block(M, d, N, seed):
    """Σ_i Z_i·B_i + b2 = bf16(GeLU(X·A + b1))·B + b2: each rank adds its own
    block of b1 before GeLU, and b2 is added once, after the sum."""
    X, A, B = make_random(M, d, 4 * d, seed, sigma=0.1)
    b1 = make_bias(4 * d, seed, sigma=0.5)
    b2 = make_bias(d, seed + 1000, sigma=0.5)
    parts = [oracle.mlp_shard_bias(X, A, b1, B, N, r) for r in range(N)]
    Y = oracle.partial_sum_rows(parts, 0, M, oracle.bf16_decode(b2))
    Yfull = oracle.mlp_unsharded_bias(X, A, b1, B, b2)
    assert _rel_maxdiff(Y, Yfull) <= 1e-12
    # the bias moves the result: the unbiased block is far from it
    assert _rel_maxdiff(oracle.mlp_unsharded(X, A, B), Yfull) > 1e-2


def test_bias_shape_is_checked():
    X, A, B = make_random(4, 8, 32, seed=73)
    with pytest.raises(ValueError):
        oracle.mlp_shard_bias(X, A, make_bias(31, 73), B, 2, 0)


# ------------------------------------------------------------- backward --

def _dy(M, d, seed):
    return bf16_bits_from_f32(np.random.default_rng(seed).standard_normal((M, d)).astype(np.float32))


def test_backward_with_a_zero_bias_is_the_unbiased_backward():
    X, A, B = make_random(6, 16, 32, seed=80, sigma=0.3)
    dY = _dy(6, 16, 81)
    g0 = oracle.mlp_shard_backward(X, A, B, dY, 2, 1)
    gb = oracle.mlp_shard_backward(X, A, B, dY, 2, 1, b1_bits=np.zeros(32, np.uint16))
    for k in ("S", "Z_bits", "dS_bits", "dX", "dA", "dB"):
        assert np.array_equal(g0[k], gb[k]), k
    assert np.array_equal(gb["db1"], oracle.bf16_decode(gb["dS_bits"]).sum(axis=0))


@pytest.mark.parametrize("N,rank", [(1, 0), (2, 1), (4, 2)])
def test_backward_bias_gradients_match_finite_differences(N, rank):
    """The unrounded chain rule against central finite differences of
    L = Σ (Y ⊙ dY) with Y = GeLU(X·A_i + b1_i)·B_i + b2, with respect to every
    entry of b1_i, b2, X and A_i."""
    M, d, H = 3, 4, 16
    X, A, B = make_random(M, d, H, 82 + N, sigma=0.5)
    b1 = make_bias(H, 82 + N, sigma=0.7)
    dY = _dy(M, d, 83)
    g = oracle.mlp_shard_backward(X, A, B, dY, N, rank, rounding=False, b1_bits=b1)
    lo, hi = oracle.shard_columns(H, N, rank)
    Xv, Av, Bv, dYv = (oracle.bf16_decode(t) for t in (X, A[:, lo:hi], B[lo:hi, :], dY))
    b1v, b2v = oracle.bf16_decode(b1)[lo:hi], np.linspace(-1, 1, d)

    def loss(x, a, c1, c2):
        return float(np.sum((oracle.gelu(x @ a + c1[None, :]) @ Bv + c2[None, :]) * dYv))
    h = 1e-6
    base = {"X": Xv, "A": Av, "b1": b1v, "b2": b2v}
    grads = {"X": g["dX"], "A": g["dA"], "b1": g["db1"], "b2": g["db2"]}
    for name, v in base.items():
        num = np.zeros_like(v)
        for idx in np.ndindex(v.shape):
            p, m = dict(base), dict(base)
            p[name], m[name] = v.copy(), v.copy()
            p[name][idx] += h
            m[name][idx] -= h
            num[idx] = (loss(p["X"], p["A"], p["b1"], p["b2"])
                        - loss(m["X"], m["A"], m["b1"], m["b2"])) / (2 * h)
        assert grads[name].shape == v.shape
        assert _rel_maxdiff(grads[name], num) <= 1e-6, name


def test_fp8_backward_with_a_zero_bias_is_the_unbiased_fp8_backward():
    X, A, B = make_random(32, 64, 256, seed=84, sigma=0.05)
    dY = _dy(32, 64, 85)
    g0 = oracle.mlp_shard_backward_fp8(X, A, B, dY, 2, 1)
    gb = oracle.mlp_shard_backward_fp8(X, A, B, dY, 2, 1, b1_bits=np.zeros(256, np.uint16))
    for k in ("S", "dS_bits", "Z_bits", "dSq", "Zq", "dX", "dA", "dB"):
        assert np.array_equal(g0[k], gb[k]), k


def test_fp8_backward_bias_enters_s_and_sums_ds():
    """The bias moves the dequantised S by exactly its block (float64 sums of
    exactly representable values), and db1 / db2 are the column sums of the
    bf16 dS and dY; against the bf16 oracle's bias gradients the fp8 ones
    differ by the quantisation only."""
    M, d, H, N, rank = 32, 64, 256, 4, 2
    X, A, B = make_random(M, d, H, seed=86, sigma=0.05)
    dY = _dy(M, d, 87)
    b1 = make_bias(H, seed=88, sigma=0.5)
    g0 = oracle.mlp_shard_backward_fp8(X, A, B, dY, N, rank)
    gb = oracle.mlp_shard_backward_fp8(X, A, B, dY, N, rank, b1_bits=b1)
    lo, hi = oracle.shard_columns(H, N, rank)
    assert np.array_equal(gb["S"] - g0["S"],
                          np.broadcast_to(oracle.bf16_decode(b1)[lo:hi], (M, hi - lo))) or \
        np.max(np.abs(gb["S"] - g0["S"] - oracle.bf16_decode(b1)[lo:hi][None, :])) <= 1e-15
    assert np.array_equal(gb["db1"], oracle.bf16_decode(gb["dS_bits"]).sum(axis=0))
    assert np.array_equal(gb["db2"], oracle.bf16_decode(dY).sum(axis=0))
    g16 = oracle.mlp_shard_backward(X, A, B, dY, N, rank, b1_bits=b1)
    assert np.array_equal(gb["db2"], g16["db2"])
    assert _rel_maxdiff(gb["db1"], g16["db1"]) <= 0.1


# plausible mistakes, each planted in the oracle, fail at least one pin above
def _pins_fail():
    for fn in (test_zero_bias_is_the_unbiased_step, test_zero_input_gives_the_gelu_of_the_bias,
               lambda: test_biased_step_matches_brute_force(7, 16, 16, 4, 62),
               lambda: test_biased_shards_sum_to_the_unsharded_block(17, 32, 8, 71)):
        try:
            fn()
        except AssertionError:
            return True
    return False


def _after_gelu(X, A, b):
    Z = oracle.gelu(oracle.bf16_decode(X) @ oracle.bf16_decode(A)) + oracle.bf16_decode(b)[None, :]
    return oracle.bf16_encode(Z)


def _bias_subtracted(X, A, b):
    S = oracle.bf16_decode(X) @ oracle.bf16_decode(A) - oracle.bf16_decode(b)[None, :]
    return oracle.bf16_encode(oracle.gelu(S))


def _bias_dropped(X, A, b):
    return oracle.col_gelu(X, A)


def _whole_bias_first_block(X, A, b):
    # a rank taking the first block of the bias whatever its columns: here the
    # reversed block stands in, so a shard gets columns of the wrong positions
    S = oracle.bf16_decode(X) @ oracle.bf16_decode(A)
    return oracle.bf16_encode(oracle.gelu(S + oracle.bf16_decode(b[::-1])[None, :]))


@pytest.mark.parametrize("mutant", [_after_gelu, _bias_subtracted, _bias_dropped,
                                    _whole_bias_first_block])
def test_bias_mutant_is_caught(mutant, monkeypatch):
    from oracle import mlp as omlp
    monkeypatch.setattr(omlp, "col_gelu_bias", mutant)
    monkeypatch.setattr(oracle, "col_gelu_bias", mutant)
    assert _pins_fail(), f"{mutant.__name__} passed every pin"


# -- the biased fp8 backward pinned to the biased bf16 backward ------------------
# With integer inputs whose largest magnitude is 7, every scale is a power of
# two (448/7 = 2^6 for e4m3, 57344/7 = 2^13 for e5m2) and every quantised code
# is exact, so the fp8 backward computes the bf16 backward's S, dZ, dS and Z;
# with the column bias (bf16, never quantised) it must then also match its
# bias gradients. The bf16 biased backward is pinned by central differences
# above, so this ties the fp8 bias path to the chain rule.

def _sevens(M, d, H, seed):
    rng = np.random.default_rng(seed)
    out = []
    for shape in ((M, d), (d, H), (H, d), (M, d)):
        v = rng.integers(-7, 8, size=shape).astype(np.float32)
        v.flat[rng.integers(0, v.size)] = 7.0 * (1 if rng.integers(2) else -1)   # amax exactly 7
        out.append(bf16_bits_from_f32(v))
    return out


def _fp8_bias_pin(M=24, d=32, H=128, N=4, rank=1, seed=90):
    X, A, B, dY = _sevens(M, d, H, seed)
    b1 = make_bias(H, seed=seed + 1, sigma=2.0)
    g8 = oracle.mlp_shard_backward_fp8(X, A, B, dY, N, rank, b1_bits=b1)
    assert (g8["sX"], g8["sA"], g8["sB"], g8["sdY"]) == (64.0, 64.0, 64.0, 8192.0)
    g16 = oracle.mlp_shard_backward(X, A, B, dY, N, rank, b1_bits=b1)
    for k8, k16 in (("S", "S"), ("dZ", "dZ")):
        assert np.array_equal(g8[k8], g16[k16]), k8
    assert np.array_equal(oracle.bf16_decode(g8["dS_bits"]), g16["dS"]), "dS"
    assert np.array_equal(oracle.bf16_decode(g8["Z_bits"]), g16["Z"]), "Z"
    assert np.array_equal(g8["db1"], g16["db1"]), "db1"
    assert np.array_equal(g8["db2"], g16["db2"]), "db2"


def test_fp8_backward_with_bias_equals_bf16_backward_on_exact_codes():
    _fp8_bias_pin()
    _fp8_bias_pin(M=40, d=48, H=96, N=3, rank=2, seed=91)


_real_fp8_bwd = oracle.mlp_shard_backward_fp8


def _db1_from_e5m2(X, A, B, dY, N, rank, b1_bits=None):
    g = _real_fp8_bwd(X, A, B, dY, N, rank, b1_bits=b1_bits)
    if b1_bits is not None:
        g["db1"] = (oracle.e5m2_decode(g["dSq"]) / float(g["sdS"])).sum(axis=0)
    return g


def _bias_quantised(X, A, B, dY, N, rank, b1_bits=None):
    if b1_bits is None:
        return _real_fp8_bwd(X, A, B, dY, N, rank)
    q, s = oracle.quantize_inputs_e4m3(b1_bits)
    b1q = bf16_bits_from_f32((oracle.e4m3_decode(q) / float(s)).astype(np.float32))
    return _real_fp8_bwd(X, A, B, dY, N, rank, b1_bits=b1q)


def _bias_before_dequantising(X, A, B, dY, N, rank, b1_bits=None):
    if b1_bits is None:
        return _real_fp8_bwd(X, A, B, dY, N, rank)
    # S = (Xq·Aq + b1)/(sX·sA): the bias divided by the scales' product
    sX = oracle.quantize_inputs_e4m3(X)[1]
    sA = oracle.quantize_inputs_e4m3(A)[1]
    b = oracle.bf16_decode(b1_bits) / (float(sX) * float(sA))
    return _real_fp8_bwd(X, A, B, dY, N, rank, b1_bits=bf16_bits_from_f32(b.astype(np.float32)))


@pytest.mark.parametrize("mutant", [_db1_from_e5m2, _bias_quantised, _bias_before_dequantising])
def test_fp8_bias_mutant_is_caught(mutant, monkeypatch):
    monkeypatch.setattr(oracle, "mlp_shard_backward_fp8", mutant)
    with pytest.raises(AssertionError):
        _fp8_bias_pin()
