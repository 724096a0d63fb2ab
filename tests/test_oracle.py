"""Pins for the oracle (CPU only): it is checked against things other than
itself - an exact rational brute force, the pages' closed form, textbook
values of the normal CDF, structured inputs that reduce the path to a known
function, and the pages' printed TP=2 shard map.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import brute
import oracle
from oracle import mlp as omlp
from workloads import WORKLOADS, make_inputs, make_random, bf16_bits_from_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _table(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                out.append(line.split())
    return out


def _rel_maxdiff(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------- GeLU ----

def test_gelu_matches_normal_table():
    for x, phi, tol in _table("normal_cdf.txt"):
        x, phi, tol = float(x), float(phi), float(tol)
        g = float(oracle.gelu(np.array([x]))[0])
        if x == 0:
            assert g == 0.0
        else:
            assert abs(g / x - phi) <= tol, (x, g / x, phi)


def test_gelu_identities():
    x = np.linspace(-12, 12, 20001)
    g = oracle.gelu(x)
    # Φ(−x) = 1 − Φ(x)  =>  GeLU(x) − GeLU(−x) = x
    assert np.max(np.abs(g - oracle.gelu(-x) - x)) <= 4e-15 * 12
    assert oracle.gelu(np.array([0.0]))[0] == 0.0
    big = x[x >= 10]
    assert np.all(np.abs(oracle.gelu(big) / big - 1) < 1e-22 + 1e-15)
    neg = x[x <= -10]
    gn = oracle.gelu(neg)
    assert np.all(gn <= 0) and np.all(np.abs(gn) < 1e-20)
    # far tail is accurate (no cancellation): x·Φ(x) with Φ(−10) ≈ 7.62e-24
    assert abs(oracle.gelu(np.array([-10.0]))[0] / (-10 * 7.619853024160527e-24) - 1) < 1e-12


def test_gelu_matches_math_erf_dense_grid():
    x = np.linspace(-10, 10, 4001)
    ref = np.array([v * 0.5 * (1 + math.erf(v / math.sqrt(2))) for v in x])
    assert np.max(np.abs(oracle.gelu(x) - ref)) < 1e-14


# ----------------------------------------------------------- shard map ----

def test_shard_map_matches_tp2_example():
    for d, N, rank, lo, hi in _table("tp2_shard_map.txt"):
        d, N, rank, lo, hi = map(int, (d, N, rank, lo, hi))
        assert oracle.shard_columns(4 * d, N, rank) == (lo, hi)


def test_shard_map_partitions_and_errors():
    for H, N in [(256, 1), (256, 2), (256, 8), (16384, 8), (3072, 3)]:
        blocks = [oracle.shard_columns(H, N, r) for r in range(N)]
        assert blocks[0][0] == 0 and blocks[-1][1] == H
        assert all(blocks[r][1] == blocks[r + 1][0] for r in range(N - 1))
        assert len({hi - lo for lo, hi in blocks}) == 1
    with pytest.raises(ValueError):
        oracle.shard_columns(256, 3, 0)       # 4d not divisible by N
    with pytest.raises(ValueError):
        oracle.shard_columns(256, 2, 2)       # rank out of range
    with pytest.raises(ValueError):
        oracle.shard_columns(256, 0, 0)


# --------------------------------------------------------- brute force ----

def _check_against_brute(X, A, B, N):
    for rank in range(N):
        Y, Z = oracle.mlp_shard(X, A, B, N, rank, return_z=True)
        Zb, Yb = brute.shard_exact(X, A, B, N, rank)
        Zb_f = np.array([[float(z) for z in row] for row in Zb])
        Yb_f = np.array([[float(y) for y in row] for row in Yb])
        assert np.array_equal(oracle.bf16_decode(Z), Zb_f), f"Z mismatch at rank {rank}"
        assert _rel_maxdiff(Y, Yb_f) <= 1e-13, f"Y mismatch at rank {rank}"


def test_tiny_tp2_matches_brute_force():
    X, A, B = make_inputs("tiny_tp2")
    _check_against_brute(X, A, B, 2)


@pytest.mark.parametrize("M,d,H,N,seed", [
    (3, 4, 16, 1, 10), (5, 8, 16, 2, 11), (7, 16, 16, 4, 12), (16, 12, 8, 2, 13),
    (1, 16, 16, 4, 14), (9, 5, 12, 3, 15),
])
def test_random_tiny_matches_brute_force(M, d, H, N, seed):
    # wider spread of A so GeLU sees large positive and negative arguments
    X, A, B = make_random(M, d, H, seed, sigma=0.5)
    _check_against_brute(X, A, B, N)


# --------------------------------------------------------- closed form ----

@pytest.mark.parametrize("M,d,N,seed", [(32, 64, 2, 0), (40, 48, 4, 21), (17, 32, 8, 22),
                                        (64, 128, 8, 23), (5, 24, 3, 24)])
def test_sum_of_shards_equals_unsharded(M, d, N, seed):
    """Output = Z·W2 = Σ_i Z_i·W2_i = Σ_i Y_i ("Megatron-LM deep architecture",
    eq. for Output)."""
    X, A, B = make_random(M, d, 4 * d, seed)
    parts = [oracle.mlp_shard(X, A, B, N, r) for r in range(N)]
    Ysum = oracle.partial_sum(parts)
    Yfull = oracle.mlp_unsharded(X, A, B)
    assert _rel_maxdiff(Ysum, Yfull) <= 1e-12


def test_tiny_tp2_closed_form():
    X, A, B = make_inputs("tiny_tp2")
    Y0 = oracle.mlp_shard(X, A, B, 2, 0)
    Y1 = oracle.mlp_shard(X, A, B, 2, 1)
    assert _rel_maxdiff(Y0 + Y1, oracle.mlp_unsharded(X, A, B)) <= 1e-12


def test_n1_is_unsharded():
    X, A, B = make_random(24, 32, 128, 5)
    assert np.array_equal(oracle.mlp_shard(X, A, B, 1, 0), oracle.mlp_unsharded(X, A, B))


def test_partial_sum_rank_order_and_errors():
    parts = [np.full((2, 2), 1e16), np.ones((2, 2)), np.full((2, 2), -1e16)]
    # (1e16 + 1) - 1e16 in float64 loses the 1: rank order is what is summed
    assert np.all(oracle.partial_sum(parts) == 0.0)
    with pytest.raises(ValueError):
        oracle.partial_sum([])


# ------------------------------------- sequence-parallel share and bias ----

def _tiny_parts(N, M=32, d=64, H=256, seed=40):
    X, A, B = make_random(M, d, H, seed)
    return X, A, B, [oracle.mlp_shard(X, A, B, N, r) for r in range(N)]


@pytest.mark.parametrize("N", [2, 4, 8])
def test_all_gather_of_reduce_scatter_is_all_reduce(N):
    # AllReduce(Y) = AllGather(ReduceScatter(Y)): the N shares, stacked in
    # rank order, are the full sum, element for element
    _, _, _, parts = _tiny_parts(N)
    shares = [oracle.reduce_scatter_share(parts, r) for r in range(N)]
    assert all(s.shape == (32 // N, 64) for s in shares)
    assert np.array_equal(np.concatenate(shares, axis=0), oracle.partial_sum(parts))


def test_reduce_scatter_shares_sum_to_unsharded_output():
    X, A, B, parts = _tiny_parts(4)
    full = np.concatenate([oracle.reduce_scatter_share(parts, r) for r in range(4)])
    assert _rel_maxdiff(full, oracle.mlp_unsharded(X, A, B)) <= 1e-12


def test_bias_added_once_after_the_sum_brute_force():
    # each element against an exact rational sum of its partials plus one bias
    rng = np.random.default_rng(41)
    N, M, d = 3, 6, 16
    parts = [rng.standard_normal((M, d)) for _ in range(N)]
    bias = rng.standard_normal(d)
    for rank in range(N):
        got = oracle.reduce_scatter_share(parts, rank, bias)
        lo = rank * (M // N)
        for r in range(M // N):
            for c in range(d):
                exact = sum(Fraction(float(p[lo + r, c])) for p in parts) + Fraction(float(bias[c]))
                assert abs(Fraction(float(got[r, c])) - exact) <= Fraction(1, 2 ** 48) * max(1, abs(exact))


def test_partial_sum_rows_ranges_and_errors():
    _, _, _, parts = _tiny_parts(2)
    full = oracle.partial_sum(parts)
    assert np.array_equal(oracle.partial_sum_rows(parts, 5, 19), full[5:19])
    assert oracle.partial_sum_rows(parts, 7, 7).shape == (0, 64)
    with pytest.raises(ValueError):
        oracle.partial_sum_rows(parts, 10, 40)
    with pytest.raises(ValueError):
        oracle.sp_rows(30, 4, 0)           # rows not divisible by N
    with pytest.raises(ValueError):
        oracle.sp_rows(32, 4, 4)
    assert oracle.sp_rows(8192, 8, 7) == (7168, 8192)


# ---------------------------------------------------- structured inputs ----

def test_zero_input_gives_zero():
    _, A, B = make_random(8, 16, 64, 3)
    X = np.zeros((8, 16), np.uint16)
    for r in range(4):
        Y = oracle.mlp_shard(X, A, B, 4, r)
        assert np.all(Y == 0.0)


def test_identity_weights_reduce_to_elementwise_gelu():
    d, M = 16, 10
    rng = np.random.default_rng(4)
    X = bf16_bits_from_f32(rng.standard_normal((M, d)).astype(np.float32) * 3)
    eye = np.zeros((d, 4 * d), np.float32)
    eye[:, :d] = np.eye(d)
    A = bf16_bits_from_f32(eye)
    B = bf16_bits_from_f32(eye.T.copy())
    Y, Z = oracle.mlp_shard(X, A, B, 1, 0, return_z=True)
    xv = oracle.bf16_decode(X)
    expect = np.array([[float(brute.bf16_round(Fraction(brute.gelu_float(v)))) for v in row]
                       for row in xv])
    assert np.array_equal(Y, expect)
    assert np.all(oracle.bf16_decode(Z)[:, d:] == 0)
    # with N=4 only rank 0 holds the identity block
    assert np.array_equal(oracle.mlp_shard(X, A, B, 4, 0), expect)
    for r in (1, 2, 3):
        assert np.all(oracle.mlp_shard(X, A, B, 4, r) == 0)


def test_permuted_columns_permute_z():
    """A column permutation of A_i permutes Z_i's columns (GeLU is elementwise)."""
    X, A, B = make_random(12, 16, 32, 8, sigma=0.3)
    perm = np.random.default_rng(0).permutation(32)
    Z = oracle.col_gelu(X, A)
    Zp = oracle.col_gelu(X, A[:, perm])
    assert np.array_equal(Z[:, perm], Zp)


# --------------------------------------------------------------- fp8 -----

def test_quant_scale_and_codes():
    T = bf16_bits_from_f32(np.array([[0.5, -2.0, 0.001, 1.75]], np.float32))
    a = oracle.amax(T)
    assert a == 2.0
    s = oracle.quant_scale(a)
    assert s == np.float32(224.0)
    q = oracle.quant_e4m3(T, s)
    # 0.5·224 = 112, −2·224 = −448, 0.001·224 ≈ 0.224 → 0.21875 (RNE), 1.75·224 = 392 → 384
    assert oracle.e4m3_decode(q).tolist() == [[112.0, -448.0, 0.21875, 384.0]]
    assert oracle.quant_scale(0.0) == 1.0


def test_quant_matches_torch_float8():
    import torch
    X, _, _ = make_random(64, 256, 16, 9)
    q, s = oracle.quantize_inputs_e4m3(X)
    prod = torch.from_numpy(oracle.bf16_decode(X).astype(np.float32)) * float(s)
    ref = prod.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)
    # the amax element maps exactly to ±448
    assert np.max(np.abs(oracle.e4m3_decode(q))) == 448.0


@pytest.mark.parametrize("M,d,F,seed", [(4, 16, 8, 30), (6, 32, 16, 31), (3, 16, 32, 32)])
def test_fp8_path_matches_brute_force(M, d, F, seed):
    X, A, B = make_random(M, d, F, seed, sigma=0.3)
    Xq, sX = oracle.quantize_inputs_e4m3(X)
    Aq, sA = oracle.quantize_inputs_e4m3(A)
    Bq, sB = oracle.quantize_inputs_e4m3(B)
    Y, Z, Zq, sZ = oracle.mlp_shard_e4m3(Xq, sX, Aq, sA, Bq, sB, return_all=True)
    Zb, Zqb, sZb, Yb = brute.fp8_shard_exact(Xq, sX, Aq, sA, Bq, sB)
    assert np.array_equal(oracle.bf16_decode(Z), np.array([[float(z) for z in r] for r in Zb]))
    assert sZ == sZb
    assert np.array_equal(oracle.e4m3_decode(Zq), np.array([[float(z) for z in r] for r in Zqb]))
    assert _rel_maxdiff(Y, np.array([[float(y) for y in r] for r in Yb])) <= 1e-13


def test_fp8_close_to_bf16_on_small_175b_like_shapes():
    """Quantisation error of the e4m3 path is a few per cent of max|Y|."""
    X, A, B = make_random(64, 384, 192, 3, sigma=0.006)
    Yb = oracle.mlp_shard(X, A, B, 1, 0)
    Xq, sX = oracle.quantize_inputs_e4m3(X)
    Aq, sA = oracle.quantize_inputs_e4m3(A)
    Bq, sB = oracle.quantize_inputs_e4m3(B)
    Yq = oracle.mlp_shard_e4m3(Xq, sX, Aq, sA, Bq, sB)
    assert _rel_maxdiff(Yq, Yb) < 0.06


# ------------------------------------------------- fp8 delayed scaling ----

def test_delayed_scale_moving_average_window():
    # small integers: every mean below is exact, so each scale is 448/mean
    # rounded once; the window keeps the last L amaxes
    h, L = [], 4
    expect_windows = [[1], [1, 2], [1, 2, 3], [1, 2, 3, 4], [2, 3, 4, 5], [3, 4, 5, 6]]
    for step, a in enumerate([1, 2, 3, 4, 5, 6]):
        h, s = oracle.amax_history_push(h, float(a), L)
        assert h == [float(v) for v in expect_windows[step]]
        mean = Fraction(sum(expect_windows[step]), len(expect_windows[step]))
        assert s == np.float32(np.float32(448) / np.float32(float(mean)))
    assert oracle.amax_history_push([], 7.0, 1)[0] == [7.0]
    assert oracle.delayed_scale([]) == 1.0
    assert oracle.delayed_scale([0.0, 0.0]) == 1.0
    assert oracle.delayed_scale([2.0, 2.0]) == np.float32(224.0)
    with pytest.raises(ValueError):
        oracle.amax_history_push([], 1.0, 0)


def _fp8_tiny(M, d, F, seed):
    X, A, B = make_random(M, d, F, seed, sigma=0.3)
    return (*oracle.quantize_inputs_e4m3(X), *oracle.quantize_inputs_e4m3(A),
            *oracle.quantize_inputs_e4m3(B))


def test_delayed_path_with_the_current_scale_is_the_current_path():
    Xq, sX, Aq, sA, Bq, sB = _fp8_tiny(6, 32, 16, 31)
    Y, Z, Zq, sZ = oracle.mlp_shard_e4m3(Xq, sX, Aq, sA, Bq, sB, return_all=True)
    Yd, Zqd, za = oracle.mlp_shard_e4m3_delayed(Xq, sX, Aq, sA, Bq, sB, sZ)
    assert np.array_equal(Zq, Zqd) and np.array_equal(Y, Yd)
    assert za == oracle.amax(Z)


@pytest.mark.parametrize("factor", [0.37, 1.0, 3.5])
def test_delayed_path_matches_brute_force_with_a_predicted_scale(factor):
    # a predicted scale below, at and above the current one (above: the
    # largest |Z| saturate at ±448 instead of overflowing)
    M, d, F = 4, 16, 8
    Xq, sX, Aq, sA, Bq, sB = _fp8_tiny(M, d, F, 33)
    Zc = oracle.col_gelu_e4m3(Xq, sX, Aq, sA)
    sZ = np.float32(oracle.quant_scale(oracle.amax(Zc)) * np.float32(factor))
    Y, Zq, za = oracle.mlp_shard_e4m3_delayed(Xq, sX, Aq, sA, Bq, sB, sZ)
    Zb, Zqb, sZb, Yb = brute.fp8_shard_exact(Xq, sX, Aq, sA, Bq, sB, sZ_given=sZ)
    assert sZb == sZ
    assert np.array_equal(oracle.e4m3_decode(Zq), np.array([[float(z) for z in r] for r in Zqb]))
    assert za == max(abs(float(z)) for r in Zb for z in r)
    assert _rel_maxdiff(Y, np.array([[float(y) for y in r] for r in Yb])) <= 1e-13
    codes = Zq.astype(np.int64)
    assert not np.any((codes & 0x7F) == 0x7F)             # never NaN
    if factor > 1:
        assert np.max(np.abs(oracle.e4m3_decode(Zq))) == 448.0


# ------------------------------------------------------------- backward ----

def test_gelu_grad_identities_and_numerical_derivative():
    assert oracle.gelu_grad(np.array([0.0]))[0] == 0.5
    x = np.linspace(-8, 8, 4001)
    g = oracle.gelu_grad(x)
    # GeLU(x) − GeLU(−x) = x, so GeLU'(x) + GeLU'(−x) = 1
    assert np.max(np.abs(g + oracle.gelu_grad(-x) - 1.0)) <= 2e-15
    h = 1e-5
    num = (omlp.gelu(x + h) - omlp.gelu(x - h)) / (2 * h)
    assert np.max(np.abs(num - g)) <= 1e-9
    assert abs(oracle.gelu_grad(np.array([10.0]))[0] - 1.0) < 1e-20
    assert -1e-20 < oracle.gelu_grad(np.array([-10.0]))[0] < 0


def _dy(M, d, seed):
    rng = np.random.default_rng(seed)
    return bf16_bits_from_f32(rng.standard_normal((M, d)).astype(np.float32))


@pytest.mark.parametrize("N,rank", [(1, 0), (2, 1), (4, 2)])
def test_backward_formulas_match_finite_differences(N, rank):
    # the exact chain rule of the unrounded forward against central finite
    # differences of L = Σ Y ⊙ dY, Y = GeLU(X·A_i)·B_i, in float64
    M, d, H = 3, 4, 16
    X, A, B = make_random(M, d, H, 60 + N, sigma=0.5)
    dY = _dy(M, d, 61)
    g = oracle.mlp_shard_backward(X, A, B, dY, N, rank, rounding=False)
    lo, hi = omlp.shard_columns(H, N, rank)
    Xv, Av, Bv, dYv = (oracle.bf16_decode(t) for t in (X, A[:, lo:hi], B[lo:hi, :], dY))

    def loss(x, a, b):
        return float(np.sum((omlp.gelu(x @ a) @ b) * dYv))
    h = 1e-6
    for name, base, grad in (("X", Xv, g["dX"]), ("A", Av, g["dA"]), ("B", Bv, g["dB"])):
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            p, m = base.copy(), base.copy()
            p[idx] += h
            m[idx] -= h
            args_p = {"X": (p, Av, Bv), "A": (Xv, p, Bv), "B": (Xv, Av, p)}[name]
            args_m = {"X": (m, Av, Bv), "A": (Xv, m, Bv), "B": (Xv, Av, m)}[name]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert grad.shape == base.shape
        assert _rel_maxdiff(grad, num) <= 1e-6, name


@pytest.mark.parametrize("M,d,H,N,rank,seed", [(4, 8, 16, 2, 0, 62), (3, 16, 32, 4, 3, 63)])
def test_backward_matches_brute_force(M, d, H, N, rank, seed):
    X, A, B = make_random(M, d, H, seed, sigma=0.3)
    dY = _dy(M, d, seed + 1)
    g = oracle.mlp_shard_backward(X, A, B, dY, N, rank)
    Z, dS, dX, dA, dB = brute.shard_backward_exact(X, A, B, dY, N, rank)
    as_f = lambda T: np.array([[float(v) for v in r] for r in T])
    assert np.array_equal(g["Z"], as_f(Z))
    assert np.array_equal(g["dS"], as_f(dS))
    assert _rel_maxdiff(g["dX"], as_f(dX)) <= 1e-13
    assert _rel_maxdiff(g["dA"], as_f(dA)) <= 1e-13
    assert _rel_maxdiff(g["dB"], as_f(dB)) <= 1e-13


def test_backward_shards_compose_to_the_unsharded_gradients():
    # the ranks' dX_i sum to the unsharded dX (the backward AllReduce); the
    # weight gradients are the column blocks of dA and the row blocks of dB
    M, d, H, N = 24, 32, 128, 4
    X, A, B = make_random(M, d, H, 64, sigma=0.1)
    dY = _dy(M, d, 65)
    full = oracle.mlp_shard_backward(X, A, B, dY, 1, 0)
    parts = [oracle.mlp_shard_backward(X, A, B, dY, N, r) for r in range(N)]
    assert _rel_maxdiff(oracle.partial_sum([p["dX"] for p in parts]), full["dX"]) <= 1e-12
    assert _rel_maxdiff(np.concatenate([p["dA"] for p in parts], axis=1), full["dA"]) <= 1e-12
    assert _rel_maxdiff(np.concatenate([p["dB"] for p in parts], axis=0), full["dB"]) <= 1e-12


def test_workload_table_shapes():
    wl = WORKLOADS["7b_tp8"]
    assert (wl.M, wl.d, wl.F) == (8192, 4096, 2048) and wl.H == 4 * wl.d
    wl = WORKLOADS["175b_tp8"]
    assert (wl.M, wl.d, wl.F) == (2048, 12288, 6144)
    assert WORKLOADS["tiny_tp2"].flops_per_shard() == 4 * 32 * 64 * 128


# ------------------------------------------------------ fp8 backward (hybrid) --

@pytest.mark.parametrize("M,d,H,N,rank,seed", [(4, 16, 32, 2, 1, 70), (5, 32, 64, 4, 2, 71)])
def test_fp8_backward_matches_brute_force(M, d, H, N, rank, seed):
    """Every code, scale and gradient of the hybrid fp8 backward against the
    exact rational evaluation (own decoders and rounding in tests/brute.py)."""
    X, A, B = make_random(M, d, H, seed, sigma=0.3)
    dY = _dy(M, d, seed + 1)
    g = oracle.mlp_shard_backward_fp8(X, A, B, dY, N, rank)
    ex = brute.shard_backward_fp8_exact(X, A, B, dY, N, rank)
    as_f = lambda T: np.array([[float(v) for v in r] for r in T])
    for k in ("sX", "sA", "sB", "sdY", "sdS", "sZ"):
        assert np.float32(g[k]) == np.float32(ex[k]), k
    assert np.array_equal(oracle.e4m3_decode(g["Xq"]), as_f(ex["Xq"]))
    assert np.array_equal(oracle.e4m3_decode(g["Aq_i"]), as_f(ex["Aq_i"]))
    assert np.array_equal(oracle.e4m3_decode(g["Bq_i"]), as_f(ex["Bq_i"]))
    assert np.array_equal(oracle.e5m2_decode(g["dYq"]), as_f(ex["dYq"]))
    assert np.array_equal(oracle.bf16_decode(g["Z_bits"]), as_f(ex["Z"]))
    assert np.array_equal(oracle.bf16_decode(g["dS_bits"]), as_f(ex["dS"]))
    assert np.array_equal(oracle.e5m2_decode(g["dSq"]), as_f(ex["dSq"]))
    assert np.array_equal(oracle.e4m3_decode(g["Zq"]), as_f(ex["Zq"]))
    for k in ("dX", "dA", "dB"):
        assert _rel_maxdiff(g[k], as_f(ex[k])) <= 1e-13, k


def _int_bits(rng, shape, top=7):
    """Small integers in [-top, top] with ±top present, as bfloat16 bits."""
    v = rng.integers(-top, top + 1, size=shape).astype(np.float32)
    v.flat[0] = top
    return bf16_bits_from_f32(v)


def test_fp8_backward_on_exact_inputs_reduces_to_the_bf16_backward():
    """With integers in [-7, 7] (amax 7), the scales are 448/7 = 2^6 (e4m3) and
    57344/7 = 2^13 (e5m2): X, A, B and dY quantise exactly, so S, dZ, and the
    rounded dS and Z equal the bf16 backward's (a separate code path)."""
    rng = np.random.default_rng(5)
    M, d, H, N, rank = 6, 16, 64, 4, 1
    X, A, B, dY = (_int_bits(rng, s) for s in ((M, d), (d, H), (H, d), (M, d)))
    g = oracle.mlp_shard_backward_fp8(X, A, B, dY, N, rank)
    ref = oracle.mlp_shard_backward(X, A, B, dY, N, rank)
    assert float(g["sX"]) == 64.0 and float(g["sdY"]) == 8192.0
    assert np.array_equal(g["S"], ref["S"]) and np.array_equal(g["dZ"], ref["dZ"])
    assert np.array_equal(g["dS_bits"], ref["dS_bits"]) and np.array_equal(g["Z_bits"], ref["Z_bits"])
    # and the gradients agree with the bf16 ones up to the quantisation of dS and Z
    for k in ("dX", "dA", "dB"):
        assert _rel_maxdiff(g[k], ref[k]) <= 0.13, k
