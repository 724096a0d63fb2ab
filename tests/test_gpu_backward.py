"""Parity of the shard's backward on the GPU (through the C ABI) with the
oracle's chain rule.

Each output is checked element by element against a bound computed from the
oracle's own values: the worst-case fp32 accumulation error of a K-term dot
product (K·2^-24·Σ|terms|), the one-ulp rounding of the bf16 intermediates
(Z, dS) and how those carry into the GEMMs that consume them, and the GeLU /
GeLU' approximation error (A&S 7.1.26 erf, |Δ| <= 1.5e-7; |GeLU'| <= 1.13,
|GeLU''| <= 0.8). On top of that, every output meets the parity bar
max|got − ref| <= 1e-2·max|ref|, and Z is bit-identical to the forward's Z_i.
"""
import numpy as np
import pytest

import oracle
from helpers import bf16_ulp, dev_bf16, host_bf16_bits, host_f64, log, max_err_ratio
from workloads import WORKLOADS, make_inputs, make_output_grad, make_random, sample_rows

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-2
U = 2.0 ** -24          # fp32 unit roundoff
GELU_APPROX = 3e-7      # |ΔGeLU(s)| / |s| and |ΔGeLU'(s)| of the fp32 evaluation
G1, G2 = 1.13, 0.8      # max |GeLU'|, max |GeLU''|


@pytest.fixture(scope="module")
def tpm():
    import torch
    import megatron_tensor_transformer_shard_amd as m
    assert torch.cuda.is_available()
    return m


def _sync():
    import torch
    torch.cuda.synchronize()


def _dec(bits):
    return oracle.bf16_decode(bits)


def _bounds(X, A_i, B_i, dY, ref):
    """Elementwise bounds on |gpu − ref| for S, Z, dS, dX, dA, dB."""
    aX, aA, aB, adY = np.abs(_dec(X)), np.abs(_dec(A_i)), np.abs(_dec(B_i)), np.abs(_dec(dY))
    M, d = aX.shape
    F = aA.shape[1]
    dS_abs = aX @ aA                      # Σ|x·a| of S
    tS = d * U * dS_abs
    dZ_abs = adY @ aB.T                   # Σ|dy·b| of dZ
    tdZ = d * U * dZ_abs
    S, dZ = ref["S"], ref["dZ"]
    # Z = bf16(GeLU(S)): one ulp, the carried S error, the approximation
    tZ = bf16_ulp(np.maximum(np.abs(ref["Z"]), np.abs(oracle.gelu(S)) + G1 * tS)) + G1 * tS + \
        GELU_APPROX * np.abs(S)
    # dS = bf16(dZ·GeLU'(S)): one ulp, the dZ error through GeLU', the S error
    # through GeLU'' (times |dZ|), the GeLU' approximation, fp32 product rounding
    raw = np.abs(dZ * oracle.gelu_grad(S))
    carry = G1 * tdZ + (np.abs(dZ) + tdZ) * (G2 * tS + GELU_APPROX) + 2 * U * raw
    tdS = bf16_ulp(raw + carry) + carry
    adS = np.abs(ref["dS"]) + tdS
    aZ = np.abs(ref["Z"]) + tZ
    tdX = F * U * (adS @ aA.T) + tdS @ aA.T
    tdA = M * U * (aX.T @ adS) + aX.T @ tdS
    tdB = M * U * (aZ.T @ adY) + tZ.T @ adY
    return {"S": tS, "Z": tZ, "dS": tdS, "dX": tdX, "dA": tdA, "dB": tdB}


def _check(name, got, ref, bound, what):
    err = np.abs(got - ref)
    bad = err > bound
    r = max_err_ratio(got, ref)
    worst = float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0
    log(f"{what} {name}: err ratio {r:.3e}, worst err/bound {worst:.3f}")
    assert not np.any(bad), f"{what} {name}: {int(bad.sum())} elements beyond the bound"
    assert r <= TOL_BF16, f"{what} {name}: err ratio {r:.3e}"


def _run(tpm, Xd, Ad, Bd, dYd, M, d, H, N, rank):
    import torch
    ws = torch.empty(tpm.tp_mlp_shard_backward_workspace_size(M, d, H, N), dtype=torch.uint8,
                     device="cuda")
    F = H // N
    nan = float("nan")
    dX = torch.full((M, d), nan, dtype=torch.float32, device="cuda")
    dA = torch.full((d, F), nan, dtype=torch.float32, device="cuda")
    dB = torch.full((F, d), nan, dtype=torch.float32, device="cuda")
    tpm.tp_mlp_shard_backward(Xd, Ad, Bd, dYd, N, rank, dX_i=dX, dA_i=dA, dB_i=dB, workspace=ws)
    return dX, dA, dB, ws


# ------------------------------------------------- ragged, several tiles --

CASES = [
    # M, d, H, N (M, d, F multiples of 8; tails in every GEMM dimension)
    (32, 64, 256, 2),
    (296, 136, 528, 2),
    (520, 264, 1056, 4),
    (8, 64, 256, 1),
    (264, 8, 64, 8),
    (1032, 520, 4160, 8),
    (200, 1032, 2064, 1),
    (264, 200, 2400, 3),            # N = 3: F = 800
]


@pytest.mark.parametrize("M,d,H,N", CASES)
def test_backward_vs_oracle(tpm, M, d, H, N):
    import torch
    log(f"case backward M={M} d={d} H={H} N={N}")
    X, A, B = make_random(M, d, H, seed=7 * M + d + H + N, sigma=0.05)
    dY = make_output_grad(M, d, seed=M + d, sigma=1.0)
    Xd, Ad, Bd, dYd = dev_bf16(X), dev_bf16(A), dev_bf16(B), dev_bf16(dY)
    F = H // N
    ranks = range(N) if N <= 2 else (0, N - 1)
    dX_parts = []
    for rank in range(N):
        dX, dA, dB, ws = _run(tpm, Xd, Ad, Bd, dYd, M, d, H, N, rank)
        dX_parts.append(dX)
        if rank not in ranks:
            continue
        _sync()
        ref = oracle.mlp_shard_backward(X, A, B, dY, N, rank)
        lo, hi = oracle.shard_columns(H, N, rank)
        bnd = _bounds(X, A[:, lo:hi], B[lo:hi, :], dY, ref)
        S_g, dS_g, Z_g = tpm.backward_workspace_views(ws, M, F)
        what = f"rank {rank}"
        _check("S", host_f64(S_g), ref["S"], bnd["S"], what)
        _check("Z", host_f64(Z_g), ref["Z"], bnd["Z"], what)
        _check("dS", host_f64(dS_g), ref["dS"], bnd["dS"], what)
        for name, t in (("dX", dX), ("dA", dA), ("dB", dB)):
            g = host_f64(t)
            assert not np.isnan(g).any(), f"{what} {name}: unwritten elements"
            _check(name, g, ref[name], bnd[name], what)
        # the backward's Z is the forward's Z_i, bit for bit
        Zf = tpm.tp_mlp_col_gelu(Xd, Ad[:, lo:hi])
        _sync()
        assert np.array_equal(host_bf16_bits(Zf), host_bf16_bits(Z_g)), f"{what}: Z != forward Z_i"
    # Σ_i dX_i is the input gradient of the unsharded block
    dXsum = tpm.tp_partial_sum(dX_parts)
    _sync()
    full = oracle.mlp_shard_backward(X, A, B, dY, 1, 0)
    r = max_err_ratio(host_f64(dXsum), full["dX"])
    log(f"sum of dX_i vs unsharded dX: err ratio {r:.3e}")
    assert r <= TOL_BF16


def test_backward_zero_gradient_and_deterministic(tpm):
    import torch
    M, d, H, N = 264, 136, 1088, 2
    X, A, B = make_random(M, d, H, seed=5, sigma=0.05)
    Xd, Ad, Bd = dev_bf16(X), dev_bf16(A), dev_bf16(B)
    dY0 = torch.zeros((M, d), dtype=torch.bfloat16, device="cuda")
    dX, dA, dB, ws = _run(tpm, Xd, Ad, Bd, dY0, M, d, H, N, 1)
    _sync()
    for name, t in (("dX", dX), ("dA", dA), ("dB", dB)):
        assert torch.count_nonzero(t).item() == 0, f"{name} nonzero for dY = 0"
    dY = dev_bf16(make_output_grad(M, d, seed=9))
    outs = [_run(tpm, Xd, Ad, Bd, dY, M, d, H, N, 1) for _ in range(2)]
    _sync()
    for a, b in zip(outs[0][:3], outs[1][:3]):
        assert torch.equal(a, b), "reruns differ"
    assert torch.equal(outs[0][3], outs[1][3]), "workspace contents differ between reruns"


def test_backward_is_linear_in_dY(tpm):
    """dY scaled by 2: dA, dB, dX scale exactly by 2 (a power of two commutes
    with every rounding, far from overflow and subnormals)."""
    import torch
    M, d, H, N = 136, 72, 576, 2
    X, A, B = make_random(M, d, H, seed=11, sigma=0.05)
    Xd, Ad, Bd = dev_bf16(X), dev_bf16(A), dev_bf16(B)
    dY = dev_bf16(make_output_grad(M, d, seed=12))
    o1 = _run(tpm, Xd, Ad, Bd, dY, M, d, H, N, 0)
    o2 = _run(tpm, Xd, Ad, Bd, dY * 2, M, d, H, N, 0)
    _sync()
    for a, b, name in zip(o1[:3], o2[:3], ("dX", "dA", "dB")):
        assert torch.equal(a * 2, b), f"{name} not exactly linear under dY -> 2·dY"


# ------------------------------------------------ full-size workload -----

def test_full_7b_tp8_backward_sampled(tpm):
    """The 7B-class TP=8 backward at full size, in the launch configuration
    the benchmark times: sampled rows of dX_i and of Σ dX_i, sampled columns
    of dA_i and rows of dB_i, against the oracle on the matching slices."""
    import torch
    wl = WORKLOADS["7b_tp8_bwd"]
    log(f"case {wl.name}: {wl.description}")
    X, A, B = make_inputs(wl)
    dY = make_output_grad(wl.M, wl.d, wl.seed, wl.grad_sigma)
    Xd, Ad, Bd, dYd = dev_bf16(X), dev_bf16(A), dev_bf16(B), dev_bf16(dY)
    M, d, H, N, F = wl.M, wl.d, wl.H, wl.N, wl.F
    ws = torch.empty(tpm.tp_mlp_shard_backward_workspace_size(M, d, H, N), dtype=torch.uint8,
                     device="cuda")
    rows = sample_rows(M, 24)
    cols = sample_rows(F, 12, seed=99)
    dXs = []
    checked = (0, N - 1)
    for rank in range(N):
        dX = torch.empty((M, d), dtype=torch.float32, device="cuda")
        dA = torch.empty((d, F), dtype=torch.float32, device="cuda")
        dB = torch.empty((F, d), dtype=torch.float32, device="cuda")
        tpm.tp_mlp_shard_backward(Xd, Ad, Bd, dYd, N, rank, dX_i=dX, dA_i=dA, dB_i=dB,
                                  workspace=ws)
        dXs.append(dX)
        if rank not in checked:
            continue
        _sync()
        lo, hi = oracle.shard_columns(H, N, rank)
        # rows of dX_i: the oracle on those rows of X and dY
        ref = oracle.mlp_shard_backward(X[rows], A, B, dY[rows], N, rank)
        r = max_err_ratio(host_f64(dX[torch.from_numpy(rows).cuda()]), ref["dX"])
        log(f"rank {rank}: dX_i sampled rows err ratio {r:.3e}")
        assert r <= TOL_BF16
        # columns c of the shard: A_i[:, c] and B_i[c, :] alone (as an N = 1 shard)
        # give S[:, c], dS[:, c], dA_i[:, c] and dB_i[c, :] exactly
        ci = torch.from_numpy(cols).cuda()
        refc = oracle.mlp_shard_backward(X, A[:, lo + cols], B[lo + cols, :], dY, 1, 0)
        r = max_err_ratio(host_f64(dA[:, ci]), refc["dA"])
        log(f"rank {rank}: dA_i sampled columns err ratio {r:.3e}")
        assert r <= TOL_BF16
        r = max_err_ratio(host_f64(dB[ci, :]), refc["dB"])
        log(f"rank {rank}: dB_i sampled rows err ratio {r:.3e}")
        assert r <= TOL_BF16
    dXsum = tpm.tp_partial_sum(dXs)
    _sync()
    ref = oracle.mlp_shard_backward(X[rows], A, B, dY[rows], 1, 0)
    r = max_err_ratio(host_f64(dXsum[torch.from_numpy(rows).cuda()]), ref["dX"])
    log(f"sum of {N} dX_i, sampled rows, vs unsharded: err ratio {r:.3e}")
    assert r <= TOL_BF16
