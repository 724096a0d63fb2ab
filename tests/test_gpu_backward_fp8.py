"""Parity of the hybrid fp8 backward (E4M3 activations and weights, E5M2
gradients) on the GPU with the oracle.

Bar: every quantised operand code and every scale bit-exact (the scales are
fp32 divisions of exact amaxes on both sides); S within the fp32
accumulation bound; dS and Z within one bf16 ulp plus the carried errors;
the gradients within 6e-2·max|ref| (the fp8 parity bar).
"""
import numpy as np
import pytest

import oracle
from helpers import bf16_ulp, dev_bf16, host_bf16_bits, host_f64, log, max_err_ratio
from workloads import WORKLOADS, make_inputs, make_output_grad, make_random

pytestmark = pytest.mark.gpu

TOL_FP8 = 6e-2
U = 2.0 ** -24
# The scaled fp8 MFMA sums each 128-term block of products at a precision of
# its own (not one IEEE fp32 rounding per product): measured up to 2.6e-5 of
# the block's Σ|terms| on MI355X. The bounds allow 2^-12 of Σ|terms| for it
# on top of K·2^-24 for the fp32 accumulation across blocks.
MFMA8 = 2.0 ** -12


@pytest.fixture(scope="module")
def tpm():
    import torch
    import megatron_tensor_transformer_shard_amd as m
    assert torch.cuda.is_available()
    return m


def _sync():
    import torch
    torch.cuda.synchronize()


def _u8(t):
    return t.detach().contiguous().cpu().numpy().astype(np.uint8)


def check_fp8_backward(what, v, g, dX, dA, dB, d, b1_block=None):
    """Every check of the fp8 backward against the oracle's dict g: the
    scales and every quantised operand code bit-exact, S within the scaled
    MFMA's accumulation bound (plus the bias add's rounding when a bias
    block is given), dS and Z within one ulp plus the carried errors with
    their codes equal wherever the values and scales agree, and the
    gradients within the fp8 bar."""
    sc = v["scale"].cpu().numpy()
    for i, k in enumerate(("sX", "sA", "sB", "sdY")):
        assert np.float32(sc[i]) == np.float32(g[k]), f"{what}: scale {k}"
    assert np.array_equal(_u8(v["Xq"]), g["Xq"]), "Xq codes"
    assert np.array_equal(_u8(v["XqT"]), g["Xq"].T), "Xq transposed codes"
    assert np.array_equal(_u8(v["Aq"]), g["Aq_i"]), "Aq_i codes"
    assert np.array_equal(_u8(v["AqT"]), g["Aq_i"].T), "Aq_i transposed codes"
    assert np.array_equal(_u8(v["BqT"]), g["Bq_i"].T), "Bq_i transposed codes"
    assert np.array_equal(_u8(v["dYq"]), g["dYq"]), "dY e5m2 codes"
    # S: fp32 accumulation of exact fp8 products (+ one rounding for the bias)
    Xv, Av = oracle.e4m3_decode(g["Xq"]), oracle.e4m3_decode(g["Aq_i"])
    absS = (np.abs(Xv) @ np.abs(Av)) / (float(g["sX"]) * float(g["sA"]))
    S = host_f64(v["S"])
    errS = np.abs(S - g["S"]) / np.maximum(absS, 1e-30)
    log(f"{what}: S error / Σ|terms| max {float(errS.max()):.3e}, "
        f"err ratio {max_err_ratio(S, g['S']):.3e}")
    tS = (MFMA8 + d * U) * absS
    if b1_block is not None:
        tS = tS + 2 * U * (np.abs(g["S"]) + np.abs(b1_block)[None, :])
    assert np.all(np.abs(S - g["S"]) <= tS * 1.01 + 1e-30), f"{what}: S"
    # dS and Z: one ulp plus the fp32 errors of dZ and S carried through GeLU' and GeLU
    dYv, Bv = oracle.e5m2_decode(g["dYq"]), oracle.e4m3_decode(g["Bq_i"])
    absdZ = (np.abs(dYv) @ np.abs(Bv).T) / (float(g["sdY"]) * float(g["sB"]))
    tdZ = (MFMA8 + d * U) * absdZ
    raw = np.abs(g["dZ"] * oracle.gelu_grad(g["S"]))
    carry = 1.13 * tdZ + (np.abs(g["dZ"]) + tdZ) * (0.8 * tS + 3e-7) + 4 * U * raw
    dS_ref = oracle.bf16_decode(g["dS_bits"])
    dS = host_f64(v["dS"])
    assert np.all(np.abs(dS - dS_ref) <= bf16_ulp(raw + carry) + carry), f"{what}: dS"
    Z_ref = oracle.bf16_decode(g["Z_bits"])
    Z = host_f64(v["Z"])
    tZ = bf16_ulp(np.abs(Z_ref) + 1.13 * tS) + 1.13 * tS + 3e-7 * np.abs(g["S"])
    assert np.all(np.abs(Z - Z_ref) <= tZ), f"{what}: Z"
    same_dS = float(np.mean(dS == dS_ref))
    log(f"{what}: dS bit-identical {same_dS:.4f}, Z bit-identical {float(np.mean(Z == Z_ref)):.4f}")
    # where the scales agree, the quantised dS and Z codes agree wherever dS and Z do
    if np.float32(sc[4]) == np.float32(g["sdS"]):
        eq = dS == dS_ref
        assert np.array_equal(_u8(v["dSq"])[eq], g["dSq"][eq]), "dS e5m2 codes"
    if np.float32(sc[5]) == np.float32(g["sZ"]):
        eq = (Z == Z_ref).T
        assert np.array_equal(_u8(v["ZqT"])[eq], g["Zq"].T[eq]), "Z e4m3 codes"
    for name, t in (("dX", dX), ("dA", dA), ("dB", dB)):
        r = max_err_ratio(host_f64(t), g[name])
        log(f"{what}: {name} err ratio {r:.3e}")
        assert r <= TOL_FP8, f"{what}: {name} err ratio {r:.3e}"


CASES = [
    # M, d, H, N (multiples of 16; tails against the 128/192/256 tiles and 128-byte k-slices)
    (32, 64, 256, 2),
    (272, 144, 576, 2),
    (528, 272, 1088, 4),
    (1040, 528, 4224, 8),
    (272, 208, 2496, 3),            # N = 3: F = 832
]


@pytest.mark.parametrize("M,d,H,N", CASES)
def test_backward_fp8_vs_oracle(tpm, M, d, H, N):
    import torch
    log(f"case fp8 backward M={M} d={d} H={H} N={N}")
    X, A, B = make_random(M, d, H, seed=3 * M + d + N, sigma=0.05)
    dY = make_output_grad(M, d, seed=M + 2 * d, sigma=1.0)
    Xd, Ad, Bd, dYd = dev_bf16(X), dev_bf16(A), dev_bf16(B), dev_bf16(dY)
    F = H // N
    for rank in sorted({0, N - 1}):
        dX, dA, dB, ws = tpm.tp_mlp_shard_backward_fp8(Xd, Ad, Bd, dYd, N, rank)
        _sync()
        g = oracle.mlp_shard_backward_fp8(X, A, B, dY, N, rank)
        v = tpm.fp8_backward_workspace_views(ws, M, d, F)
        check_fp8_backward(f"rank {rank}", v, g, dX, dA, dB, d)


def test_backward_fp8_zero_gradient(tpm):
    """dY = 0: its scale is 1 (amax 0), dS = 0 (scale 1), and every gradient is exactly 0."""
    import torch
    M, d, H, N = 48, 64, 256, 2
    X, A, B = make_random(M, d, H, seed=41, sigma=0.05)
    Xd, Ad, Bd = dev_bf16(X), dev_bf16(A), dev_bf16(B)
    dY0 = torch.zeros((M, d), dtype=torch.bfloat16, device="cuda")
    dX, dA, dB, ws = tpm.tp_mlp_shard_backward_fp8(Xd, Ad, Bd, dY0, N, 0)
    _sync()
    sc = tpm.fp8_backward_workspace_views(ws, M, d, H // N)["scale"].cpu().numpy()
    assert sc[3] == 1.0 and sc[4] == 1.0
    for name, t in (("dX", dX), ("dA", dA), ("dB", dB)):
        assert torch.count_nonzero(t).item() == 0, f"{name} nonzero for dY = 0"


@pytest.mark.parametrize("M,d,H,N", [(272, 144, 576, 2), (528, 272, 1088, 4)])
def test_backward_fp8_given_weight_amaxes(tpm, M, d, H, N):
    """max|A| and max|B| passed in (from tp_amax_bf16) give the same bits as
    computing them inside the call, for every rank."""
    import torch
    log(f"case fp8 backward, given weight amaxes, M={M} d={d} H={H} N={N}")
    X, A, B = make_random(M, d, H, seed=5 * M + N, sigma=0.05)
    dY = make_output_grad(M, d, seed=M + 3, sigma=1.0)
    Xd, Ad, Bd, dYd = dev_bf16(X), dev_bf16(A), dev_bf16(B), dev_bf16(dY)
    wam = torch.full((2,), float("nan"), dtype=torch.float32, device="cuda")
    tpm.tp_amax_bf16(Ad, amax=wam[0:1])
    tpm.tp_amax_bf16(Bd, amax=wam[1:2])
    _sync()
    assert float(wam[0]) == float(np.max(np.abs(oracle.bf16_decode(A))))
    assert float(wam[1]) == float(np.max(np.abs(oracle.bf16_decode(B))))
    for rank in range(N):
        ref = tpm.tp_mlp_shard_backward_fp8(Xd, Ad, Bd, dYd, N, rank)
        got = tpm.tp_mlp_shard_backward_fp8(Xd, Ad, Bd, dYd, N, rank, w_amax=wam)
        _sync()
        F = H // N
        sr = tpm.fp8_backward_workspace_views(ref[3], M, d, F)["scale"].cpu().numpy()
        sg = tpm.fp8_backward_workspace_views(got[3], M, d, F)["scale"].cpu().numpy()
        assert np.array_equal(sr[:6], sg[:6]), f"rank {rank}: scales"
        for name, a, b in zip(("dX", "dA", "dB"), ref[:3], got[:3]):
            assert torch.equal(a, b), f"rank {rank}: {name} differs with given weight amaxes"


def test_backward_fp8_close_to_bf16_backward(tpm):
    """The fp8 gradients against the bf16 backward of the same inputs: the
    difference is the quantisation, a few percent of the largest gradient."""
    M, d, H, N = 272, 144, 576, 2
    X, A, B = make_random(M, d, H, seed=21, sigma=0.05)
    dY = make_output_grad(M, d, seed=22)
    Xd, Ad, Bd, dYd = dev_bf16(X), dev_bf16(A), dev_bf16(B), dev_bf16(dY)
    g8 = tpm.tp_mlp_shard_backward_fp8(Xd, Ad, Bd, dYd, N, 1)[:3]
    g16 = tpm.tp_mlp_shard_backward(Xd, Ad, Bd, dYd, N, 1)[:3]
    _sync()
    for name, a, b in zip(("dX", "dA", "dB"), g8, g16):
        r = max_err_ratio(host_f64(a), host_f64(b))
        log(f"fp8 vs bf16 {name}: {r:.3e}")
        assert r <= 0.1


def test_full_7b_tp8_backward_fp8(tpm):
    """The 7B-class TP=8 fp8 backward at full size (ranks 0 and 7) against the
    oracle (five float64 GEMMs of 137 GFLOP per rank): every code, scale and
    element checked as at the moderate sizes."""
    import torch
    wl = WORKLOADS["7b_tp8_bwd"]
    log(f"case {wl.name} fp8")
    X, A, B = make_inputs(wl)
    dY = make_output_grad(wl.M, wl.d, wl.seed, wl.grad_sigma)
    Xd, Ad, Bd, dYd = dev_bf16(X), dev_bf16(A), dev_bf16(B), dev_bf16(dY)
    M, d, H, N, F = wl.M, wl.d, wl.H, wl.N, wl.F
    for rank in (0, N - 1):
        dX, dA, dB, ws = tpm.tp_mlp_shard_backward_fp8(Xd, Ad, Bd, dYd, N, rank)
        _sync()
        v = tpm.fp8_backward_workspace_views(ws, M, d, F)
        g = oracle.mlp_shard_backward_fp8(X, A, B, dY, N, rank)
        sc = v["scale"].cpu().numpy()
        for i, k in enumerate(("sX", "sA", "sB", "sdY", "sdS", "sZ")):
            log(f"rank {rank}: {k} gpu {sc[i]:.6g} oracle {float(g[k]):.6g}")
        check_fp8_backward(f"{wl.name} fp8 rank {rank}", v, g, dX, dA, dB, d)
