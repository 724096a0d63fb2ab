"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bar: max|Y − Y_ref| <= 1e-2·max|Y_ref| for bf16 and 6e-2·max|Y_ref| for e4m3;
bit-exact for integer-valued GEMMs, partial sums and quantised codes; Z within
one bf16 ulp (plus the fp32-accumulation slack) of the oracle's Z.
"""
import numpy as np
import pytest

import oracle
from helpers import (bf16_ulp, dev_bf16, dev_f32, dev_u8, host_bf16_bits, host_f64, log,
                     max_err_ratio)
from workloads import (WORKLOADS, bf16_bits_from_f32, make_inputs, make_integer_valued, make_random,
                       tile_rows)

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-2
TOL_E4M3 = 6e-2


@pytest.fixture(scope="module")
def tpm():
    import torch
    import megatron_tensor_transformer_shard_amd as m
    assert torch.cuda.is_available()
    return m


def _sync():
    import torch
    torch.cuda.synchronize()


# The GPU evaluates GeLU with the Abramowitz & Stegun 7.1.26 approximation of
# erf (|error| <= 1.5e-7); with fp32 evaluation |ΔGeLU(s)| <= 3e-7·|s|.
GELU_APPROX_REL = 3e-7


def _check_z(z_gpu_bits, z_ref_bits, what, absdot=None, K=None):
    """Z within one bf16 ulp of the oracle's Z, plus the worst-case fp32
    accumulation error of the GPU's S = Σ_k x_k·a_k (recursive summation:
    |ΔS| <= K·2^-24·Σ_k|x_k·a_k|) carried through GeLU (|GeLU'| <= 1.13), plus
    the GeLU approximation's bound (|s| <= Σ_k|x_k·a_k|).
    At least 95% of the elements must be bit-identical."""
    zg = oracle.bf16_decode(z_gpu_bits)
    zr = oracle.bf16_decode(z_ref_bits)
    tol = bf16_ulp(zr)
    if absdot is not None:
        tol = tol + (1.13 * K * 2.0 ** -24 + GELU_APPROX_REL) * absdot
    bad = np.abs(zg - zr) > tol
    frac_exact = float(np.mean(zg == zr))
    log(f"{what}: Z bit-identical fraction {frac_exact:.6f}")
    assert not np.any(bad), f"{what}: {int(bad.sum())} Z elements beyond the bound"
    assert frac_exact >= 0.95, f"{what}: only {frac_exact:.4f} of Z bit-identical"
    return frac_exact


def _absdot_bf16(X, A_i):
    return np.abs(oracle.bf16_decode(X)) @ np.abs(oracle.bf16_decode(A_i))


def _absdot_e4m3(Xq, sX, Aq_i, sA):
    return (np.abs(oracle.e4m3_decode(Xq)) @ np.abs(oracle.e4m3_decode(Aq_i))) / (float(sX) * float(sA))


# ------------------------------------------------------------ tiny config --

def test_tiny_tp2_both_ranks(tpm):
    import torch
    wl = WORKLOADS["tiny_tp2"]
    log("case tiny_tp2", wl.description)
    X, A, B = make_inputs(wl)
    Xd, Ad, Bd = dev_bf16(X), dev_bf16(A), dev_bf16(B)
    parts = []
    for rank in range(wl.N):
        lo, hi = oracle.shard_columns(wl.H, wl.N, rank)
        ws = torch.empty(tpm.tp_mlp_shard_workspace_size(wl.M, wl.d, wl.H, wl.N),
                         dtype=torch.uint8, device="cuda")
        Y = tpm.tp_mlp_shard(Xd, Ad, Bd, wl.N, rank, workspace=ws)
        _sync()
        Yref, Zref = oracle.mlp_shard(X, A, B, wl.N, rank, return_z=True)
        Zgpu = host_bf16_bits(ws[: wl.M * wl.F * 2].view(torch.bfloat16).view(wl.M, wl.F))
        _check_z(Zgpu, Zref, f"tiny rank {rank}", _absdot_bf16(X, A[:, lo:hi]), wl.d)
        r = max_err_ratio(host_f64(Y), Yref)
        log(f"tiny rank {rank}: err ratio {r:.3e}")
        assert r <= TOL_BF16
        parts.append(Y)
    Ysum = tpm.tp_partial_sum(parts)
    _sync()
    r = max_err_ratio(host_f64(Ysum), oracle.mlp_unsharded(X, A, B))
    log(f"tiny sum vs unsharded: err ratio {r:.3e}")
    assert r <= TOL_BF16


# ------------------------------------------------- ragged, several tiles --

RAGGED = [
    # M, d, H, N, out dtype
    (300, 136, 528, 2, "f32"),
    (513, 264, 1056, 4, "f32"),
    (700, 1032, 2064, 1, "bf16"),
    (1, 64, 256, 1, "f32"),
    (257, 8, 64, 8, "f32"),
    (1030, 520, 4160, 8, "bf16"),
    (333, 200, 2400, 3, "f32"),     # N = 3: F = 800, not a power of two
    (130, 96, 1152, 6, "bf16"),     # N = 6: F = 192
]


@pytest.mark.parametrize("M,d,H,N,odt", RAGGED)
def test_ragged_shapes_all_ranks(tpm, M, d, H, N, odt):
    import torch
    log(f"case ragged M={M} d={d} H={H} N={N} out={odt}")
    X, A, B = make_random(M, d, H, seed=M + d + H + N, sigma=0.05)
    Xd, Ad, Bd = dev_bf16(X), dev_bf16(A), dev_bf16(B)
    out_dtype = torch.float32 if odt == "f32" else torch.bfloat16
    parts = []
    for rank in range(N):
        F = H // N
        ws = torch.empty(tpm.tp_mlp_shard_workspace_size(M, d, H, N), dtype=torch.uint8,
                         device="cuda")
        Y = torch.full((M, d), float("nan"), dtype=out_dtype, device="cuda")
        tpm.tp_mlp_shard(Xd, Ad, Bd, N, rank, Y_i=Y, workspace=ws)
        _sync()
        Yref, Zref = oracle.mlp_shard(X, A, B, N, rank, return_z=True)
        lo, hi = oracle.shard_columns(H, N, rank)
        _check_z(host_bf16_bits(ws[: M * F * 2].view(torch.bfloat16).view(M, F)), Zref,
                 f"rank {rank}", _absdot_bf16(X, A[:, lo:hi]), d)
        Yg = host_f64(Y)
        assert not np.isnan(Yg).any(), "unwritten output elements"
        r = max_err_ratio(Yg, Yref)
        log(f"rank {rank}: err ratio {r:.3e}")
        assert r <= TOL_BF16
        parts.append(Y)
    Ysum = tpm.tp_partial_sum(parts, out_dtype=torch.float32)
    _sync()
    r = max_err_ratio(host_f64(Ysum), oracle.mlp_unsharded(X, A, B))
    log(f"sum vs unsharded: err ratio {r:.3e}")
    assert r <= TOL_BF16


def test_col_gelu_on_strided_column_view(tpm):
    import torch
    M, d, H, N = 200, 96, 768, 3
    X, A, B = make_random(M, d, H, seed=5, sigma=0.1)
    Xd, Ad = dev_bf16(X), dev_bf16(A)
    for rank in range(N):
        lo, hi = oracle.shard_columns(H, N, rank)
        Z = tpm.tp_mlp_col_gelu(Xd, Ad[:, lo:hi])
        _sync()
        _check_z(host_bf16_bits(Z), oracle.col_gelu(X, A[:, lo:hi]), f"view rank {rank}",
                 _absdot_bf16(X, A[:, lo:hi]), d)


def test_row_partial_integer_inputs_bit_exact(tpm):
    import torch
    M, F, d = 333, 520, 264
    Zi, Bi, _ = make_integer_valued(M, F, d, seed=3)     # Zi [M, F], Bi [F, d]
    Zd, Bd = dev_bf16(Zi), dev_bf16(Bi)
    Y = tpm.tp_mlp_row_partial(Zd, Bd)
    _sync()
    ref = oracle.bf16_decode(Zi) @ oracle.bf16_decode(Bi)
    assert np.array_equal(host_f64(Y), ref)
    Yb = tpm.tp_mlp_row_partial(Zd, Bd, out_dtype=torch.bfloat16)
    _sync()
    assert np.array_equal(host_bf16_bits(Yb), oracle.bf16_encode(ref))


def test_identity_weights_give_elementwise_gelu(tpm):
    import torch
    from workloads import bf16_bits_from_f32
    M, d = 130, 64
    rng = np.random.default_rng(9)
    X = bf16_bits_from_f32((rng.standard_normal((M, d)) * 3).astype(np.float32))
    eye = np.zeros((d, 4 * d), np.float32)
    eye[:, :d] = np.eye(d)
    A = bf16_bits_from_f32(eye)
    B = bf16_bits_from_f32(eye.T.copy())
    ws = torch.empty(tpm.tp_mlp_shard_workspace_size(M, d, 4 * d, 1), dtype=torch.uint8,
                     device="cuda")
    Y = tpm.tp_mlp_shard(dev_bf16(X), dev_bf16(A), dev_bf16(B), 1, 0, workspace=ws)
    _sync()
    Z = host_bf16_bits(ws[: M * 4 * d * 2].view(torch.bfloat16).view(M, 4 * d))
    assert np.all(oracle.bf16_decode(Z[:, d:]) == 0)
    _check_z(Z[:, :d], oracle.bf16_encode(oracle.gelu(oracle.bf16_decode(X))), "identity",
             np.abs(oracle.bf16_decode(X)), 1)
    # B = [I; 0] makes Y the first d columns of Z exactly
    assert np.array_equal(host_f64(Y), oracle.bf16_decode(Z[:, :d]))


def test_zero_rows_and_empty(tpm):
    import torch
    X = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    A = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((256, 64), dtype=torch.bfloat16, device="cuda")
    Y = tpm.tp_mlp_shard(X, A, B, 2, 1)
    assert Y.shape == (0, 64)
    Xz = torch.zeros((50, 64), dtype=torch.bfloat16, device="cuda")
    _, A1, B1 = make_random(50, 64, 256, seed=2)
    Y = tpm.tp_mlp_shard(Xz, dev_bf16(A1), dev_bf16(B1), 2, 0)
    _sync()
    assert torch.all(Y == 0).item()


def test_deterministic_reruns(tpm):
    import torch
    M, d, H = 777, 512, 2048
    X, A, B = make_random(M, d, H, seed=17)
    Xd, Ad, Bd = dev_bf16(X), dev_bf16(A), dev_bf16(B)
    outs = [tpm.tp_mlp_shard(Xd, Ad, Bd, 2, 1).cpu() for _ in range(3)]
    assert all(torch.equal(outs[0], o) for o in outs[1:])


# ----------------------------------------------------------- partial sum --

@pytest.mark.parametrize("nparts,numel", [(1, 4096), (2, 1000003), (3, 77), (8, 1 << 20),
                                          (9, 12345), (64, 40000)])
def test_partial_sum_integer_exact(tpm, nparts, numel):
    import torch
    rng = np.random.default_rng(nparts * 7 + numel)
    parts = rng.integers(-1000, 1000, size=(nparts, numel)).astype(np.float32)
    dparts = [torch.from_numpy(p).cuda() for p in parts]
    Y = tpm.tp_partial_sum(dparts)
    _sync()
    assert np.array_equal(Y.cpu().numpy(), parts.sum(axis=0, dtype=np.float64).astype(np.float32))
    # bf16 partials (small integers are exact in bf16) -> fp32 and bf16 sums
    from workloads import bf16_bits_from_f32
    small = rng.integers(-100, 100, size=(nparts, numel)).astype(np.float32)
    bparts = [dev_bf16(bf16_bits_from_f32(p)) for p in small]
    Yf = tpm.tp_partial_sum(bparts, out_dtype=torch.float32)
    Yb = tpm.tp_partial_sum(bparts, out_dtype=torch.bfloat16)
    _sync()
    exact = small.sum(axis=0, dtype=np.float64)
    assert np.array_equal(host_f64(Yf), exact)
    assert np.array_equal(host_bf16_bits(Yb), oracle.bf16_encode(exact))


def test_partial_sum_rank_order_and_in_place(tpm):
    import torch
    # (1e8 + 1) − 1e8 in fp32 is 0; any other association gives 1
    p = [torch.full((1000,), v, dtype=torch.float32, device="cuda") for v in (1e8, 1.0, -1e8)]
    Y = tpm.tp_partial_sum(p)
    _sync()
    assert torch.all(Y == 0).item()
    q = [torch.full((4099,), float(i + 1), device="cuda") for i in range(5)]
    out = tpm.tp_partial_sum(q, Y=q[0])
    _sync()
    assert out.data_ptr() == q[0].data_ptr() and torch.all(q[0] == 15.0).item()


# ------------------------------------------ sequence-parallel share, bias --

@pytest.mark.parametrize("N,M,d", [(2, 32, 64), (4, 1000, 72), (8, 8192, 4096)])
def test_reduce_scatter_shares_integer_exact_with_bias(tpm, N, M, d):
    # integer-valued fp32 partials and bias: every fp32 sum is exact, so each
    # share must equal the oracle's element for element; the shares stacked in
    # rank order must equal the all-reduce form (bias added once)
    import torch
    rng = np.random.default_rng(N * 1000 + M)
    parts = rng.integers(-1000, 1000, size=(N, M, d)).astype(np.float32)
    bias = rng.integers(-50, 50, size=d).astype(np.float32)
    dparts = [torch.from_numpy(p).cuda() for p in parts]
    dbias = torch.from_numpy(bias).cuda()
    log(f"reduce-scatter N={N} M={M} d={d}")
    shares = [tpm.tp_reduce_scatter_share(dparts, r, bias=dbias) for r in range(N)]
    full = tpm.tp_partial_sum_rows(dparts, 0, M, bias=dbias)
    _sync()
    ref = [oracle.reduce_scatter_share(parts, r, bias) for r in range(N)]
    for r in range(N):
        assert np.array_equal(host_f64(shares[r]), ref[r]), f"rank {r}"
    assert np.array_equal(host_f64(full), oracle.partial_sum_rows(parts, 0, M, bias))
    assert np.array_equal(np.concatenate([host_f64(x) for x in shares]), host_f64(full))


@pytest.mark.parametrize("part_dt,bias_dt,out_dt", [("f32", "f32", "f32"), ("f32", "bf16", "bf16"),
                                                    ("bf16", "bf16", "f32"), ("bf16", None, "bf16")])
def test_partial_sum_rows_matches_oracle_on_ragged_range(tpm, part_dt, bias_dt, out_dt):
    # partial outputs of a real tiny TP=4 shard, an arbitrary row range
    import torch
    from workloads import bf16_bits_from_f32
    X, A, B = make_random(40, 64, 256, 11)
    parts64 = [oracle.mlp_shard(X, A, B, 4, r) for r in range(4)]
    rng = np.random.default_rng(12)
    bias64 = rng.standard_normal(64) * 0.1
    if part_dt == "f32":
        parts = [p.astype(np.float32) for p in parts64]
        dparts = [torch.from_numpy(p).cuda() for p in parts]
        host_parts = [p.astype(np.float64) for p in parts]
    else:
        bits = [bf16_bits_from_f32(p.astype(np.float32)) for p in parts64]
        dparts = [dev_bf16(b) for b in bits]
        host_parts = [oracle.bf16_decode(b) for b in bits]
    dbias, host_bias = None, None
    if bias_dt == "f32":
        dbias = torch.from_numpy(bias64.astype(np.float32)).cuda()
        host_bias = bias64.astype(np.float32).astype(np.float64)
    elif bias_dt == "bf16":
        bb = bf16_bits_from_f32(bias64.astype(np.float32))
        dbias, host_bias = dev_bf16(bb), oracle.bf16_decode(bb)
    odt = torch.float32 if out_dt == "f32" else torch.bfloat16
    Y = tpm.tp_partial_sum_rows(dparts, 7, 33, bias=dbias, out_dtype=odt)
    _sync()
    ref = oracle.partial_sum_rows(host_parts, 7, 33, host_bias)
    got = host_f64(Y) if out_dt == "f32" else oracle.bf16_decode(host_bf16_bits(Y))
    err = max_err_ratio(got, ref)
    log(f"rows [7,33) parts {part_dt} bias {bias_dt} out {out_dt}: err ratio {err:.3e}")
    assert err <= (1e-6 if out_dt == "f32" else TOL_BF16)
    # empty range: no-op
    E = tpm.tp_partial_sum_rows(dparts, 5, 5)
    assert E.numel() == 0


def test_partial_sum_rows_in_place(tpm):
    import torch
    M, d, N = 64, 128, 4
    q = [torch.full((M, d), float(i + 1), device="cuda") for i in range(N)]
    before = q[0].clone()
    out = tpm.tp_partial_sum_rows(q, 16, 32, Y=q[0][16:32])
    _sync()
    assert out.data_ptr() == q[0][16:32].data_ptr()
    assert torch.all(q[0][16:32] == 10.0).item()
    assert torch.equal(q[0][:16], before[:16]) and torch.equal(q[0][32:], before[32:])


# ------------------------------------------------------------ fp8 path ---

def _quant_on_gpu(tpm, bits):
    T = dev_bf16(bits)
    amax = tpm.tp_amax_bf16(T)
    Tq, s = tpm.tp_quant_e4m3(T, amax)
    return amax, Tq, s


# ----------------------------------------------- fp8 delayed scaling ------

def test_amax_history_push_ring_and_scale(tpm):
    import torch
    L = 5
    hist = tpm.AmaxHistory(L, initial_scale=1.0)
    rng = np.random.default_rng(50)
    window = []
    pushed = []
    for step in range(12):
        # small integers first (every mean exact), then general floats
        a = float(step + 1) if step < 7 else float(np.float32(rng.uniform(0.1, 9.0)))
        pushed.append(a)
        s = hist.push(dev_f32([a]))
        _sync()
        window, s_ref = oracle.amax_history_push(window, a, L)
        got = np.float32(s.item())
        if step < 7:
            assert got == s_ref, f"step {step}: {got} vs {s_ref}"
        else:
            # the GPU sums the window in fp32: relative error <= (n-1)·2^-24 on
            # the mean, plus one rounding of the mean and of the division
            n = len(window)
            assert abs(float(got) - float(s_ref)) <= ((n + 2) * 2.0 ** -24) * float(s_ref)
    _sync()
    assert int(hist.count.item()) == 12
    ring = hist.history.cpu().numpy()
    for c, a in enumerate(pushed[-L:], start=12 - L):
        assert ring[c % L] == np.float32(a)


def _fp8_inputs(M, d, F, seed, sigma=0.3):
    X, A, B = make_random(M, d, F, seed, sigma=sigma)
    return [oracle.quantize_inputs_e4m3(T) for T in (X, A, B)]


@pytest.mark.parametrize("M,d,F", [(300, 272, 800), (257, 512, 2048), (1, 64, 64)])
def test_col_gelu_e4m3_delayed_equals_current_path_at_the_current_scale(tpm, M, d, F):
    import torch
    (Xq, sX), (Aq, sA), _ = _fp8_inputs(M, d, F, M + d)
    dX, dA, dsX, dsA = dev_u8(Xq), dev_u8(Aq), dev_f32([sX]), dev_f32([sA])
    za = torch.empty(1, dtype=torch.float32, device="cuda")
    Z = tpm.tp_mlp_col_gelu_e4m3(dX, dsX, dA, dsA, z_amax=za)
    Zq, sZ = tpm.tp_quant_e4m3(Z, za)
    Zq_d, za_d = tpm.tp_mlp_col_gelu_e4m3_delayed(dX, dsX, dA, dsA, sZ)
    _sync()
    log(f"delayed at the current scale M={M} d={d} F={F}: sZ={sZ.item()}")
    assert np.array_equal(Zq_d.cpu().numpy(), Zq.cpu().numpy())
    assert za_d.item() == za.item()


@pytest.mark.parametrize("factor", [0.37, 3.5])
def test_col_gelu_e4m3_delayed_with_a_predicted_scale(tpm, factor):
    # codes must be the oracle's quantisation of the GPU's own bf16 Z with the
    # same scale (same fp32 product, clamp and rounding); a scale above the
    # current one saturates at ±448, never NaN
    import torch
    (Xq, sX), (Aq, sA), _ = _fp8_inputs(257, 512, 2048, 77)
    dX, dA, dsX, dsA = dev_u8(Xq), dev_u8(Aq), dev_f32([sX]), dev_f32([sA])
    za = torch.empty(1, dtype=torch.float32, device="cuda")
    Z = tpm.tp_mlp_col_gelu_e4m3(dX, dsX, dA, dsA, z_amax=za)
    _sync()
    sZ = np.float32(np.float32(448.0) / np.float32(za.item()) * np.float32(factor))
    Zq_d, _ = tpm.tp_mlp_col_gelu_e4m3_delayed(dX, dsX, dA, dsA, dev_f32([sZ]))
    _sync()
    ref = oracle.quant_e4m3(host_bf16_bits(Z), sZ)
    got = Zq_d.cpu().numpy()
    assert np.array_equal(got, ref)
    assert not np.any((got & 0x7F) == 0x7F)
    if factor > 1:
        assert np.max(np.abs(oracle.e4m3_decode(got))) == 448.0


def test_fp8_shard_delayed_steps_vs_oracle(tpm):
    # three steps of one rank's shard: the first with the initial scale, the
    # next ones with the scale predicted from the recorded amaxes
    import torch
    M, d, H, N, rank = 257, 512, 2048, 2, 1
    L = 16
    hist = tpm.AmaxHistory(L, initial_scale=64.0)
    window = []
    for step in range(3):
        (Xq, sX), (Aq, sA), (Bq, sB) = _fp8_inputs(M, d, H, 90 + step)
        sZ_used = np.float32(hist.scale.item())
        Y, za = tpm.tp_mlp_shard_e4m3_delayed(dev_u8(Xq), dev_f32([sX]), dev_u8(Aq), dev_f32([sA]),
                                              dev_u8(Bq), dev_f32([sB]), hist.scale, N, rank)
        _sync()
        Y_ref, _, za_ref = oracle.mlp_shard_e4m3_delayed(Xq, sX, Aq, sA, Bq, sB, sZ_used, N, rank)
        err = max_err_ratio(oracle.bf16_decode(host_bf16_bits(Y)), Y_ref)
        log(f"delayed step {step}: sZ={sZ_used} amax {za.item():.5f} vs {za_ref:.5f} err {err:.3e}")
        assert err <= TOL_E4M3
        assert abs(za.item() - za_ref) <= 2.0 ** -7 * za_ref   # one bf16 ulp of the largest |Z|
        window, _ = oracle.amax_history_push(window, za.item(), L)
        hist.push(za)
    _sync()
    assert int(hist.count.item()) == 3


@pytest.mark.parametrize("shape,sigma", [((300, 272), 1.0), ((64, 4096), 0.006), ((17, 16), 3.0)])
def test_amax_and_quant_codes_bit_exact(tpm, shape, sigma):
    X, _, _ = make_random(shape[0], shape[1], 16, seed=shape[0], x_sigma=sigma)
    amax, Tq, s = _quant_on_gpu(tpm, X)
    _sync()
    a_ref = oracle.amax(X)
    q_ref, s_ref = oracle.quantize_inputs_e4m3(X)
    assert float(amax.item()) == a_ref
    assert np.float32(s.item()) == s_ref
    assert np.array_equal(Tq.cpu().numpy(), q_ref)


# sizes that reach each part of the amax kernel: the scalar tail alone, vectors
# after the last whole chunk (a chunk is 8 x 1024 vectors of 8 values), several
# chunks, and more chunks than workgroups (grid-stride over chunks)
AMAX_SIZES = [1, 7, 8, 9, 1000, 65536, 65536 + 8 * 33 + 5, 3 * 65536 + 17, 300 * 65536 + 8 * 1024 + 3]


@pytest.mark.parametrize("numel", AMAX_SIZES)
def test_amax_bf16_sizes_and_positions(tpm, numel):
    """max|T| wherever the largest magnitude sits: first element, inside the
    first chunk, among the vectors after the last whole chunk, in the scalar
    tail, last element; negative values count by magnitude."""
    import torch
    log(f"case amax numel={numel}")
    rng = np.random.default_rng(numel)
    base = bf16_bits_from_f32((0.5 * rng.standard_normal(numel)).astype(np.float32))
    nvec = numel // 8
    last_chunk_end = (nvec // 8192) * 8192 * 8
    spots = sorted({0, min(numel - 1, 4099), numel - 1, min(numel - 1, last_chunk_end + 3),
                    min(numel - 1, nvec * 8)})
    for pos in spots:
        bits = base.copy()
        bits[pos] = bf16_bits_from_f32(np.array([-7.75], dtype=np.float32))[0]
        a = tpm.tp_amax_bf16(dev_bf16(bits))
        _sync()
        ref = float(np.max(np.abs(oracle.bf16_decode(bits))))
        assert ref == 7.75
        assert float(a.item()) == ref, f"numel {numel}: max at {pos} not found"
    # all zeros (and negative zeros) give 0
    z = np.zeros(numel, dtype=np.uint16)
    z[::3] = 0x8000
    a = tpm.tp_amax_bf16(dev_bf16(z))
    _sync()
    assert float(a.item()) == 0.0


def test_quant_zero_tensor_scale_one(tpm):
    import torch
    T = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    amax = tpm.tp_amax_bf16(T)
    Tq, s = tpm.tp_quant_e4m3(T, amax)
    _sync()
    assert amax.item() == 0.0 and s.item() == 1.0 and torch.all(Tq == 0).item()


@pytest.mark.parametrize("M,d,H,N", [(300, 272, 800, 1), (257, 512, 2048, 4), (1, 64, 64, 1)])
def test_fp8_shard_vs_oracle(tpm, M, d, H, N):
    import torch
    log(f"case fp8 M={M} d={d} H={H} N={N}")
    X, A, B = make_random(M, d, H, seed=M + H, sigma=0.05)
    _, Xq, sX = _quant_on_gpu(tpm, X)
    _, Aq, sA = _quant_on_gpu(tpm, A)
    _, Bq, sB = _quant_on_gpu(tpm, B)
    Xq_ref, sX_ref = oracle.quantize_inputs_e4m3(X)
    Aq_ref, sA_ref = oracle.quantize_inputs_e4m3(A)
    Bq_ref, sB_ref = oracle.quantize_inputs_e4m3(B)
    for rank in range(N):
        F = H // N
        ws = torch.empty(tpm.tp_mlp_shard_e4m3_workspace_size(M, d, H, N), dtype=torch.uint8,
                         device="cuda")
        Y = tpm.tp_mlp_shard_e4m3(Xq, sX, Aq, sA, Bq, sB, N, rank, workspace=ws)
        _sync()
        lo, hi = oracle.shard_columns(H, N, rank)
        Yref, Zref, Zq_ref, sZ_ref = oracle.mlp_shard_e4m3(Xq_ref, sX_ref, Aq_ref, sA_ref,
                                                           Bq_ref, sB_ref, N, rank,
                                                           return_all=True)
        Zg = host_bf16_bits(ws[: M * F * 2].view(torch.bfloat16).view(M, F))
        _check_z(Zg, Zref, f"fp8 rank {rank}", _absdot_e4m3(Xq_ref, sX_ref, Aq_ref[:, lo:hi], sA_ref), d)
        r = max_err_ratio(host_f64(Y), Yref)
        log(f"fp8 rank {rank}: err ratio {r:.3e}")
        assert r <= TOL_E4M3


def test_fp8_steps_individually(tpm):
    import torch
    M, d, F = 130, 96, 208
    X, A, B = make_random(M, d, F, seed=44, sigma=0.1)
    Xq_ref, sX_ref = oracle.quantize_inputs_e4m3(X)
    Aq_ref, sA_ref = oracle.quantize_inputs_e4m3(A)
    Bq_ref, sB_ref = oracle.quantize_inputs_e4m3(B)
    sX, sA, sB = dev_f32([sX_ref]), dev_f32([sA_ref]), dev_f32([sB_ref])
    za = torch.empty(1, dtype=torch.float32, device="cuda")
    Z = tpm.tp_mlp_col_gelu_e4m3(dev_u8(Xq_ref), sX, dev_u8(Aq_ref), sA, z_amax=za)
    _sync()
    Zref = oracle.col_gelu_e4m3(Xq_ref, sX_ref, Aq_ref, sA_ref)
    Zg = host_bf16_bits(Z)
    _check_z(Zg, Zref, "fp8 col_gelu", _absdot_e4m3(Xq_ref, sX_ref, Aq_ref, sA_ref), d)
    assert za.item() == oracle.amax(Zg)
    # requantise the GPU's own Z and check the codes bit for bit
    Zq, sZ = tpm.tp_quant_e4m3(Z, za)
    _sync()
    Zq_ref, sZ_ref = oracle.requant_z(Zg)
    assert np.float32(sZ.item()) == sZ_ref
    assert np.array_equal(Zq.cpu().numpy(), Zq_ref)
    Y = tpm.tp_mlp_row_partial_e4m3(Zq, sZ, dev_u8(Bq_ref), sB)
    _sync()
    r = max_err_ratio(host_f64(Y), oracle.row_partial_e4m3(Zq_ref, sZ_ref, Bq_ref, sB_ref))
    log(f"fp8 row_partial: err ratio {r:.3e}")
    assert r <= 1e-2   # same codes on both sides: only fp32 accumulation and bf16 output


# ------------------------------------------------ full-size workloads ----
# The workloads at their full sizes, in the launch configuration the benchmark
# times (the tile shapes the launchers pick for them: 256x256 for the 7B-class
# GEMMs, 256x192 for the GPT-2-small column GEMM and the 175B-class GEMMs,
# 128x192 for the GPT-2-small row GEMM).
# Every element of every rank's Y_i is compared with the oracle, and Z_i of the
# ranks in z_ranks element by element with the Z bound and its bit-identical
# floor. The sum of the ranks is compared in full with the sum of the
# oracle's partials in rank order, and with the unsharded block on rows that
# hit every 64-row part of every 256-row M-tile.

def _full_size_bf16(tpm, name, z_ranks):
    import torch
    wl = WORKLOADS[name]
    log(f"case {name}: {wl.description}")
    X, A, B = make_inputs(wl)
    Xd, Ad, Bd = dev_bf16(X), dev_bf16(A), dev_bf16(B)
    M, d, H, N, F = wl.M, wl.d, wl.H, wl.N, wl.F
    ws = torch.empty(tpm.tp_mlp_shard_workspace_size(M, d, H, N), dtype=torch.uint8,
                     device="cuda")
    parts = []
    ref_sum = None
    for rank in range(N):
        Y = torch.full((M, d), float("nan"), dtype=torch.float32, device="cuda")
        tpm.tp_mlp_shard(Xd, Ad, Bd, N, rank, Y_i=Y, workspace=ws)
        _sync()
        Yref, Zref = oracle.mlp_shard(X, A, B, N, rank, return_z=True)
        if rank in z_ranks:
            lo, hi = oracle.shard_columns(H, N, rank)
            Zg = host_bf16_bits(ws[: M * F * 2].view(torch.bfloat16).view(M, F))
            _check_z(Zg, Zref, f"{name} rank {rank}", _absdot_bf16(X, A[:, lo:hi]), d)
        Yg = host_f64(Y)
        assert not np.isnan(Yg).any(), f"{name} rank {rank}: unwritten output elements"
        r = max_err_ratio(Yg, Yref)
        log(f"{name} rank {rank}: every element, err ratio {r:.3e}")
        assert r <= TOL_BF16
        ref_sum = Yref if ref_sum is None else ref_sum + Yref
        parts.append(Y)
    if N > 1:
        Ysum = tpm.tp_partial_sum(parts)
        _sync()
        r = max_err_ratio(host_f64(Ysum), ref_sum)
        log(f"{name}: sum of {N} ranks, every element vs the oracle's partials summed, "
            f"err ratio {r:.3e}")
        assert r <= TOL_BF16
        rows = tile_rows(M)
        r = max_err_ratio(host_f64(Ysum[torch.from_numpy(rows).cuda()]),
                          oracle.mlp_unsharded(X[rows], A, B))
        log(f"{name}: sum vs unsharded on {len(rows)} tile-covering rows, err ratio {r:.3e}")
        assert r <= TOL_BF16


def test_full_gpt2s_n1(tpm):
    _full_size_bf16(tpm, "gpt2s_n1", z_ranks=(0,))


def test_full_7b_tp8_all_ranks_and_sum(tpm):
    _full_size_bf16(tpm, "7b_tp8", z_ranks=(0, 7))


def test_full_175b_tp8(tpm):
    _full_size_bf16(tpm, "175b_tp8", z_ranks=(0,))


def test_full_175b_tp8_e4m3(tpm):
    import torch
    wl = WORKLOADS["175b_tp8_e4m3"]
    log(f"case {wl.name}: {wl.description}")
    X, A, B = make_inputs(wl)
    _, Xq, sX = _quant_on_gpu(tpm, X)
    _, Aq, sA = _quant_on_gpu(tpm, A)
    _, Bq, sB = _quant_on_gpu(tpm, B)
    ws = torch.empty(tpm.tp_mlp_shard_e4m3_workspace_size(wl.M, wl.d, wl.H, wl.N),
                     dtype=torch.uint8, device="cuda")
    Y = tpm.tp_mlp_shard_e4m3(Xq, sX, Aq, sA, Bq, sB, workspace=ws)
    _sync()
    Xq_ref, sX_ref = oracle.quantize_inputs_e4m3(X)
    Aq_ref, sA_ref = oracle.quantize_inputs_e4m3(A)
    Bq_ref, sB_ref = oracle.quantize_inputs_e4m3(B)
    assert np.array_equal(Xq.cpu().numpy(), Xq_ref) and np.array_equal(Aq.cpu().numpy(), Aq_ref)
    assert np.array_equal(Bq.cpu().numpy(), Bq_ref)
    # every element of Y against the oracle's fp8 path (Z in full decides Z's scale)
    Zref = oracle.col_gelu_e4m3(Xq_ref, sX_ref, Aq_ref, sA_ref)
    Zq_ref, sZ_ref = oracle.requant_z(Zref)
    Zg = host_bf16_bits(ws[: wl.M * wl.F * 2].view(torch.bfloat16).view(wl.M, wl.F))
    _check_z(Zg, Zref, wl.name, _absdot_e4m3(Xq_ref, sX_ref, Aq_ref, sA_ref), wl.d)
    Yref = oracle.row_partial_e4m3(Zq_ref, sZ_ref, Bq_ref, sB_ref)
    r = max_err_ratio(host_f64(Y), Yref)
    log(f"{wl.name}: every element, err ratio {r:.3e}")
    assert r <= TOL_E4M3
    rows = tile_rows(wl.M)
    # informational: quantisation error against the bf16 oracle
    rb = max_err_ratio(host_f64(Y[torch.from_numpy(rows).cuda()]),
                       oracle.mlp_shard(X[rows], A, B, 1, 0))
    log(f"{wl.name}: vs bf16 oracle (quantisation error) {rb:.3e}")
