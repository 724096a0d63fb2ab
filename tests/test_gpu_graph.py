"""The C-ABI entry points under HIP graph capture: every call only enqueues
kernels on the caller's stream (amax outputs are cleared by a fill kernel,
never by a memset), so a captured step replays to the same bits as the eager
one. Each replay is preceded by eager work on the outputs and followed by a
synchronisation, and every replay is compared with the eager result."""
import numpy as np
import pytest

from helpers import dev_bf16, log
from workloads import make_output_grad, make_random

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tpm():
    import torch
    import megatron_tensor_transformer_shard_amd as m
    assert torch.cuda.is_available()
    return m


def _replay_and_compare(step, outputs, reps=3):
    import torch
    # eager reference
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outputs]
    # capture (after a warm-up on the capture's side stream)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(reps):
        for o in outputs:                   # eager work between replays
            o.fill_(float("nan") if o.is_floating_point() else 123)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outputs, ref)):
            assert torch.equal(o, r), f"replay {rep}: output {i} differs from the eager result"
        log(f"replay {rep}: {len(outputs)} outputs equal to eager")


def test_forward_step_in_a_graph(tpm):
    import torch
    M, d, H, N = 300, 136, 544, 2
    X, A, B = make_random(M, d, H, seed=31, sigma=0.05)
    Xd, Ad, Bd = dev_bf16(X), dev_bf16(A), dev_bf16(B)
    parts = [torch.empty((M, d), dtype=torch.float32, device="cuda") for _ in range(N)]
    ws = [torch.empty(tpm.tp_mlp_shard_workspace_size(M, d, H, N), dtype=torch.uint8,
                      device="cuda") for _ in range(N)]
    Y = torch.empty((M, d), dtype=torch.float32, device="cuda")

    def step():
        for r in range(N):
            tpm.tp_mlp_shard(Xd, Ad, Bd, N, r, Y_i=parts[r], workspace=ws[r])
        tpm.tp_partial_sum(parts, Y=Y)
    _replay_and_compare(step, parts + [Y])


def test_backward_bf16_and_fp8_in_a_graph(tpm):
    import torch
    M, d, H, N = 272, 144, 576, 2
    F = H // N
    X, A, B = make_random(M, d, H, seed=32, sigma=0.05)
    dY = make_output_grad(M, d, seed=33)
    Xd, Ad, Bd, dYd = dev_bf16(X), dev_bf16(A), dev_bf16(B), dev_bf16(dY)
    outs = [torch.empty(shp, dtype=torch.float32, device="cuda")
            for _ in range(2) for shp in ((M, d), (d, F), (F, d))]
    ws16 = torch.empty(tpm.tp_mlp_shard_backward_workspace_size(M, d, H, N), dtype=torch.uint8,
                       device="cuda")
    ws8 = torch.empty(tpm.tp_mlp_shard_backward_fp8_workspace_size(M, d, H, N), dtype=torch.uint8,
                      device="cuda")

    def step():
        tpm.tp_mlp_shard_backward(Xd, Ad, Bd, dYd, N, 1, dX_i=outs[0], dA_i=outs[1], dB_i=outs[2],
                                  workspace=ws16)
        tpm.tp_mlp_shard_backward_fp8(Xd, Ad, Bd, dYd, N, 1, dX_i=outs[3], dA_i=outs[4],
                                      dB_i=outs[5], workspace=ws8)
    _replay_and_compare(step, outs)


def test_transposed_weight_forward_in_a_graph(tpm):
    import torch
    M, d, H, N = 300, 136, 544, 2
    X, A, B = make_random(M, d, H, seed=34, sigma=0.05)
    Xd = dev_bf16(X)
    W1, W2 = dev_bf16(A).t().contiguous(), dev_bf16(B).t().contiguous()
    parts = [torch.empty((M, d), dtype=torch.float32, device="cuda") for _ in range(N)]
    ws = [torch.empty(tpm.tp_mlp_shard_workspace_size(M, d, H, N), dtype=torch.uint8,
                      device="cuda") for _ in range(N)]

    def step():
        for r in range(N):
            tpm.tp_mlp_shard_wt(Xd, W1, W2, N, r, Y_i=parts[r], workspace=ws[r])
    _replay_and_compare(step, parts)


def test_bias_forward_backward_and_bias_gradient_in_a_graph(tpm):
    import torch
    from workloads import make_bias
    M, d, H, N = 272, 144, 576, 2
    F = H // N
    X, A, B = make_random(M, d, H, seed=35, sigma=0.05)
    dY = make_output_grad(M, d, seed=36)
    Xd, Ad, Bd, dYd = dev_bf16(X), dev_bf16(A), dev_bf16(B), dev_bf16(dY)
    b1 = dev_bf16(make_bias(H, seed=37))
    Z = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    outs = [torch.empty(shp, dtype=torch.float32, device="cuda")
            for shp in ((M, d), (d, F), (F, d), (F,), (d,))]
    ws = torch.empty(tpm.tp_mlp_shard_backward_bias_workspace_size(M, d, H, N), dtype=torch.uint8,
                     device="cuda")
    wsg = torch.empty(max(tpm.tp_bias_grad_workspace_size(M, d), 256), dtype=torch.uint8,
                      device="cuda")

    def step():
        tpm.tp_mlp_col_gelu_bias(Xd, Ad[:, F:], b1[F:], Z)
        tpm.tp_mlp_shard_backward_bias(Xd, Ad, b1, Bd, dYd, N, 1, dX_i=outs[0], dA_i=outs[1],
                                       dB_i=outs[2], db1_i=outs[3], workspace=ws)
        tpm.tp_bias_grad_bf16(dYd, db=outs[4], workspace=wsg)
    _replay_and_compare(step, [Z] + outs)


def test_e4m3_forward_step_in_a_graph(tpm):
    # the fp8 forward as the benchmark runs it: Z = GeLU(X·A_i) with its amax,
    # Z requantised with its own scale, then the fp8 row step
    import torch
    M, d, F = 264, 272, 384  # the fp8 calls take d and F in multiples of 16
    X, A, B = make_random(M, d, F, seed=38, sigma=0.3)

    def quant(bits):
        T = dev_bf16(bits)
        return tpm.tp_quant_e4m3(T, tpm.tp_amax_bf16(T))
    (Xq, sX), (Aq, sA), (Bq, sB) = quant(X), quant(A), quant(B)
    Z = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    Zq = torch.empty((M, F), dtype=torch.uint8, device="cuda")
    za = torch.empty(1, dtype=torch.float32, device="cuda")
    sZ = torch.empty(1, dtype=torch.float32, device="cuda")
    Y = torch.empty((M, d), dtype=torch.bfloat16, device="cuda")

    def step():
        tpm.tp_mlp_col_gelu_e4m3(Xq, sX, Aq, sA, Z, za)
        tpm.tp_quant_e4m3(Z, za, Zq, sZ)
        tpm.tp_mlp_row_partial_e4m3(Zq, sZ, Bq, sB, Y)
    _replay_and_compare(step, [Z, za, Zq, sZ, Y])


def test_e4m3_delayed_scaling_steps_in_a_graph(tpm):
    # the delayed-scaling step changes its own state (amax history, scale) on
    # every run: three replays from the initial state must give the three
    # eager steps' outputs and states, in order
    import torch
    M, d, F = 264, 272, 384  # the fp8 calls take d and F in multiples of 16
    X, A, B = make_random(M, d, F, seed=39, sigma=0.3)

    def quant(bits):
        T = dev_bf16(bits)
        return tpm.tp_quant_e4m3(T, tpm.tp_amax_bf16(T))
    (Xq, sX), (Aq, sA), (Bq, sB) = quant(X), quant(A), quant(B)
    hist = tpm.AmaxHistory(4, initial_scale=1.0)
    Zq = torch.empty((M, F), dtype=torch.uint8, device="cuda")
    za = torch.empty(1, dtype=torch.float32, device="cuda")
    Y = torch.empty((M, d), dtype=torch.bfloat16, device="cuda")

    def reset():
        hist.history.zero_()
        hist.count.zero_()
        hist.scale.fill_(1.0)
        torch.cuda.synchronize()

    def step():
        tpm.tp_mlp_col_gelu_e4m3_delayed(Xq, sX, Aq, sA, hist.scale, Zq, za)
        tpm.tp_mlp_row_partial_e4m3(Zq, hist.scale, Bq, sB, Y)
        hist.push(za)

    state = [Zq, za, Y, hist.history, hist.count, hist.scale]
    reset()
    ref = []
    for _ in range(3):
        step()
        torch.cuda.synchronize()
        ref.append([t.clone() for t in state])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    reset()
    for rep in range(3):
        Y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(state, ref[rep])):
            assert torch.equal(o, r), f"replay {rep}: state {i} differs from eager step {rep}"
        log(f"replay {rep}: outputs and delayed-scaling state equal to eager step {rep}")


def test_attention_block_in_a_graph(tpm):
    import torch
    from workloads import AttnWorkload, make_attn_inputs
    wl = AttnWorkload("graph_attn", B=2, S=192, d=512, heads=4, N=2, sigma=0.02, seed=40)
    X, Wqkv, Wo = make_attn_inputs(wl)
    Xd, Wd, Wod = dev_bf16(X), dev_bf16(Wqkv), dev_bf16(Wo)
    M, F = wl.B * wl.S, wl.F
    hr = wl.heads // wl.N
    QKV = torch.empty((M, 3 * F), dtype=torch.bfloat16, device="cuda")
    O = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    parts = [torch.empty((M, wl.d), dtype=torch.float32, device="cuda") for _ in range(wl.N)]
    Y = torch.empty((M, wl.d), dtype=torch.float32, device="cuda")

    def step():
        for r in range(wl.N):
            tpm.tp_attn_qkv(Xd, Wd[:, r * 3 * F:(r + 1) * 3 * F], QKV)
            tpm.tp_attn_heads(QKV, wl.B, wl.S, hr, True, O)
            tpm.tp_mlp_row_partial(O, Wod[r * F:(r + 1) * F, :], parts[r])
        tpm.tp_partial_sum(parts, Y=Y)
    _replay_and_compare(step, parts + [Y])
