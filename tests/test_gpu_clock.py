"""The clock-stamped measurement calls on the GPU: the same results as the
production calls, bit for bit, and one well-formed stamp quadruple per
workgroup (start before end on both counters, a plausible shader clock)."""
import numpy as np
import pytest

from helpers import dev_bf16, log
from workloads import make_random

pytestmark = pytest.mark.gpu

# constant counter read by s_memrealtime on MI300-series GPUs: 100 MHz
WALL_HZ = 100e6


@pytest.fixture(scope="module")
def tpm():
    import torch
    import megatron_tensor_transformer_shard_amd as m
    assert torch.cuda.is_available()
    return m


def _quads(stamps):
    q = stamps.cpu().numpy().view(np.uint64).reshape(-1, 4)
    used = q[np.any(q != 0, axis=1)]
    return q, used


def _check_quads(stamps, what):
    q, used = _quads(stamps)
    assert len(used) >= 1, f"{what}: no workgroup wrote its stamps"
    # the written quadruples are the first ones (workgroup ids 0 .. n-1)
    assert np.all(np.any(q[: len(used)] != 0, axis=1)), f"{what}: gaps in the stamps"
    s0, w0, s1, w1 = (used[:, i].astype(np.float64) for i in range(4))
    assert np.all(s1 > s0) and np.all(w1 > w0), f"{what}: an end stamp precedes its start"
    ghz = (s1 - s0) / ((w1 - w0) / WALL_HZ) / 1e9
    log(f"{what}: {len(used)} workgroups, shader clock median {np.median(ghz):.3f} GHz "
        f"(min {ghz.min():.3f}, max {ghz.max():.3f})")
    assert 0.1 < np.median(ghz) < 4.0
    return len(used)


@pytest.mark.parametrize("M,d,F", [(1024, 1024, 1024), (8192, 4096, 2048), (300, 136, 264)])
def test_stamped_bf16_steps_equal_production(tpm, M, d, F):
    import torch
    X, A, B = make_random(M, d, F, seed=M + d, sigma=0.05)
    Xd, Ad, Bd = dev_bf16(X), dev_bf16(A), dev_bf16(B)
    Z = tpm.tp_mlp_col_gelu(Xd, Ad)
    st = torch.zeros(tpm.tp_clock_stamp_count(M, F), dtype=torch.int64, device="cuda")
    Zs = tpm.tp_mlp_col_gelu_stamped(Xd, Ad, st)
    torch.cuda.synchronize()
    assert torch.equal(Z, Zs)
    _check_quads(st, f"col_gelu {M}x{d}x{F}")
    Y = tpm.tp_mlp_row_partial(Z, Bd)
    st2 = torch.zeros(tpm.tp_clock_stamp_count(M, d), dtype=torch.int64, device="cuda")
    Ys = tpm.tp_mlp_row_partial_stamped(Z, Bd, st2)
    torch.cuda.synchronize()
    assert torch.equal(Y, Ys)
    _check_quads(st2, f"row_partial {M}x{F}x{d}")


def test_stamped_fp8_row_step_equals_production(tpm):
    import torch
    import oracle
    from helpers import dev_f32, dev_u8
    M, F, d = 520, 512, 784
    Z, B, _ = make_random(M, F, d, seed=3, sigma=0.3)
    Zq, sZ = oracle.quantize_inputs_e4m3(Z)
    Bq, sB = oracle.quantize_inputs_e4m3(B)
    args = (dev_u8(Zq), dev_f32([sZ]), dev_u8(Bq), dev_f32([sB]))
    Y = tpm.tp_mlp_row_partial_e4m3(*args)
    st = torch.zeros(tpm.tp_clock_stamp_count(M, d), dtype=torch.int64, device="cuda")
    Ys = tpm.tp_mlp_row_partial_e4m3_stamped(*args, st)
    torch.cuda.synchronize()
    assert torch.equal(Y, Ys)
    _check_quads(st, f"row_partial_e4m3 {M}x{F}x{d}")
