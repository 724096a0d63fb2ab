"""Host-side helpers shared by the GPU tests: moving bit arrays to and from the
device and the error norm of the parity bar (no arithmetic of the path)."""
import sys

import numpy as np


def log(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_u8(codes: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).cuda()


def dev_f32(values) -> "torch.Tensor":
    import torch
    return torch.tensor(np.asarray(values, dtype=np.float32).reshape(-1)).cuda()


def host_bf16_bits(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def host_f64(t) -> np.ndarray:
    import torch
    return t.detach().cpu().to(torch.float64).numpy()


def max_err_ratio(got, ref) -> float:
    """max|got − ref| / max|ref| (the parity bar's norm)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (2^(e−7), subnormal floor 2^-133)."""
    ax = np.abs(np.asarray(x, np.float64))
    _, e = np.frexp(np.maximum(ax, 2.0 ** -126))
    return np.ldexp(1.0, e - 1 - 7)
