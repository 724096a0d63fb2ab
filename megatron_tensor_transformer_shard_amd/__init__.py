"""One tensor-parallel rank's share of the Megatron MLP block on MI355X.

Y_i = GeLU(X·A_i)·B_i, with A_i the column block and B_i the matching row
block of the MLP weights ("Megatron architecture and 6D parallel guide",
§3.1; "Megatron-LM deep architecture", column/row-parallel section), and
Y = Σ_i Y_i.

This module is a thin ctypes binding over libtpmlp.so (C ABI in
include/tpmlp.h): it checks tensor dtypes/devices/contiguity, passes raw
device pointers, sizes and torch's current HIP stream, and raises on a
non-zero status. Every step of the computation runs in the library's HIP
kernels; there is no fallback. Importing fails loudly when the library has
not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime that libtpmlp.so then binds to

__all__ = [
    "LIB_PATH", "ABI_VERSION", "TpmError", "abi_version", "status_string",
    "tp_mlp_col_gelu", "tp_mlp_row_partial", "tp_mlp_shard", "tp_mlp_shard_workspace_size",
    "tp_mlp_col_gelu_wt", "tp_mlp_row_partial_wt", "tp_mlp_shard_wt",
    "tp_mlp_col_gelu_bias", "tp_mlp_col_gelu_bias_wt",
    "tp_partial_sum", "tp_partial_sum_rows", "tp_reduce_scatter_share", "tp_amax_bf16", "tp_quant_e4m3", "tp_mlp_col_gelu_e4m3",
    "tp_mlp_row_partial_e4m3", "tp_mlp_shard_e4m3", "tp_mlp_shard_e4m3_workspace_size",
    "tp_amax_history_push", "tp_mlp_col_gelu_e4m3_delayed", "tp_mlp_shard_e4m3_delayed",
    "tp_mlp_shard_e4m3_delayed_workspace_size", "AmaxHistory",
    "tp_mlp_shard_backward", "tp_mlp_shard_backward_workspace_size", "backward_workspace_views",
    "tp_mlp_shard_backward_bias", "tp_mlp_shard_backward_bias_workspace_size",
    "tp_bias_grad_bf16", "tp_bias_grad_workspace_size",
    "tp_mlp_shard_backward_fp8_bias", "tp_mlp_shard_backward_fp8_bias_workspace_size",
    "tp_mlp_shard_backward_fp8", "tp_mlp_shard_backward_fp8_workspace_size",
    "tp_attn_qkv", "tp_attn_heads", "tp_attn_shard", "tp_attn_shard_workspace_size",
    "attn_workspace_views", "ATTN_HEAD_DIM", "fp8_backward_workspace_views",
    "TPM_BF16", "TPM_F32", "TPM_E4M3", "EXPORTED_SYMBOLS",
    "tp_mlp_shard_noalloc", "NOALLOC_SCRATCH_BYTES", "tp_clock_stamp_count",
    "tp_mlp_col_gelu_stamped", "tp_mlp_row_partial_stamped", "tp_mlp_row_partial_e4m3_stamped",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtpmlp.so")

TPM_BF16, TPM_F32, TPM_E4M3 = 0, 1, 2
ATTN_HEAD_DIM = 128  # TPM_ATTN_HEAD_DIM
TPM_MAX_PARTS = 64
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024  # TPM_NOALLOC_SCRATCH_BYTES

_i64, _int, _vp, _sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
_fp = ctypes.c_void_p  # float* (device)

# name -> (restype, argtypes); mirrors include/tpmlp.h
_SIGNATURES = {
    "tp_abi_version": (_int, []),
    "tp_status_string": (ctypes.c_char_p, [_int]),
    "tp_mlp_col_gelu": (_int, [_vp, _vp, _i64, _vp, _i64, _i64, _i64, _vp]),
    "tp_mlp_row_partial": (_int, [_vp, _vp, _vp, _int, _i64, _i64, _i64, _vp]),
    "tp_mlp_shard_workspace_size": (_sz, [_i64, _i64, _i64, _int]),
    "tp_mlp_shard": (_int, [_vp, _vp, _vp, _vp, _int, _i64, _i64, _i64, _int, _int, _vp, _sz, _vp]),
    "tp_mlp_col_gelu_wt": (_int, [_vp, _vp, _i64, _vp, _i64, _i64, _i64, _vp]),
    "tp_mlp_col_gelu_bias": (_int, [_vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _vp]),
    "tp_mlp_col_gelu_bias_wt": (_int, [_vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _vp]),
    "tp_mlp_row_partial_wt": (_int, [_vp, _vp, _i64, _vp, _int, _i64, _i64, _i64, _vp]),
    "tp_mlp_shard_wt": (_int, [_vp, _vp, _vp, _vp, _int, _i64, _i64, _i64, _int, _int, _vp, _sz, _vp]),
    "tp_partial_sum": (_int, [ctypes.POINTER(_vp), _int, _int, _vp, _int, _i64, _vp]),
    "tp_partial_sum_rows": (_int, [ctypes.POINTER(_vp), _int, _int, _i64, _i64, _i64, _i64, _vp,
                                   _int, _vp, _int, _vp]),
    "tp_amax_bf16": (_int, [_vp, _i64, _fp, _vp]),
    "tp_quant_e4m3": (_int, [_vp, _i64, _fp, _vp, _fp, _vp]),
    "tp_mlp_col_gelu_e4m3": (_int, [_vp, _fp, _vp, _i64, _fp, _vp, _fp, _i64, _i64, _i64, _vp]),
    "tp_mlp_row_partial_e4m3": (_int, [_vp, _fp, _vp, _fp, _vp, _i64, _i64, _i64, _vp]),
    "tp_mlp_shard_e4m3_workspace_size": (_sz, [_i64, _i64, _i64, _int]),
    "tp_mlp_shard_e4m3": (_int, [_vp, _fp, _vp, _fp, _vp, _fp, _vp, _i64, _i64, _i64, _int, _int,
                                 _vp, _sz, _vp]),
    "tp_amax_history_push": (_int, [_fp, _vp, _int, _fp, _fp, _vp]),
    "tp_mlp_col_gelu_e4m3_delayed": (_int, [_vp, _fp, _vp, _i64, _fp, _fp, _vp, _fp, _i64, _i64,
                                            _i64, _vp]),
    "tp_mlp_shard_e4m3_delayed_workspace_size": (_sz, [_i64, _i64, _i64, _int]),
    "tp_mlp_shard_e4m3_delayed": (_int, [_vp, _fp, _vp, _fp, _vp, _fp, _fp, _vp, _fp, _i64, _i64,
                                         _i64, _int, _int, _vp, _sz, _vp]),
    "tp_mlp_shard_backward_workspace_size": (_sz, [_i64, _i64, _i64, _int]),
    "tp_mlp_shard_backward": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int,
                                     _int, _vp, _sz, _vp]),
    "tp_mlp_shard_backward_bias_workspace_size": (_sz, [_i64, _i64, _i64, _int]),
    "tp_mlp_shard_backward_bias": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64,
                                          _i64, _int, _int, _vp, _sz, _vp]),
    "tp_bias_grad_workspace_size": (_sz, [_i64, _i64]),
    "tp_mlp_shard_backward_fp8_bias_workspace_size": (_sz, [_i64, _i64, _i64, _int]),
    "tp_mlp_shard_backward_fp8_bias": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64,
                                              _i64, _i64, _int, _int, _vp, _vp, _sz, _vp]),
    "tp_bias_grad_bf16": (_int, [_vp, _i64, _i64, _i64, _vp, _vp, _sz, _vp]),
    "tp_attn_qkv": (_int, [_vp, _vp, _i64, _vp, _i64, _i64, _i64, _vp]),
    "tp_attn_heads": (_int, [_vp, _i64, _vp, _i64, _i64, _i64, _i64, _int, _vp]),
    "tp_attn_shard_workspace_size": (_sz, [_i64, _i64, _int]),
    "tp_attn_shard": (_int, [_vp, _vp, _vp, _vp, _int, _i64, _i64, _i64, _i64, _int, _int, _int,
                             _vp, _sz, _vp]),
    "tp_mlp_shard_backward_fp8_workspace_size": (_sz, [_i64, _i64, _i64, _int]),
    "tp_mlp_shard_backward_fp8": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                         _int, _int, _vp, _vp, _sz, _vp]),
    "tp_reduce_scatter_share": (_int, [ctypes.POINTER(_vp), _int, _int, _i64, _i64, _int, _vp, _int,
                                       _vp, _int, _vp]),
    "tp_mlp_shard_noalloc": (_int, [_vp, _vp, _vp, _vp, _int, _i64, _i64, _i64, _int, _int, _vp]),
    "tp_clock_stamp_count": (_i64, [_i64, _i64]),
    "tp_mlp_col_gelu_stamped": (_int, [_vp, _vp, _i64, _vp, _i64, _i64, _i64, _vp, _i64, _vp]),
    "tp_mlp_row_partial_stamped": (_int, [_vp, _vp, _vp, _int, _i64, _i64, _i64, _vp, _i64, _vp]),
    "tp_mlp_row_partial_e4m3_stamped": (_int, [_vp, _fp, _vp, _fp, _vp, _i64, _i64, _i64, _vp, _i64,
                                               _vp]),
}
EXPORTED_SYMBOLS = tuple(_SIGNATURES)


# The entry-point signatures below are those of this ABI version of include/tpmlp.h.
ABI_VERSION = 7


def _load_library():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python megatron_tensor_transformer_shard_amd/build_lib.py` "
            "from the repository root (there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.tp_abi_version() != ABI_VERSION:
        raise ImportError(
            f"{LIB_PATH} has ABI version {lib.tp_abi_version()}, these bindings expect "
            f"{ABI_VERSION}: rebuild it with `python megatron_tensor_transformer_shard_amd/build_lib.py`")
    return lib


lib = _load_library()


class TpmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def abi_version() -> int:
    return lib.tp_abi_version()


def status_string(status: int) -> str:
    return lib.tp_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise TpmError(status, where)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, name: str, dtype, ndim=None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D (got shape {tuple(t.shape)})")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dtype_code(dt) -> int:
    if dt == torch.float32:
        return TPM_F32
    if dt == torch.bfloat16:
        return TPM_BF16
    raise TypeError(f"unsupported dtype {dt}")


def _fptr(t: torch.Tensor) -> int:
    _need(t, "scale/amax", torch.float32, contiguous=False)
    return t.data_ptr()


# --------------------------------------------------------------- bf16 path

def tp_mlp_col_gelu(X: torch.Tensor, A_i: torch.Tensor, Z_i: torch.Tensor | None = None,
                    stream=None, stamps: torch.Tensor | None = None) -> torch.Tensor:
    """Z_i = bf16(GeLU(X·A_i)). X [M, d] bf16; A_i [d, F] bf16 (may be a column
    slice of a full A: unit column stride, any row stride)."""
    _need(X, "X", torch.bfloat16, 2)
    _need(A_i, "A_i", torch.bfloat16, 2, contiguous=False)
    if A_i.stride(1) != 1:
        raise ValueError("A_i must have unit column stride")
    M, d = X.shape
    d2, F = A_i.shape
    if d2 != d:
        raise ValueError(f"inner dimensions differ: X {tuple(X.shape)}, A_i {tuple(A_i.shape)}")
    if Z_i is None:
        Z_i = torch.empty((M, F), dtype=torch.bfloat16, device=X.device)
    _need(Z_i, "Z_i", torch.bfloat16, 2)
    if tuple(Z_i.shape) != (M, F):
        raise ValueError("Z_i has the wrong shape")
    if stamps is None:
        _check(lib.tp_mlp_col_gelu(X.data_ptr(), A_i.data_ptr(), A_i.stride(0), Z_i.data_ptr(),
                                   M, d, F, _stream(stream)), "tp_mlp_col_gelu")
    else:
        _need(stamps, "stamps", torch.int64, 1)
        _check(lib.tp_mlp_col_gelu_stamped(X.data_ptr(), A_i.data_ptr(), A_i.stride(0),
                                           Z_i.data_ptr(), M, d, F, stamps.data_ptr(),
                                           stamps.numel(), _stream(stream)),
               "tp_mlp_col_gelu_stamped")
    return Z_i


def tp_clock_stamp_count(M: int, N: int) -> int:
    """Length of the stamps array the clock-stamped calls need for an [M, N] output."""
    return int(lib.tp_clock_stamp_count(M, N))


def tp_mlp_col_gelu_stamped(X, A_i, stamps, Z_i=None, stream=None):
    """tp_mlp_col_gelu with per-workgroup clock stamps in `stamps` (int64
    [tp_clock_stamp_count(M, F)], device; 4 per workgroup: shader-clock and
    100 MHz counters at the start and after the stores)."""
    return tp_mlp_col_gelu(X, A_i, Z_i, stream, stamps=stamps)


def tp_mlp_col_gelu_bias(X: torch.Tensor, A_i: torch.Tensor, b_i: torch.Tensor,
                         Z_i: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Z_i = bf16(GeLU(X·A_i + b_i)), the column-parallel linear with its bias.
    X [M, d] bf16; A_i [d, F] bf16 (unit column stride, any row stride);
    b_i [F] bf16, dense."""
    return _col_gelu_bias(X, A_i, b_i, Z_i, False, stream)


def tp_mlp_col_gelu_bias_wt(X: torch.Tensor, W1_i: torch.Tensor, b_i: torch.Tensor,
                            Z_i: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """tp_mlp_col_gelu_bias with W1_i [F, d] bf16, the [out, in] layout (unit
    column stride, any row stride)."""
    return _col_gelu_bias(X, W1_i, b_i, Z_i, True, stream)


def _col_gelu_bias(X, A_i, b_i, Z_i, transposed, stream):
    _need(X, "X", torch.bfloat16, 2)
    _need(A_i, "W1_i" if transposed else "A_i", torch.bfloat16, 2, contiguous=False)
    if A_i.stride(1) != 1:
        raise ValueError("the weight must have unit column stride")
    M, d = X.shape
    F, d2 = A_i.shape if transposed else A_i.shape[::-1]
    if d2 != d:
        raise ValueError(f"inner dimensions differ: X {tuple(X.shape)}, weight {tuple(A_i.shape)}")
    _need(b_i, "b_i", torch.bfloat16, 1)
    if b_i.numel() != F:
        raise ValueError(f"b_i has {b_i.numel()} values, the shard is {F} wide")
    if Z_i is None:
        Z_i = torch.empty((M, F), dtype=torch.bfloat16, device=X.device)
    _need(Z_i, "Z_i", torch.bfloat16, 2)
    if tuple(Z_i.shape) != (M, F):
        raise ValueError("Z_i has the wrong shape")
    fn = lib.tp_mlp_col_gelu_bias_wt if transposed else lib.tp_mlp_col_gelu_bias
    _check(fn(X.data_ptr(), A_i.data_ptr(), A_i.stride(0), b_i.data_ptr(), Z_i.data_ptr(),
              M, d, F, _stream(stream)),
           "tp_mlp_col_gelu_bias_wt" if transposed else "tp_mlp_col_gelu_bias")
    return Z_i


def tp_mlp_row_partial(Z_i: torch.Tensor, B_i: torch.Tensor, Y_i: torch.Tensor | None = None,
                       out_dtype=torch.float32, stream=None,
                       stamps: torch.Tensor | None = None) -> torch.Tensor:
    """Y_i = Z_i·B_i (fp32 or bf16). Z_i [M, F] bf16; B_i [F, d] bf16."""
    _need(Z_i, "Z_i", torch.bfloat16, 2)
    _need(B_i, "B_i", torch.bfloat16, 2)
    M, F = Z_i.shape
    F2, d = B_i.shape
    if F2 != F:
        raise ValueError(f"inner dimensions differ: Z_i {tuple(Z_i.shape)}, B_i {tuple(B_i.shape)}")
    if Y_i is None:
        Y_i = torch.empty((M, d), dtype=out_dtype, device=Z_i.device)
    _need(Y_i, "Y_i", None, 2)
    if tuple(Y_i.shape) != (M, d):
        raise ValueError("Y_i has the wrong shape")
    if stamps is None:
        _check(lib.tp_mlp_row_partial(Z_i.data_ptr(), B_i.data_ptr(), Y_i.data_ptr(),
                                      _dtype_code(Y_i.dtype), M, F, d, _stream(stream)),
               "tp_mlp_row_partial")
    else:
        _need(stamps, "stamps", torch.int64, 1)
        _check(lib.tp_mlp_row_partial_stamped(Z_i.data_ptr(), B_i.data_ptr(), Y_i.data_ptr(),
                                              _dtype_code(Y_i.dtype), M, F, d, stamps.data_ptr(),
                                              stamps.numel(), _stream(stream)),
               "tp_mlp_row_partial_stamped")
    return Y_i


def tp_mlp_row_partial_stamped(Z_i, B_i, stamps, Y_i=None, out_dtype=torch.float32, stream=None):
    """tp_mlp_row_partial with per-workgroup clock stamps (see tp_mlp_col_gelu_stamped)."""
    return tp_mlp_row_partial(Z_i, B_i, Y_i, out_dtype, stream, stamps=stamps)


def tp_mlp_shard_workspace_size(M: int, d: int, H: int, N: int) -> int:
    return int(lib.tp_mlp_shard_workspace_size(M, d, H, N))


def tp_mlp_shard(X: torch.Tensor, A: torch.Tensor, B: torch.Tensor, N: int, rank: int,
                 Y_i: torch.Tensor | None = None, out_dtype=torch.float32,
                 workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Rank `rank`'s partial output GeLU(X·A_i)·B_i of the N-way split of A [d, H], B [H, d]."""
    _need(X, "X", torch.bfloat16, 2)
    _need(A, "A", torch.bfloat16, 2)
    _need(B, "B", torch.bfloat16, 2)
    M, d = X.shape
    dA, H = A.shape
    if dA != d or tuple(B.shape) != (H, d):
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, A {tuple(A.shape)}, B {tuple(B.shape)}")
    if Y_i is None:
        Y_i = torch.empty((M, d), dtype=out_dtype, device=X.device)
    _need(Y_i, "Y_i", None, 2)
    if tuple(Y_i.shape) != (M, d):
        raise ValueError("Y_i has the wrong shape")
    need = tp_mlp_shard_workspace_size(M, d, H, N) if N >= 1 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=X.device)
    _need(workspace, "workspace", None)
    _check(lib.tp_mlp_shard(X.data_ptr(), A.data_ptr(), B.data_ptr(), Y_i.data_ptr(),
                            _dtype_code(Y_i.dtype), M, d, H, N, rank, workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), _stream(stream)),
           "tp_mlp_shard")
    return Y_i


def tp_mlp_shard_noalloc(X: torch.Tensor, A: torch.Tensor, B: torch.Tensor, N: int, rank: int,
                         Y_i: torch.Tensor, stream=None) -> torch.Tensor:
    """tp_mlp_shard without a workspace: Z_i goes to the library's static
    device scratch (NOALLOC_SCRATCH_BYTES per device), so the call allocates
    nothing; the caller passes the output. Calls that overlap in time on one
    device share that scratch and race."""
    _need(X, "X", torch.bfloat16, 2)
    _need(A, "A", torch.bfloat16, 2)
    _need(B, "B", torch.bfloat16, 2)
    _need(Y_i, "Y_i", None, 2)
    M, d = X.shape
    H = A.shape[1]
    _check(lib.tp_mlp_shard_noalloc(X.data_ptr(), A.data_ptr(), B.data_ptr(), Y_i.data_ptr(),
                                    _dtype_code(Y_i.dtype), M, d, H, N, rank, _stream(stream)),
           "tp_mlp_shard_noalloc")
    return Y_i


# The forward with the weights stored transposed, as the pages' column- and
# row-parallel linear layers keep them ([out_features, in_features]).

def tp_mlp_col_gelu_wt(X: torch.Tensor, W1_i: torch.Tensor, Z_i: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """Z_i = bf16(GeLU(X·W1_iᵀ)). X [M, d] bf16; W1_i [F, d] bf16 (the column-parallel
    layer's weight: unit column stride, any row stride)."""
    _need(X, "X", torch.bfloat16, 2)
    _need(W1_i, "W1_i", torch.bfloat16, 2, contiguous=False)
    if W1_i.stride(1) != 1:
        raise ValueError("W1_i must have unit column stride")
    M, d = X.shape
    F, d2 = W1_i.shape
    if d2 != d:
        raise ValueError(f"inner dimensions differ: X {tuple(X.shape)}, W1_i {tuple(W1_i.shape)}")
    if Z_i is None:
        Z_i = torch.empty((M, F), dtype=torch.bfloat16, device=X.device)
    _need(Z_i, "Z_i", torch.bfloat16, 2)
    if tuple(Z_i.shape) != (M, F):
        raise ValueError("Z_i has the wrong shape")
    _check(lib.tp_mlp_col_gelu_wt(X.data_ptr(), W1_i.data_ptr(), W1_i.stride(0), Z_i.data_ptr(),
                                  M, d, F, _stream(stream)), "tp_mlp_col_gelu_wt")
    return Z_i


def tp_mlp_row_partial_wt(Z_i: torch.Tensor, W2_i: torch.Tensor, Y_i: torch.Tensor | None = None,
                          out_dtype=torch.float32, stream=None) -> torch.Tensor:
    """Y_i = Z_i·W2_iᵀ (fp32 or bf16). Z_i [M, F] bf16; W2_i [d, F] bf16 (the row-parallel
    layer's weight, e.g. a column block of a full [d, H] weight: unit column stride)."""
    _need(Z_i, "Z_i", torch.bfloat16, 2)
    _need(W2_i, "W2_i", torch.bfloat16, 2, contiguous=False)
    if W2_i.stride(1) != 1:
        raise ValueError("W2_i must have unit column stride")
    M, F = Z_i.shape
    d, F2 = W2_i.shape
    if F2 != F:
        raise ValueError(f"inner dimensions differ: Z_i {tuple(Z_i.shape)}, W2_i {tuple(W2_i.shape)}")
    if Y_i is None:
        Y_i = torch.empty((M, d), dtype=out_dtype, device=Z_i.device)
    _need(Y_i, "Y_i", None, 2)
    if tuple(Y_i.shape) != (M, d):
        raise ValueError("Y_i has the wrong shape")
    _check(lib.tp_mlp_row_partial_wt(Z_i.data_ptr(), W2_i.data_ptr(), W2_i.stride(0),
                                     Y_i.data_ptr(), _dtype_code(Y_i.dtype), M, F, d,
                                     _stream(stream)), "tp_mlp_row_partial_wt")
    return Y_i


def tp_mlp_shard_wt(X: torch.Tensor, W1: torch.Tensor, W2: torch.Tensor, N: int, rank: int,
                    Y_i: torch.Tensor | None = None, out_dtype=torch.float32,
                    workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """tp_mlp_shard with the weights stored transposed: W1 = Aᵀ [H, d], W2 = Bᵀ [d, H]."""
    _need(X, "X", torch.bfloat16, 2)
    _need(W1, "W1", torch.bfloat16, 2)
    _need(W2, "W2", torch.bfloat16, 2)
    M, d = X.shape
    H, d1 = W1.shape
    if d1 != d or tuple(W2.shape) != (d, H):
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, W1 {tuple(W1.shape)}, W2 {tuple(W2.shape)}")
    if Y_i is None:
        Y_i = torch.empty((M, d), dtype=out_dtype, device=X.device)
    _need(Y_i, "Y_i", None, 2)
    if tuple(Y_i.shape) != (M, d):
        raise ValueError("Y_i has the wrong shape")
    need = tp_mlp_shard_workspace_size(M, d, H, N) if N >= 1 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=X.device)
    _need(workspace, "workspace", None)
    _check(lib.tp_mlp_shard_wt(X.data_ptr(), W1.data_ptr(), W2.data_ptr(), Y_i.data_ptr(),
                               _dtype_code(Y_i.dtype), M, d, H, N, rank, workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _stream(stream)),
           "tp_mlp_shard_wt")
    return Y_i


def tp_partial_sum(parts, Y: torch.Tensor | None = None, out_dtype=None,
                   stream=None) -> torch.Tensor:
    """Y = Σ_i parts[i], in rank order, fp32 accumulation."""
    parts = list(parts)
    if not parts:
        raise ValueError("no partials")
    dt = parts[0].dtype
    for i, p in enumerate(parts):
        _need(p, f"parts[{i}]", dt)
        if p.shape != parts[0].shape:
            raise ValueError("partials differ in shape")
    if Y is None:
        Y = torch.empty(parts[0].shape, dtype=out_dtype or dt, device=parts[0].device)
    _need(Y, "Y", None)
    if Y.numel() != parts[0].numel():
        raise ValueError("Y has the wrong size")
    arr = (_vp * len(parts))(*[p.data_ptr() for p in parts])
    _check(lib.tp_partial_sum(arr, len(parts), _dtype_code(dt), Y.data_ptr(),
                              _dtype_code(Y.dtype), parts[0].numel(), _stream(stream)),
           "tp_partial_sum")
    return Y


def tp_partial_sum_rows(parts, row_begin: int, row_end: int, bias: torch.Tensor | None = None,
                        Y: torch.Tensor | None = None, out_dtype=None, stream=None) -> torch.Tensor:
    """Rows [row_begin, row_end) of Σ_i parts[i] (rank order, fp32), plus
    `bias` once after the sum. parts are [M, d] tensors of one dtype."""
    parts = list(parts)
    if not parts:
        raise ValueError("no partials")
    dt = parts[0].dtype
    for i, p in enumerate(parts):
        _need(p, f"parts[{i}]", dt)
        if p.dim() != 2 or p.shape != parts[0].shape:
            raise ValueError("partials must be [M, d] tensors of one shape")
    M, d = parts[0].shape
    if Y is None:
        Y = torch.empty((max(0, row_end - row_begin), d), dtype=out_dtype or dt,
                        device=parts[0].device)
    _need(Y, "Y", None)
    if Y.numel() != max(0, row_end - row_begin) * d:
        raise ValueError("Y has the wrong size")
    bptr, bdt = None, TPM_F32
    if bias is not None:
        _need(bias, "bias", None)
        if bias.numel() != d:
            raise ValueError("bias must have d elements")
        bptr, bdt = bias.data_ptr(), _dtype_code(bias.dtype)
    arr = (_vp * len(parts))(*[p.data_ptr() for p in parts])
    _check(lib.tp_partial_sum_rows(arr, len(parts), _dtype_code(dt), M, d, row_begin, row_end,
                                   bptr, bdt, Y.data_ptr(), _dtype_code(Y.dtype), _stream(stream)),
           "tp_partial_sum_rows")
    return Y


def tp_reduce_scatter_share(parts, rank: int, bias: torch.Tensor | None = None,
                            Y: torch.Tensor | None = None, out_dtype=None,
                            stream=None) -> torch.Tensor:
    """Rank `rank`'s share of the sequence-parallel reduce-scatter: rows
    [rank·M/N, (rank+1)·M/N) of Σ_i parts[i] (N = len(parts)), plus bias once."""
    parts = list(parts)
    if not parts:
        raise ValueError("no partials")
    dt = parts[0].dtype
    for i, p in enumerate(parts):
        _need(p, f"parts[{i}]", dt, 2)
        if p.shape != parts[0].shape:
            raise ValueError("partials must be [M, d] tensors of one shape")
    M, d = parts[0].shape
    N = len(parts)
    if Y is None:
        Y = torch.empty((M // N if N else 0, d), dtype=out_dtype or dt, device=parts[0].device)
    _need(Y, "Y", None)
    bptr, bdt = None, TPM_F32
    if bias is not None:
        _need(bias, "bias", None)
        if bias.numel() != d:
            raise ValueError("bias must have d elements")
        bptr, bdt = bias.data_ptr(), _dtype_code(bias.dtype)
    if Y.numel() != (M // N) * d:
        raise ValueError("Y has the wrong size")
    arr = (_vp * N)(*[p.data_ptr() for p in parts])
    _check(lib.tp_reduce_scatter_share(arr, N, _dtype_code(dt), M, d, rank, bptr, bdt, Y.data_ptr(),
                                       _dtype_code(Y.dtype), _stream(stream)),
           "tp_reduce_scatter_share")
    return Y


# ---------------------------------------------------------------- fp8 path
# e4m3 tensors are carried as torch.uint8 tensors of codes.

def tp_amax_bf16(T: torch.Tensor, amax: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    _need(T, "T", torch.bfloat16)
    if amax is None:
        amax = torch.empty(1, dtype=torch.float32, device=T.device)
    _check(lib.tp_amax_bf16(T.data_ptr(), T.numel(), _fptr(amax), _stream(stream)), "tp_amax_bf16")
    return amax


def tp_quant_e4m3(T: torch.Tensor, amax: torch.Tensor, Tq: torch.Tensor | None = None,
                  scale: torch.Tensor | None = None, stream=None):
    """(Tq, scale): e4m3 codes (uint8) of T·s, s = 448/amax (device fp32)."""
    _need(T, "T", torch.bfloat16)
    if Tq is None:
        Tq = torch.empty(T.shape, dtype=torch.uint8, device=T.device)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=T.device)
    _need(Tq, "Tq", torch.uint8)
    _check(lib.tp_quant_e4m3(T.data_ptr(), T.numel(), _fptr(amax), Tq.data_ptr(), _fptr(scale),
                             _stream(stream)), "tp_quant_e4m3")
    return Tq, scale


def tp_mlp_col_gelu_e4m3(Xq, sX, Aq_i, sA, Z_i=None, z_amax=None, stream=None):
    _need(Xq, "Xq", torch.uint8, 2)
    _need(Aq_i, "Aq_i", torch.uint8, 2, contiguous=False)
    if Aq_i.stride(1) != 1:
        raise ValueError("Aq_i must have unit column stride")
    M, d = Xq.shape
    d2, F = Aq_i.shape
    if d2 != d:
        raise ValueError("inner dimensions differ")
    if Z_i is None:
        Z_i = torch.empty((M, F), dtype=torch.bfloat16, device=Xq.device)
    _need(Z_i, "Z_i", torch.bfloat16, 2)
    za = _fptr(z_amax) if z_amax is not None else None
    _check(lib.tp_mlp_col_gelu_e4m3(Xq.data_ptr(), _fptr(sX), Aq_i.data_ptr(), Aq_i.stride(0),
                                    _fptr(sA), Z_i.data_ptr(), za, M, d, F, _stream(stream)),
           "tp_mlp_col_gelu_e4m3")
    return Z_i


def tp_mlp_row_partial_e4m3(Zq, sZ, Bq_i, sB, Y_i=None, stream=None, stamps=None):
    _need(Zq, "Zq", torch.uint8, 2)
    _need(Bq_i, "Bq_i", torch.uint8, 2)
    M, F = Zq.shape
    F2, d = Bq_i.shape
    if F2 != F:
        raise ValueError("inner dimensions differ")
    if Y_i is None:
        Y_i = torch.empty((M, d), dtype=torch.bfloat16, device=Zq.device)
    _need(Y_i, "Y_i", torch.bfloat16, 2)
    if stamps is None:
        _check(lib.tp_mlp_row_partial_e4m3(Zq.data_ptr(), _fptr(sZ), Bq_i.data_ptr(), _fptr(sB),
                                           Y_i.data_ptr(), M, F, d, _stream(stream)),
               "tp_mlp_row_partial_e4m3")
    else:
        _need(stamps, "stamps", torch.int64, 1)
        _check(lib.tp_mlp_row_partial_e4m3_stamped(Zq.data_ptr(), _fptr(sZ), Bq_i.data_ptr(),
                                                   _fptr(sB), Y_i.data_ptr(), M, F, d,
                                                   stamps.data_ptr(), stamps.numel(),
                                                   _stream(stream)),
               "tp_mlp_row_partial_e4m3_stamped")
    return Y_i


def tp_mlp_row_partial_e4m3_stamped(Zq, sZ, Bq_i, sB, stamps, Y_i=None, stream=None):
    """tp_mlp_row_partial_e4m3 with per-workgroup clock stamps (see tp_mlp_col_gelu_stamped)."""
    return tp_mlp_row_partial_e4m3(Zq, sZ, Bq_i, sB, Y_i, stream, stamps=stamps)


def tp_mlp_shard_e4m3_workspace_size(M: int, d: int, H: int, N: int) -> int:
    return int(lib.tp_mlp_shard_e4m3_workspace_size(M, d, H, N))


def tp_mlp_shard_e4m3(Xq, sX, Aq, sA, Bq, sB, N: int = 1, rank: int = 0, Y_i=None,
                      workspace=None, stream=None):
    """fp8 partial output of one rank (bf16 [M, d]); see include/tpmlp.h."""
    _need(Xq, "Xq", torch.uint8, 2)
    _need(Aq, "Aq", torch.uint8, 2)
    _need(Bq, "Bq", torch.uint8, 2)
    M, d = Xq.shape
    dA, H = Aq.shape
    if dA != d or tuple(Bq.shape) != (H, d):
        raise ValueError("shape mismatch")
    if Y_i is None:
        Y_i = torch.empty((M, d), dtype=torch.bfloat16, device=Xq.device)
    _need(Y_i, "Y_i", torch.bfloat16, 2)
    need = tp_mlp_shard_e4m3_workspace_size(M, d, H, N) if N >= 1 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=Xq.device)
    _check(lib.tp_mlp_shard_e4m3(Xq.data_ptr(), _fptr(sX), Aq.data_ptr(), _fptr(sA), Bq.data_ptr(),
                                 _fptr(sB), Y_i.data_ptr(), M, d, H, N, rank, workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), _stream(stream)),
           "tp_mlp_shard_e4m3")
    return Y_i


# ------------------------------------------------------ fp8 delayed scaling

class AmaxHistory:
    """Device state of one tensor's delayed scale: a ring of the last L
    recorded amaxes, the count of recorded steps, and the scale the next step
    applies (`scale`, device fp32 [1]; `initial_scale` until the first push)."""

    def __init__(self, L: int, initial_scale: float = 1.0, device="cuda"):
        self.L = int(L)
        self.history = torch.zeros(self.L, dtype=torch.float32, device=device)
        self.count = torch.zeros(1, dtype=torch.int32, device=device)   # read as uint32
        self.scale = torch.full((1,), float(initial_scale), dtype=torch.float32, device=device)

    def push(self, amax: torch.Tensor, stream=None) -> torch.Tensor:
        tp_amax_history_push(self.history, self.count, amax, self.scale, stream)
        return self.scale


def tp_amax_history_push(history: torch.Tensor, count: torch.Tensor, amax: torch.Tensor,
                         next_scale: torch.Tensor, stream=None) -> torch.Tensor:
    _need(history, "history", torch.float32)
    if count.dtype != torch.int32 or count.numel() != 1 or not count.is_cuda:
        raise ValueError("count must be a one-element int32 device tensor")
    _check(lib.tp_amax_history_push(_fptr(history), count.data_ptr(), history.numel(), _fptr(amax),
                                    _fptr(next_scale), _stream(stream)), "tp_amax_history_push")
    return next_scale


def tp_mlp_col_gelu_e4m3_delayed(Xq, sX, Aq_i, sA, sZ, Zq_i=None, z_amax=None, stream=None):
    """(Zq_i, z_amax): Z quantised to e4m3 in the GEMM's epilogue with the
    given (predicted) scale sZ, and max|Z| of this call."""
    _need(Xq, "Xq", torch.uint8, 2)
    _need(Aq_i, "Aq_i", torch.uint8, 2, contiguous=False)
    if Aq_i.stride(1) != 1:
        raise ValueError("Aq_i must have unit column stride")
    M, d = Xq.shape
    d2, F = Aq_i.shape
    if d2 != d:
        raise ValueError("inner dimensions differ")
    if Zq_i is None:
        Zq_i = torch.empty((M, F), dtype=torch.uint8, device=Xq.device)
    if z_amax is None:
        z_amax = torch.empty(1, dtype=torch.float32, device=Xq.device)
    _need(Zq_i, "Zq_i", torch.uint8, 2)
    _check(lib.tp_mlp_col_gelu_e4m3_delayed(Xq.data_ptr(), _fptr(sX), Aq_i.data_ptr(),
                                            Aq_i.stride(0), _fptr(sA), _fptr(sZ), Zq_i.data_ptr(),
                                            _fptr(z_amax), M, d, F, _stream(stream)),
           "tp_mlp_col_gelu_e4m3_delayed")
    return Zq_i, z_amax


def tp_mlp_shard_e4m3_delayed_workspace_size(M: int, d: int, H: int, N: int) -> int:
    return int(lib.tp_mlp_shard_e4m3_delayed_workspace_size(M, d, H, N))


def tp_mlp_shard_e4m3_delayed(Xq, sX, Aq, sA, Bq, sB, sZ, N: int, rank: int, Y_i=None,
                              z_amax=None, workspace=None, stream=None):
    """(Y_i, z_amax): rank `rank`'s fp8 partial output with Z quantised by sZ."""
    for t, n in ((Xq, "Xq"), (Aq, "Aq"), (Bq, "Bq")):
        _need(t, n, torch.uint8, 2)
    M, d = Xq.shape
    H = Aq.shape[1]
    if Y_i is None:
        Y_i = torch.empty((M, d), dtype=torch.bfloat16, device=Xq.device)
    if z_amax is None:
        z_amax = torch.empty(1, dtype=torch.float32, device=Xq.device)
    need = tp_mlp_shard_e4m3_delayed_workspace_size(M, d, H, N)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=Xq.device)
    _check(lib.tp_mlp_shard_e4m3_delayed(Xq.data_ptr(), _fptr(sX), Aq.data_ptr(), _fptr(sA),
                                         Bq.data_ptr(), _fptr(sB), _fptr(sZ), Y_i.data_ptr(),
                                         _fptr(z_amax), M, d, H, N, rank, workspace.data_ptr(),
                                         workspace.numel() * workspace.element_size(),
                                         _stream(stream)), "tp_mlp_shard_e4m3_delayed")
    return Y_i, z_amax


def tp_mlp_shard_backward_workspace_size(M: int, d: int, H: int, N: int) -> int:
    return int(lib.tp_mlp_shard_backward_workspace_size(M, d, H, N))


def tp_mlp_shard_backward(X, A, B, dY, N: int, rank: int, dX_i=None, dA_i=None, dB_i=None,
                          workspace=None, stream=None, b1=None, db1_i=None):
    """Gradients of rank `rank`'s shard for the output gradient dY.

    Returns (dX_i, dA_i, dB_i, workspace): fp32 [M, d], [d, F], [F, d]; the
    workspace (uint8) holds S (fp32), dS and Z (bf16), [M, F] each, at the
    offsets `backward_workspace_views` gives. With the column layer's bias b1
    the tuple has five entries, (dX_i, dA_i, dB_i, db1_i, workspace); db1_i
    without b1 is an error (there is no bias gradient to write).
    """
    if b1 is None and db1_i is not None:
        raise ValueError("db1_i is given without b1")
    _need(X, "X", torch.bfloat16, 2)
    _need(A, "A", torch.bfloat16, 2)
    _need(B, "B", torch.bfloat16, 2)
    _need(dY, "dY", torch.bfloat16, 2)
    M, d = X.shape
    dA, H = A.shape
    if dA != d or tuple(B.shape) != (H, d) or tuple(dY.shape) != (M, d):
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, A {tuple(A.shape)}, "
                         f"B {tuple(B.shape)}, dY {tuple(dY.shape)}")
    if N < 1 or H % N != 0:
        raise ValueError("H must be divisible by N")
    F = H // N
    dev = X.device
    if dX_i is None:
        dX_i = torch.empty((M, d), dtype=torch.float32, device=dev)
    if dA_i is None:
        dA_i = torch.empty((d, F), dtype=torch.float32, device=dev)
    if dB_i is None:
        dB_i = torch.empty((F, d), dtype=torch.float32, device=dev)
    for t, name, shp in ((dX_i, "dX_i", (M, d)), (dA_i, "dA_i", (d, F)), (dB_i, "dB_i", (F, d))):
        _need(t, name, torch.float32, 2)
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} has the wrong shape")
    if b1 is not None:
        _need(b1, "b1", torch.bfloat16, 1)
        if b1.numel() != H:
            raise ValueError(f"b1 has {b1.numel()} values, the hidden width is {H}")
        if db1_i is None:
            db1_i = torch.empty(F, dtype=torch.float32, device=dev)
        _need(db1_i, "db1_i", torch.float32, 1)
        if db1_i.numel() != F:
            raise ValueError("db1_i has the wrong shape")
        need = tp_mlp_shard_backward_bias_workspace_size(M, d, H, N)
    else:
        need = tp_mlp_shard_backward_workspace_size(M, d, H, N)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", None)
    wsb = workspace.numel() * workspace.element_size()
    if b1 is None:
        _check(lib.tp_mlp_shard_backward(X.data_ptr(), A.data_ptr(), B.data_ptr(), dY.data_ptr(),
                                         dX_i.data_ptr(), dA_i.data_ptr(), dB_i.data_ptr(), M, d,
                                         H, N, rank, workspace.data_ptr(), wsb, _stream(stream)),
               "tp_mlp_shard_backward")
        return dX_i, dA_i, dB_i, workspace
    _check(lib.tp_mlp_shard_backward_bias(X.data_ptr(), A.data_ptr(), b1.data_ptr(), B.data_ptr(),
                                          dY.data_ptr(), dX_i.data_ptr(), dA_i.data_ptr(),
                                          dB_i.data_ptr(), db1_i.data_ptr(), M, d, H, N, rank,
                                          workspace.data_ptr(), wsb, _stream(stream)),
           "tp_mlp_shard_backward_bias")
    return dX_i, dA_i, dB_i, db1_i, workspace


def tp_mlp_shard_backward_bias_workspace_size(M: int, d: int, H: int, N: int) -> int:
    return int(lib.tp_mlp_shard_backward_bias_workspace_size(M, d, H, N))


def tp_mlp_shard_backward_bias(X, A, b1, B, dY, N: int, rank: int, dX_i=None, dA_i=None,
                               dB_i=None, db1_i=None, workspace=None, stream=None):
    """tp_mlp_shard_backward when the forward added the column layer's bias
    b1 [H] (bf16) before GeLU: S is recomputed with the rank's block of b1,
    and db1_i = Σ_m dS[m, :] (fp32 [F]) is returned as well.

    Returns (dX_i, dA_i, dB_i, db1_i, workspace); the workspace's first three
    parts are those `backward_workspace_views` gives.
    """
    if b1 is None:
        raise ValueError("b1 is required")
    return tp_mlp_shard_backward(X, A, B, dY, N, rank, dX_i, dA_i, dB_i, workspace, stream,
                                 b1=b1, db1_i=db1_i)


def tp_bias_grad_workspace_size(rows: int, cols: int) -> int:
    return int(lib.tp_bias_grad_workspace_size(rows, cols))


def tp_bias_grad_bf16(G, db=None, workspace=None, stream=None):
    """db = Σ_r G[r, :] in fp32: the gradient of a bias added to every row of a
    layer's output whose gradient is G (bf16 [rows, cols], unit column
    stride, any row stride). For the row layer's bias, G = dY."""
    _need(G, "G", torch.bfloat16, 2, contiguous=False)
    if G.stride(1) != 1:
        raise ValueError("G must have unit column stride")
    rows, cols = G.shape
    if db is None:
        db = torch.empty(cols, dtype=torch.float32, device=G.device)
    _need(db, "db", torch.float32, 1)
    if db.numel() != cols:
        raise ValueError("db has the wrong shape")
    need = tp_bias_grad_workspace_size(rows, cols)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=G.device)
    _need(workspace, "workspace", None)
    _check(lib.tp_bias_grad_bf16(G.data_ptr(), G.stride(0), rows, cols, db.data_ptr(),
                                 workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                 _stream(stream)), "tp_bias_grad_bf16")
    return db


def backward_workspace_views(workspace, M: int, F: int):
    """(S fp32, dS bf16, Z bf16) views, [M, F] each, of a backward workspace."""
    def r256(b):
        return (b + 255) // 256 * 256
    mf = M * F
    o1 = r256(4 * mf)
    o2 = o1 + r256(2 * mf)
    S = workspace[: 4 * mf].view(torch.float32).view(M, F)
    dS = workspace[o1: o1 + 2 * mf].view(torch.bfloat16).view(M, F)
    Z = workspace[o2: o2 + 2 * mf].view(torch.bfloat16).view(M, F)
    return S, dS, Z


def tp_attn_qkv(X, W_i, QKV_i=None, stream=None):
    """Column-parallel QKV projection QKV_i = bf16(X·W_i); W_i may be a column view (row stride)."""
    _need(X, "X", torch.bfloat16, 2)
    _need(W_i, "W_i", torch.bfloat16, 2, contiguous=False)
    M, d = X.shape
    if W_i.shape[0] != d or W_i.stride(1) != 1:
        raise ValueError("W_i must be [d, F3] with unit column stride")
    F3 = W_i.shape[1]
    if QKV_i is None:
        QKV_i = torch.empty((M, F3), dtype=torch.bfloat16, device=X.device)
    _need(QKV_i, "QKV_i", torch.bfloat16, 2)
    if tuple(QKV_i.shape) != (M, F3):
        raise ValueError("QKV_i has the wrong shape")
    _check(lib.tp_attn_qkv(X.data_ptr(), W_i.data_ptr(), W_i.stride(0), QKV_i.data_ptr(), M, d, F3,
                           _stream(stream)), "tp_attn_qkv")
    return QKV_i


def tp_attn_heads(QKV, B: int, S: int, heads: int, causal: bool = True, O=None, stream=None):
    """Per-head softmax attention: QKV [B·S, ≥3·heads·128] (head-major groups) -> O [B·S, heads·128]."""
    _need(QKV, "QKV", torch.bfloat16, 2, contiguous=False)
    if QKV.shape[0] != B * S or QKV.stride(1) != 1:
        raise ValueError("QKV must be [B·S, ld] with unit column stride")
    F = heads * ATTN_HEAD_DIM
    if O is None:
        O = torch.empty((B * S, F), dtype=torch.bfloat16, device=QKV.device)
    _need(O, "O", torch.bfloat16, 2, contiguous=False)
    if O.shape[0] != B * S or O.shape[1] < F or O.stride(1) != 1:
        raise ValueError("O has the wrong shape")
    _check(lib.tp_attn_heads(QKV.data_ptr(), QKV.stride(0), O.data_ptr(), O.stride(0), B, S, heads,
                             int(bool(causal)), _stream(stream)), "tp_attn_heads")
    return O


def tp_attn_shard_workspace_size(M: int, d: int, N: int) -> int:
    return int(lib.tp_attn_shard_workspace_size(M, d, N))


def tp_attn_shard(X, Wqkv, Wo, B: int, S: int, heads: int, N: int, rank: int, causal: bool = True,
                  Y_i=None, out_dtype=torch.float32, workspace=None, stream=None):
    """Rank `rank`'s partial output of the N-way split attention block (W_qkv head-major [d, 3d])."""
    _need(X, "X", torch.bfloat16, 2)
    _need(Wqkv, "Wqkv", torch.bfloat16, 2)
    _need(Wo, "Wo", torch.bfloat16, 2)
    M, d = X.shape
    if tuple(Wqkv.shape) != (d, 3 * d) or tuple(Wo.shape) != (d, d) or M != B * S:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, Wqkv {tuple(Wqkv.shape)}, "
                         f"Wo {tuple(Wo.shape)}, B·S = {B * S}")
    if Y_i is None:
        Y_i = torch.empty((M, d), dtype=out_dtype, device=X.device)
    _need(Y_i, "Y_i", None, 2)
    if tuple(Y_i.shape) != (M, d):
        raise ValueError("Y_i has the wrong shape")
    need = tp_attn_shard_workspace_size(M, d, N) if N >= 1 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=X.device)
    _need(workspace, "workspace", None)
    _check(lib.tp_attn_shard(X.data_ptr(), Wqkv.data_ptr(), Wo.data_ptr(), Y_i.data_ptr(),
                             _dtype_code(Y_i.dtype), B, S, d, heads, N, rank, int(bool(causal)),
                             workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                             _stream(stream)), "tp_attn_shard")
    return Y_i


def attn_workspace_views(workspace, M: int, F: int):
    """(QKV_i bf16 [M, 3F], O_i bf16 [M, F]) views of an attention-shard workspace."""
    o1 = (6 * M * F + 255) // 256 * 256
    QKV = workspace[: 6 * M * F].view(torch.bfloat16).view(M, 3 * F)
    O = workspace[o1: o1 + 2 * M * F].view(torch.bfloat16).view(M, F)
    return QKV, O


def tp_mlp_shard_backward_fp8_workspace_size(M: int, d: int, H: int, N: int) -> int:
    return int(lib.tp_mlp_shard_backward_fp8_workspace_size(M, d, H, N))


def tp_mlp_shard_backward_fp8(X, A, B, dY, N: int, rank: int, dX_i=None, dA_i=None, dB_i=None,
                              workspace=None, stream=None, w_amax=None, b1=None, db1_i=None):
    """Gradients of rank `rank`'s shard with hybrid fp8 GEMMs (E4M3 activations and
    weights, E5M2 gradients). w_amax: None, or a device float32 tensor of two
    values, max|A| and max|B| over the whole weights (then they are not
    recomputed). Returns (dX_i, dA_i, dB_i, workspace); with the column layer's
    bias b1, (dX_i, dA_i, dB_i, db1_i, workspace). db1_i without b1 is an error."""
    if b1 is None and db1_i is not None:
        raise ValueError("db1_i is given without b1")
    for t, name in ((X, "X"), (A, "A"), (B, "B"), (dY, "dY")):
        _need(t, name, torch.bfloat16, 2)
    M, d = X.shape
    H = A.shape[1]
    if tuple(A.shape) != (d, H) or tuple(B.shape) != (H, d) or tuple(dY.shape) != (M, d):
        raise ValueError("shape mismatch")
    if N < 1 or H % N != 0:
        raise ValueError("H must be divisible by N")
    F = H // N
    dev = X.device
    dX_i = torch.empty((M, d), dtype=torch.float32, device=dev) if dX_i is None else dX_i
    dA_i = torch.empty((d, F), dtype=torch.float32, device=dev) if dA_i is None else dA_i
    dB_i = torch.empty((F, d), dtype=torch.float32, device=dev) if dB_i is None else dB_i
    for t, name, shp in ((dX_i, "dX_i", (M, d)), (dA_i, "dA_i", (d, F)), (dB_i, "dB_i", (F, d))):
        _need(t, name, torch.float32, 2)
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} has the wrong shape")
    if b1 is not None:
        _need(b1, "b1", torch.bfloat16, 1)
        if b1.numel() != H:
            raise ValueError(f"b1 has {b1.numel()} values, the hidden width is {H}")
        if db1_i is None:
            db1_i = torch.empty(F, dtype=torch.float32, device=dev)
        _need(db1_i, "db1_i", torch.float32, 1)
        if db1_i.numel() != F:
            raise ValueError("db1_i has the wrong shape")
        need = tp_mlp_shard_backward_fp8_bias_workspace_size(M, d, H, N)
    else:
        need = tp_mlp_shard_backward_fp8_workspace_size(M, d, H, N)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", None)
    if w_amax is not None:
        _need(w_amax, "w_amax", torch.float32)
        if w_amax.numel() != 2:
            raise ValueError("w_amax holds two values: max|A| and max|B|")
    wam = 0 if w_amax is None else w_amax.data_ptr()
    wsb = workspace.numel() * workspace.element_size()
    if b1 is None:
        _check(lib.tp_mlp_shard_backward_fp8(X.data_ptr(), A.data_ptr(), B.data_ptr(),
                                             dY.data_ptr(), dX_i.data_ptr(), dA_i.data_ptr(),
                                             dB_i.data_ptr(), M, d, H, N, rank, wam,
                                             workspace.data_ptr(), wsb, _stream(stream)),
               "tp_mlp_shard_backward_fp8")
        return dX_i, dA_i, dB_i, workspace
    _check(lib.tp_mlp_shard_backward_fp8_bias(X.data_ptr(), A.data_ptr(), b1.data_ptr(),
                                              B.data_ptr(), dY.data_ptr(), dX_i.data_ptr(),
                                              dA_i.data_ptr(), dB_i.data_ptr(), db1_i.data_ptr(),
                                              M, d, H, N, rank, wam, workspace.data_ptr(), wsb,
                                              _stream(stream)),
           "tp_mlp_shard_backward_fp8_bias")
    return dX_i, dA_i, dB_i, db1_i, workspace


def tp_mlp_shard_backward_fp8_bias_workspace_size(M: int, d: int, H: int, N: int) -> int:
    return int(lib.tp_mlp_shard_backward_fp8_bias_workspace_size(M, d, H, N))


def tp_mlp_shard_backward_fp8_bias(X, A, b1, B, dY, N: int, rank: int, dX_i=None, dA_i=None,
                                   dB_i=None, db1_i=None, workspace=None, stream=None,
                                   w_amax=None):
    """tp_mlp_shard_backward_fp8 when the forward added the column layer's bias
    b1 [H] (bf16) before GeLU. Returns (dX_i, dA_i, dB_i, db1_i, workspace);
    the workspace's views are those of `fp8_backward_workspace_views`."""
    if b1 is None:
        raise ValueError("b1 is required")
    return tp_mlp_shard_backward_fp8(X, A, B, dY, N, rank, dX_i, dA_i, dB_i, workspace, stream,
                                     w_amax, b1=b1, db1_i=db1_i)


def fp8_backward_workspace_views(workspace, M: int, d: int, F: int):
    """Named views of a tp_mlp_shard_backward_fp8 workspace: amax/scale floats
    and the codes and intermediates, in the layout the library uses."""
    def r256(b):
        return (b + 255) // 256 * 256
    o = 256
    views = {}
    for name, nbytes in (("Xq", M * d), ("XqT", M * d), ("Aq", d * F), ("AqT", d * F),
                         ("BqT", d * F), ("dYq", M * d), ("S", M * F * 4), ("dS", M * F * 2),
                         ("Z", M * F * 2), ("dSq", M * F), ("ZqT", M * F)):
        views[name] = workspace[o:o + nbytes]
        o += r256(nbytes)
    fl = workspace[:64].view(torch.float32)
    views["amax"], views["scale"] = fl[:6], fl[8:14]
    views["Xq"] = views["Xq"].view(M, d)
    views["XqT"] = views["XqT"].view(d, M)
    views["Aq"] = views["Aq"].view(d, F)
    views["AqT"] = views["AqT"].view(F, d)
    views["BqT"] = views["BqT"].view(d, F)
    views["dYq"] = views["dYq"].view(M, d)
    views["S"] = views["S"].view(torch.float32).view(M, F)
    views["dS"] = views["dS"].view(torch.bfloat16).view(M, F)
    views["Z"] = views["Z"].view(torch.bfloat16).view(M, F)
    views["dSq"] = views["dSq"].view(M, F)
    views["ZqT"] = views["ZqT"].view(F, M)
    return views
