"""The C-ABI library loads, exports every symbol include/tpmlp.h declares, and
rejects invalid arguments on the host before any HIP call (CPU only: every call
here returns from validation; none reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import megatron_tensor_transformer_shard_amd as tpm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpmlp.h")

OK, ENULL, EARG, ESHAPE, EDTYPE, EALIGN, EWS, EALIAS, EHIP, ESCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
BF16, F32, E4M3 = 0, 1, 2

# Fake, never-dereferenced "device" addresses; validation only inspects them.
BASE = 1 << 40
GB = 1 << 30


def _declared_functions():
    with open(HEADER) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(tp_\w+)\s*\(", text, flags=re.M)))


def test_header_and_binding_agree():
    declared = _declared_functions()
    assert len(declared) >= 13
    assert sorted(tpm.EXPORTED_SYMBOLS) == declared


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(tpm.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    assert tpm.abi_version() == tpm.ABI_VERSION == 7
    for code in (OK, ENULL, EARG, ESHAPE, EDTYPE, EALIGN, EWS, EALIAS, EHIP, ESCRATCH):
        s = tpm.status_string(code)
        assert s.startswith("TPM_")
    assert "unknown" in tpm.status_string(12345)


L = tpm.lib


def col_gelu(X=BASE, A=BASE + GB, lda=256, Z=BASE + 2 * GB, M=32, d=64, F=256):
    return L.tp_mlp_col_gelu(X, A, lda, Z, M, d, F, None)


def test_col_gelu_validation():
    assert col_gelu(M=0) == OK                       # empty: no-op, nothing launched
    assert col_gelu(X=None) == ENULL
    assert col_gelu(Z=None) == ENULL
    assert col_gelu(M=-1) == ESHAPE
    assert col_gelu(d=0) == ESHAPE
    assert col_gelu(d=60) == ESHAPE                   # not a multiple of 8
    assert col_gelu(F=12) == ESHAPE
    assert col_gelu(lda=128) == ESHAPE                # lda < F
    assert col_gelu(lda=260) == EALIGN                # row stride not 16-byte multiple
    assert col_gelu(X=BASE + 2) == EALIGN
    assert col_gelu(Z=BASE + 96) == EALIAS            # Z overlaps X
    assert col_gelu(Z=BASE + GB + 512) == EALIAS      # Z overlaps A_i
    assert col_gelu(M=1 << 31) == ESHAPE


def row_partial(Z=BASE, B=BASE + GB, Y=BASE + 2 * GB, yd=F32, M=32, F=128, d=64):
    return L.tp_mlp_row_partial(Z, B, Y, yd, M, F, d, None)


def test_row_partial_validation():
    assert row_partial(M=0) == OK
    assert row_partial(yd=E4M3) == EDTYPE
    assert row_partial(yd=7) == EDTYPE
    assert row_partial(B=None) == ENULL
    assert row_partial(d=12) == ESHAPE
    assert row_partial(Y=BASE + 8) == EALIGN
    assert row_partial(Y=BASE + 16) == EALIAS


def shard(X=BASE, A=BASE + GB, B=BASE + 2 * GB, Y=BASE + 3 * GB, yd=F32, M=32, d=64, H=256,
          N=2, rank=0, ws=BASE + 4 * GB, wsb=None):
    if wsb is None:
        wsb = L.tp_mlp_shard_workspace_size(M, d, H, N)
    return L.tp_mlp_shard(X, A, B, Y, yd, M, d, H, N, rank, ws, wsb, None)


def test_shard_validation():
    assert L.tp_mlp_shard_workspace_size(32, 64, 256, 2) == 32 * 128 * 2
    assert L.tp_mlp_shard_workspace_size(32, 64, 256, 3) == 0
    assert shard(M=0) == OK
    assert shard(N=0) == EARG
    assert shard(rank=2) == EARG
    assert shard(rank=-1) == EARG
    assert shard(N=3) == ESHAPE                        # 4d not divisible by N
    assert shard(N=64, H=256) == ESHAPE                # F = 4 not a multiple of 8
    assert shard(yd=E4M3) == EDTYPE
    assert shard(ws=None) == EWS
    assert shard(wsb=100) == EWS
    assert shard(ws=BASE + 4 * GB + 4) == EALIGN
    assert shard(Y=BASE + 64) == EALIAS               # Y overlaps X
    assert shard(ws=BASE + GB) == EALIAS               # workspace overlaps A
    assert shard(Y=BASE + 4 * GB) == EALIAS            # Y overlaps workspace


def col_gelu_wt(X=BASE, W=BASE + GB, ldw=64, Z=BASE + 2 * GB, M=32, d=64, F=256):
    return L.tp_mlp_col_gelu_wt(X, W, ldw, Z, M, d, F, None)


def test_col_gelu_wt_validation():
    assert col_gelu_wt(M=0) == OK
    assert col_gelu_wt(W=None) == ENULL
    assert col_gelu_wt(d=60) == ESHAPE
    assert col_gelu_wt(ldw=56) == ESHAPE              # ldw < d
    assert col_gelu_wt(ldw=68) == EALIGN              # row stride not 16-byte multiple
    assert col_gelu_wt(W=BASE + GB + 8) == EALIGN
    assert col_gelu_wt(Z=BASE + GB + 4096) == EALIAS  # Z overlaps W1_i [F, d]
    assert col_gelu_wt(Z=BASE + 64) == EALIAS         # Z overlaps X


def col_gelu_bias(X=BASE, W=BASE + GB, ld=128, b=BASE + 2 * GB, Z=BASE + 3 * GB, M=32, d=64,
                  F=128, wt=False):
    fn = L.tp_mlp_col_gelu_bias_wt if wt else L.tp_mlp_col_gelu_bias
    return fn(X, W, ld, b, Z, M, d, F, None)


def test_col_gelu_bias_validation():
    for wt in (False, True):
        assert col_gelu_bias(M=0, wt=wt) == OK
        assert col_gelu_bias(b=None, wt=wt) == ENULL
        assert col_gelu_bias(W=None, wt=wt) == ENULL
        assert col_gelu_bias(F=12, wt=wt) == ESHAPE
        assert col_gelu_bias(b=BASE + 2 * GB + 8, wt=wt) == EALIGN
        assert col_gelu_bias(Z=BASE + 2 * GB + 128, wt=wt) == EALIAS   # Z overlaps b_i
        assert col_gelu_bias(Z=BASE + 64, wt=wt) == EALIAS             # Z overlaps X
        assert col_gelu_bias(ld=132, wt=wt) == EALIGN
    assert col_gelu_bias(ld=120) == ESHAPE              # math layout: ld < F
    assert col_gelu_bias(ld=56, wt=True) == ESHAPE      # [out, in] layout: ld < d
    assert col_gelu_bias(ld=64, wt=True, M=0) == OK     # ld = d is valid (no launch at M = 0)


def bwd_bias(X=BASE, A=BASE + GB, b1=BASE + 2 * GB, B=BASE + 3 * GB, dY=BASE + 4 * GB,
             dX=BASE + 5 * GB, dA=BASE + 6 * GB, dB=BASE + 7 * GB, db1=BASE + 8 * GB, M=32, d=64,
             H=256, N=2, rank=0, ws=BASE + 9 * GB, wsb=None):
    if wsb is None:
        wsb = L.tp_mlp_shard_backward_bias_workspace_size(M, d, H, N)
    return L.tp_mlp_shard_backward_bias(X, A, b1, B, dY, dX, dA, dB, db1, M, d, H, N, rank, ws,
                                        wsb, None)


def test_backward_bias_validation():
    plain = L.tp_mlp_shard_backward_workspace_size(32, 64, 256, 2)
    assert L.tp_mlp_shard_backward_bias_workspace_size(32, 64, 256, 2) == plain + 512  # 1 block x 128 x 4
    assert bwd_bias(b1=None) == ENULL
    assert bwd_bias(db1=None) == ENULL
    assert bwd_bias(b1=None, M=0) == ENULL
    assert bwd_bias(db1=BASE + 8 * GB + 4) == EALIGN
    assert bwd_bias(db1=BASE + 2 * GB + 64) == EALIAS     # db1_i overlaps b1
    assert bwd_bias(db1=BASE + 9 * GB + 256) == EALIAS    # db1_i inside the workspace
    assert bwd_bias(wsb=L.tp_mlp_shard_backward_workspace_size(32, 64, 256, 2)) == EWS
    assert bwd_bias(rank=2) == EARG
    assert bwd_bias(M=12) == ESHAPE


def bwd8_bias(b1=BASE + 2 * GB, db1=BASE + 8 * GB, M=32, d=64, H=256, N=2, rank=0, wsb=None):
    if wsb is None:
        wsb = L.tp_mlp_shard_backward_fp8_bias_workspace_size(M, d, H, N)
    return L.tp_mlp_shard_backward_fp8_bias(BASE, BASE + GB, b1, BASE + 3 * GB, BASE + 4 * GB,
                                            BASE + 5 * GB, BASE + 6 * GB, BASE + 7 * GB, db1,
                                            M, d, H, N, rank, None, BASE + 9 * GB, wsb, None)


def test_backward_fp8_bias_validation():
    plain = L.tp_mlp_shard_backward_fp8_workspace_size(32, 64, 256, 2)
    assert L.tp_mlp_shard_backward_fp8_bias_workspace_size(32, 64, 256, 2) == plain + 512
    assert bwd8_bias(b1=None) == ENULL
    assert bwd8_bias(db1=None) == ENULL
    assert bwd8_bias(db1=BASE + 8 * GB + 4) == EALIGN
    assert bwd8_bias(db1=BASE + 2 * GB + 64) == EALIAS    # db1_i overlaps b1
    assert bwd8_bias(wsb=L.tp_mlp_shard_backward_fp8_workspace_size(32, 64, 256, 2)) == EWS
    assert bwd8_bias(M=8) == ESHAPE                       # M a multiple of 16 for fp8


def bias_grad(G=BASE, ld=64, rows=300, cols=64, db=BASE + GB, ws=BASE + 2 * GB, wsb=None):
    if wsb is None:
        wsb = L.tp_bias_grad_workspace_size(rows, cols)
    return L.tp_bias_grad_bf16(G, ld, rows, cols, db, ws, wsb, None)


def test_bias_grad_validation():
    assert L.tp_bias_grad_workspace_size(300, 64) == 3 * 64 * 4     # 3 row blocks x 64 columns, fp32
    assert L.tp_bias_grad_workspace_size(0, 64) == 0
    assert L.tp_bias_grad_workspace_size(10, 0) == 0
    assert bias_grad(cols=60, ld=64) == ESHAPE
    assert bias_grad(ld=56) == ESHAPE
    assert bias_grad(ld=72 + 4) == EALIGN
    assert bias_grad(db=None) == ENULL
    assert bias_grad(G=None) == ENULL
    assert bias_grad(wsb=16) == EWS
    assert bias_grad(G=BASE + 8) == EALIGN
    assert bias_grad(db=BASE + 1024) == EALIAS            # db inside G
    assert bias_grad(ws=BASE + 4096) == EALIAS            # workspace inside G
    assert bias_grad(rows=128 * 65536) == ESHAPE          # more row blocks than the grid holds


def row_partial_wt(Z=BASE, W=BASE + GB, ldw=128, Y=BASE + 2 * GB, yd=F32, M=32, F=128, d=64):
    return L.tp_mlp_row_partial_wt(Z, W, ldw, Y, yd, M, F, d, None)


def test_row_partial_wt_validation():
    assert row_partial_wt(M=0) == OK
    assert row_partial_wt(yd=E4M3) == EDTYPE
    assert row_partial_wt(Z=None) == ENULL
    assert row_partial_wt(ldw=120) == ESHAPE          # ldw < F
    assert row_partial_wt(ldw=132) == EALIGN
    assert row_partial_wt(F=12) == ESHAPE
    assert row_partial_wt(Y=BASE + GB + 1024) == EALIAS   # Y overlaps W2_i [d, F], stride ldw


def shard_wt(X=BASE, W1=BASE + GB, W2=BASE + 2 * GB, Y=BASE + 3 * GB, yd=F32, M=32, d=64, H=256,
             N=2, rank=0, ws=BASE + 4 * GB, wsb=None):
    if wsb is None:
        wsb = L.tp_mlp_shard_workspace_size(M, d, H, N)
    return L.tp_mlp_shard_wt(X, W1, W2, Y, yd, M, d, H, N, rank, ws, wsb, None)


def test_shard_wt_validation():
    assert shard_wt(M=0) == OK
    assert shard_wt(rank=2) == EARG
    assert shard_wt(N=3) == ESHAPE
    assert shard_wt(yd=9) == EDTYPE
    assert shard_wt(W2=None) == ENULL
    assert shard_wt(wsb=100) == EWS
    assert shard_wt(W1=BASE + GB + 2) == EALIGN
    assert shard_wt(Y=BASE + 2 * GB + 256) == EALIAS   # Y overlaps W2
    assert shard_wt(ws=BASE + GB + 1024) == EALIAS     # workspace overlaps W1


def psum(parts, N=None, pd=F32, Y=BASE + 10 * GB, yd=F32, numel=4096):
    arr = (ctypes.c_void_p * max(1, len(parts)))(*parts)
    return L.tp_partial_sum(arr, len(parts) if N is None else N, pd, Y, yd, numel, None)


def test_partial_sum_validation():
    parts = [BASE + i * GB for i in range(4)]
    assert psum(parts, numel=0) == OK
    assert psum(parts, N=0) == EARG
    assert psum([BASE + i * GB for i in range(65)]) == EARG
    assert psum(parts, pd=E4M3) == EDTYPE
    assert psum(parts, yd=9) == EDTYPE
    assert psum(parts, numel=-1) == ESHAPE
    assert psum(parts[:1] + [None] + parts[2:]) == ENULL
    assert psum(parts, Y=None) == ENULL
    assert psum(parts, Y=BASE + 10 * GB + 8) == EALIGN
    assert psum([parts[0] + 4] + parts[1:]) == EALIGN
    assert psum(parts, Y=parts[1]) == EALIAS           # only parts[0] may be Y
    assert psum(parts, Y=parts[0] + 16) == EALIAS
    assert psum(parts, Y=parts[0], pd=BF16, yd=F32) == EALIAS  # in place needs equal dtypes


def psum_rows(parts, N=None, pd=F32, M=64, d=128, rb=0, re=32, bias=None, bd=F32,
              Y=BASE + 10 * GB, yd=F32):
    arr = (ctypes.c_void_p * max(1, len(parts)))(*parts)
    return L.tp_partial_sum_rows(arr, len(parts) if N is None else N, pd, M, d, rb, re, bias, bd,
                                 Y, yd, None)


def test_partial_sum_rows_validation():
    parts = [BASE + i * GB for i in range(4)]
    bias = BASE + 20 * GB
    assert psum_rows(parts, rb=5, re=5) == OK          # empty range: no-op
    assert psum_rows(parts, N=0) == EARG
    assert psum_rows(parts, pd=E4M3) == EDTYPE
    assert psum_rows(parts, yd=E4M3) == EDTYPE
    assert psum_rows(parts, bias=bias, bd=E4M3) == EDTYPE
    assert psum_rows(parts, bias=None, bd=E4M3) != EDTYPE   # bias_dtype ignored without a bias
    assert psum_rows(parts, d=100) == ESHAPE            # d not a multiple of 8
    assert psum_rows(parts, rb=-1) == ESHAPE
    assert psum_rows(parts, rb=10, re=9) == ESHAPE
    assert psum_rows(parts, re=65) == ESHAPE            # beyond M
    assert psum_rows(parts[:1] + [None] + parts[2:]) == ENULL
    assert psum_rows(parts, Y=None) == ENULL
    assert psum_rows(parts, bias=bias + 4) == EALIGN
    assert psum_rows(parts, Y=BASE + 10 * GB + 8) == EALIGN
    assert psum_rows(parts, Y=parts[1] + 128 * 4 * 8) == EALIAS   # inside parts[1]
    assert psum_rows(parts, rb=8, re=16, Y=parts[0]) == EALIAS     # not the block's first row
    assert psum_rows(parts, bias=BASE + 10 * GB + 64) == EALIAS    # bias overlaps Y


def rs_share(parts, N=None, pd=F32, M=64, d=128, rank=1, bias=None, bd=F32, Y=BASE + 10 * GB,
             yd=F32):
    N = len(parts) if N is None else N
    arr = (ctypes.c_void_p * max(1, len(parts)))(*parts)
    return L.tp_reduce_scatter_share(arr, N, pd, M, d, rank, bias, bd, Y, yd, None)


def test_reduce_scatter_share_validation():
    parts = [BASE + i * GB for i in range(4)]
    assert rs_share(parts, M=0) == OK                   # empty share: no-op
    assert rs_share(parts, rank=4) == EARG
    assert rs_share(parts, rank=-1) == EARG
    assert rs_share(parts, N=0) == EARG
    assert rs_share(parts, M=66) == ESHAPE              # 66 rows do not split over 4 ranks
    assert rs_share(parts, d=100) == ESHAPE
    assert rs_share(parts, pd=E4M3) == EDTYPE
    assert rs_share(parts, Y=None) == ENULL
    assert rs_share(parts, Y=BASE + 10 * GB + 8) == EALIGN
    # rank 1's rows [16, 32) of parts[0] in place are allowed; rows of rank 0 are not
    assert rs_share(parts, rank=0, Y=parts[0] + 16 * 128 * 4) == EALIAS


def noalloc(X=BASE, A=BASE + GB, B=BASE + 2 * GB, Y=BASE + 3 * GB, yd=F32, M=32, d=64, H=256,
            N=2, rank=1):
    return L.tp_mlp_shard_noalloc(X, A, B, Y, yd, M, d, H, N, rank, None)


def test_noalloc_validation():
    # every error below is found on the host before the device is touched
    assert noalloc(M=0) == OK
    assert noalloc(N=0) == EARG
    assert noalloc(rank=2) == EARG
    assert noalloc(N=3) == ESHAPE
    assert noalloc(yd=E4M3) == EDTYPE
    assert noalloc(X=None) == ENULL
    assert noalloc(Y=None) == ENULL
    # Z_i [M, F] bf16 must fit the 64 MiB scratch: 32768 x 1024 x 2 B = 64 MiB fits,
    # one more row does not
    assert tpm.NOALLOC_SCRATCH_BYTES == 64 << 20
    big = dict(d=256, H=2048, N=2)
    assert L.tp_mlp_shard_workspace_size(32768, 256, 2048, 2) == 64 << 20
    assert noalloc(M=32769, **big) == ESCRATCH
    assert noalloc(M=1 << 20, d=4096, H=16384, N=8) == ESCRATCH
    assert "static scratch" in tpm.status_string(ESCRATCH)


def test_clock_stamp_validation():
    assert L.tp_clock_stamp_count(8192, 4096) == 4 * 64 * 32
    assert L.tp_clock_stamp_count(1, 1) == 4
    assert L.tp_clock_stamp_count(-1, 4) == 0
    st = BASE + 9 * GB
    n = L.tp_clock_stamp_count(32, 256)
    cg = lambda stamps=st, count=n, **kw: L.tp_mlp_col_gelu_stamped(
        BASE, BASE + GB, 256, BASE + 2 * GB, 32, 64, 256, stamps, count, None)
    assert cg(stamps=None) == ENULL
    assert cg(count=n - 1) == EWS
    assert cg(stamps=st + 8) == EALIGN
    rp = lambda stamps=st, count=L.tp_clock_stamp_count(32, 64): L.tp_mlp_row_partial_stamped(
        BASE, BASE + GB, BASE + 2 * GB, E4M3, 32, 128, 64, stamps, count, None)
    assert rp() == EDTYPE                                 # the row step's own checks still apply
    assert rp(count=3) == EWS
    fp = lambda count=L.tp_clock_stamp_count(32, 64): L.tp_mlp_row_partial_e4m3_stamped(
        BASE, BASE + 3 * GB, BASE + GB, BASE + 4 * GB, BASE + 2 * GB, 32, 128, 60, st, count, None)
    assert fp() == ESHAPE                                 # d = 60 not a multiple of 16
    assert fp(count=0) == EWS


def test_fp8_validation():
    sc = BASE + 20 * GB
    assert L.tp_quant_e4m3(BASE, 100, sc, BASE + GB, sc + 64, None) == ESHAPE   # not /16
    assert L.tp_quant_e4m3(BASE, 4096, None, BASE + GB, sc, None) == ENULL
    assert L.tp_quant_e4m3(BASE, 4096, sc, BASE + 16, sc + 64, None) == EALIAS
    assert L.tp_quant_e4m3(BASE, 4096, sc, BASE + GB, sc, None) == EALIAS      # scale == amax
    assert L.tp_amax_bf16(BASE, -1, sc, None) == ESHAPE
    assert L.tp_amax_bf16(BASE, 64, None, None) == ENULL
    assert L.tp_amax_bf16(BASE, 64, BASE + 16, None) == EALIAS
    args = dict(Xq=BASE, sX=sc, Aq=BASE + GB, lda=256, sA=sc + 4, Z=BASE + 2 * GB, za=sc + 8,
                M=32, d=64, F=256)

    def cg(**kw):
        a = dict(args, **kw)
        return L.tp_mlp_col_gelu_e4m3(a["Xq"], a["sX"], a["Aq"], a["lda"], a["sA"], a["Z"],
                                      a["za"], a["M"], a["d"], a["F"], None)
    assert cg(d=40) == ESHAPE                         # e4m3 widths must be multiples of 16
    assert cg(sX=None) == ENULL
    assert cg(lda=264) == EALIGN
    assert cg(Z=BASE + 32) == EALIAS
    assert L.tp_mlp_row_partial_e4m3(BASE, sc, BASE + GB, sc, BASE + 2 * GB, 32, 24, 64, None) == ESHAPE
    ws = L.tp_mlp_shard_e4m3_workspace_size(32, 64, 256, 2)
    assert ws >= 32 * 128 * 3
    assert L.tp_mlp_shard_e4m3(BASE, sc, BASE + GB, sc, BASE + 2 * GB, sc, BASE + 3 * GB,
                               32, 64, 256, 2, 2, BASE + 4 * GB, ws, None) == EARG
    assert L.tp_mlp_shard_e4m3(BASE, sc, BASE + GB, sc, BASE + 2 * GB, sc, BASE + 3 * GB,
                               32, 64, 256, 2, 0, BASE + 4 * GB, ws - 1, None) == EWS
    assert L.tp_mlp_shard_e4m3(BASE, sc, BASE + GB, sc, BASE + 2 * GB, sc, BASE + 3 * GB,
                               32, 64, 256, 2, 0, BASE + 3 * GB, ws, None) == EALIAS


def test_fp8_delayed_validation():
    sc = BASE + 20 * GB
    hist, cnt, am, ns = BASE + 21 * GB, BASE + 22 * GB, BASE + 23 * GB, BASE + 24 * GB
    assert L.tp_amax_history_push(hist, cnt, 0, am, ns, None) == EARG
    assert L.tp_amax_history_push(hist, cnt, 65537, am, ns, None) == EARG
    assert L.tp_amax_history_push(None, cnt, 16, am, ns, None) == ENULL
    assert L.tp_amax_history_push(hist, cnt, 16, am, None, None) == ENULL
    assert L.tp_amax_history_push(hist + 2, cnt, 16, am, ns, None) == EALIGN
    assert L.tp_amax_history_push(hist, hist + 32, 16, am, ns, None) == EALIAS   # count inside the ring
    assert L.tp_amax_history_push(hist, cnt, 16, am, am, None) == EALIAS
    args = dict(Xq=BASE, sX=sc, Aq=BASE + GB, lda=256, sA=sc + 4, sZ=sc + 8, Zq=BASE + 2 * GB,
                za=sc + 12, M=32, d=64, F=256)

    def cg(**kw):
        a = dict(args, **kw)
        return L.tp_mlp_col_gelu_e4m3_delayed(a["Xq"], a["sX"], a["Aq"], a["lda"], a["sA"], a["sZ"],
                                              a["Zq"], a["za"], a["M"], a["d"], a["F"], None)
    assert cg(za=None) == ENULL                      # the step's amax is always recorded
    assert cg(sZ=None) == ENULL
    assert cg(d=40) == ESHAPE
    assert cg(lda=200) == ESHAPE
    assert cg(Zq=BASE + 16) == EALIAS                # Zq overlaps Xq
    assert cg(za=sc + 8) == EALIAS                   # amax is the scale
    ws = L.tp_mlp_shard_e4m3_delayed_workspace_size(32, 64, 256, 2)
    assert ws >= 32 * 128
    assert L.tp_mlp_shard_e4m3_delayed_workspace_size(32, 64, 256, 3) == 0

    def sh(rank=0, wsb=ws, wsp=BASE + 4 * GB, za=sc + 12, Y=BASE + 3 * GB):
        return L.tp_mlp_shard_e4m3_delayed(BASE, sc, BASE + GB, sc, BASE + 2 * GB, sc, sc + 8, Y, za,
                                           32, 64, 256, 2, rank, wsp, wsb, None)
    assert sh(rank=2) == EARG
    assert sh(wsb=ws - 1) == EWS
    assert sh(za=None) == ENULL
    assert sh(wsp=BASE + 3 * GB) == EALIAS          # workspace is Y
    assert sh(Y=BASE + 4 * GB) == EALIAS


def test_backward_validation():
    M, d, H, N = 32, 64, 256, 2
    F = H // N
    ws = L.tp_mlp_shard_backward_workspace_size(M, d, H, N)
    assert ws == 4 * M * F + 2 * (2 * M * F)          # S fp32, dS and Z bf16 (256-multiples here)
    assert L.tp_mlp_shard_backward_workspace_size(M, d, H, 3) == 0
    assert L.tp_mlp_shard_backward_workspace_size(M, d, 0, 1) == 0
    a = dict(X=BASE, A=BASE + GB, B=BASE + 2 * GB, dY=BASE + 3 * GB, dX=BASE + 4 * GB,
             dA=BASE + 5 * GB, dB=BASE + 6 * GB, M=M, d=d, H=H, N=N, rank=1, ws=BASE + 7 * GB,
             wsb=ws)

    def bw(**kw):
        b = dict(a, **kw)
        return L.tp_mlp_shard_backward(b["X"], b["A"], b["B"], b["dY"], b["dX"], b["dA"], b["dB"],
                                       b["M"], b["d"], b["H"], b["N"], b["rank"], b["ws"],
                                       b["wsb"], None)
    assert bw(M=0) == OK
    assert bw(rank=2) == EARG
    assert bw(N=0) == EARG
    assert bw(N=3) == ESHAPE                  # H not divisible by N
    assert bw(M=36) == ESHAPE                 # M is a contraction length: multiple of 8
    assert bw(d=60) == ESHAPE
    assert bw(N=64) == ESHAPE                 # F = 4
    assert bw(dY=None) == ENULL
    assert bw(dB=None) == ENULL
    assert bw(ws=None) == EWS
    assert bw(wsb=ws - 1) == EWS
    assert bw(dA=BASE + 5 * GB + 8) == EALIGN
    assert bw(dX=BASE + 3 * GB + 64) == EALIAS     # dX_i overlaps dY
    assert bw(dA=BASE + 4 * GB + 64) == EALIAS     # dA_i overlaps dX_i
    assert bw(ws=BASE + 6 * GB) == EALIAS          # workspace is dB_i
    assert bw(dB=BASE + GB + 1024) == EALIAS       # dB_i inside A


def test_backward_fp8_validation():
    M, d, H, N = 32, 64, 256, 2
    ws = L.tp_mlp_shard_backward_fp8_workspace_size(M, d, H, N)
    assert ws > 0 and L.tp_mlp_shard_backward_fp8_workspace_size(M, d, H, 3) == 0

    def bw(**kw):
        a = dict(X=BASE, A=BASE + GB, B=BASE + 2 * GB, dY=BASE + 3 * GB, dX=BASE + 4 * GB,
                 dA=BASE + 5 * GB, dB=BASE + 6 * GB, M=M, d=d, H=H, N=N, rank=0,
                 wam=None, ws=BASE + 7 * GB, wsb=ws)
        a.update(kw)
        return L.tp_mlp_shard_backward_fp8(a["X"], a["A"], a["B"], a["dY"], a["dX"], a["dA"],
                                           a["dB"], a["M"], a["d"], a["H"], a["N"], a["rank"],
                                           a["wam"], a["ws"], a["wsb"], None)
    assert bw(M=0) == OK
    assert bw(rank=2) == EARG
    assert bw(M=24) == ESHAPE             # fp8 rows of the transposed copies: multiple of 16
    assert bw(d=72) == ESHAPE
    assert bw(N=32) == ESHAPE             # F = 8
    assert bw(dX=None) == ENULL
    assert bw(wsb=ws - 1) == EWS
    assert bw(dB=BASE + 2 * GB + 32) == EALIAS
    assert bw(ws=BASE + 4 * GB) == EALIAS
    assert bw(wam=BASE + 8 * GB + 2) == EALIGN      # the weight amaxes are floats
    assert bw(wam=BASE + 7 * GB + 32) == EALIAS     # inside the workspace the call writes
    assert bw(wam=BASE + 4 * GB) == EALIAS          # dX_i


def test_attention_validation():
    # tp_attn_heads
    def heads(QKV=BASE, ld=3 * 256, O=BASE + GB, ldo=256, B=2, S=40, h=2, causal=1):
        return L.tp_attn_heads(QKV, ld, O, ldo, B, S, h, causal, None)
    assert heads(B=0) == OK
    assert heads(S=0) == OK
    assert heads(h=0) == ESHAPE
    assert heads(ld=3 * 256 - 8) == ESHAPE           # too narrow for 2 heads' Q, K, V
    assert heads(ldo=128) == ESHAPE
    assert heads(ld=3 * 256 + 4) == EALIGN
    assert heads(QKV=None) == ENULL
    assert heads(O=BASE + 8) == EALIGN
    assert heads(O=BASE + 1024) == EALIAS             # O inside QKV
    assert heads(S=1 << 20, ld=3 << 12) == ESHAPE     # 32-bit per-sequence offsets
    # tp_attn_qkv
    assert L.tp_attn_qkv(BASE, BASE + GB, 1000, BASE + 2 * GB, 80, 1024, 1536, None) == ESHAPE
    assert L.tp_attn_qkv(BASE, BASE + GB, 1536, BASE + 16, 80, 1024, 1536, None) == EALIAS
    # tp_attn_shard
    ws = L.tp_attn_shard_workspace_size(80, 1024, 2)
    assert ws == 80 * 512 * 6 + 80 * 512 * 2
    assert L.tp_attn_shard_workspace_size(80, 1024, 3) == 0

    def sh(yd=F32, B=2, S=40, d=1024, h=8, N=2, rank=1, wsp=BASE + 4 * GB, wsb=ws, Y=BASE + 3 * GB):
        return L.tp_attn_shard(BASE, BASE + GB, BASE + 2 * GB, Y, yd, B, S, d, h, N, rank, 1,
                               wsp, wsb, None)
    assert sh(B=0) == OK
    assert sh(yd=E4M3) == EDTYPE
    assert sh(rank=2) == EARG
    assert sh(h=16) == ESHAPE                         # head width 64
    assert sh(h=8, N=16, rank=0) == ESHAPE            # N does not divide the heads
    assert sh(wsp=None) == EWS
    assert sh(wsb=ws - 1) == EWS
    assert sh(Y=BASE + GB + 64) == EALIAS             # Y inside W_qkv
    assert sh(wsp=BASE + 3 * GB) == EALIAS            # workspace is Y


def test_python_wrapper_rejects_cpu_tensors():
    import torch
    X = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tpm.tp_mlp_col_gelu(X, torch.zeros(8, 8, dtype=torch.bfloat16))


def test_backward_wrappers_refuse_a_bias_gradient_without_a_bias():
    # db1_i with no b1 would never be written: refused before any tensor check
    import torch
    t = torch.zeros(4, 8, dtype=torch.bfloat16)
    db = torch.zeros(8, dtype=torch.float32)
    for fn in (tpm.tp_mlp_shard_backward, tpm.tp_mlp_shard_backward_fp8):
        with pytest.raises(ValueError, match="db1_i is given without b1"):
            fn(t, t, t, t, 1, 0, db1_i=db)


def test_import_fails_loudly_without_the_library(tmp_path):
    """The package has no CPU fallback: with libtpmlp.so absent, importing it
    raises instead of silently computing elsewhere."""
    import shutil
    import subprocess
    import sys
    pkg = os.path.join(ROOT, "megatron_tensor_transformer_shard_amd")
    dst = tmp_path / "megatron_tensor_transformer_shard_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns("*.so", "_build", "__pycache__"))
    r = subprocess.run([sys.executable, "-c", "import megatron_tensor_transformer_shard_amd"],
                       cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "libtpmlp.so" in (r.stderr + r.stdout)
