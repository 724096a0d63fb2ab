"""The tensor-parallel MLP shard, step by step, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Inputs are bfloat16 bit arrays (uint16) or e4m3 code arrays (uint8) plus
float32 scales; outputs are float64 arrays, except Z, which is returned as
bfloat16 bits because the path stores it in bfloat16.

Notation (as on the pages): X [M, d]; A [d, 4d]; B [4d, d]; N ranks;
F = 4d/N; A_i = A[:, i·F:(i+1)·F]; B_i = B[i·F:(i+1)·F, :];
Z_i = GeLU(X·A_i) [M, F]; Y_i = Z_i·B_i [M, d]; Y = Σ_i Y_i.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erfc

from .codecs import (bf16_decode, bf16_encode, e4m3_decode, e4m3_encode, e5m2_decode,
                     e5m2_encode, E4M3_MAX, E5M2_MAX)

_INV_SQRT2 = 0.7071067811865476  # 1/√2 rounded to float64


def shard_columns(H: int, N: int, rank: int) -> tuple[int, int]:
    """Column range [lo, hi) of A (and row range of B) held by `rank`.

    The first weight is split by columns and the second by rows into N equal
    contiguous blocks ("Megatron architecture and 6D parallel guide", §3.1:
    at TP=2, GPU 0 holds A[:, :2d] and B[:2d, :], GPU 1 the rest).  A width
    that N does not divide is an error here rather than a silent truncation.
    """
    if N < 1 or not (0 <= rank < N):
        raise ValueError(f"rank {rank} not in [0, {N})")
    if H % N:
        raise ValueError(f"width {H} not divisible by N={N}")
    F = H // N
    return rank * F, (rank + 1) * F


def gelu(s: np.ndarray) -> np.ndarray:
    """GeLU(s) = s·Φ(s), Φ the standard normal CDF, Φ(s) = ½·erfc(−s/√2).

    The pages apply GeLU elementwise between the two GEMMs but never define
    it; this is the exact (Gaussian-CDF) form.  erfc keeps Φ accurate in the
    far negative tail, where 1 + erf(s/√2) would cancel.
    """
    s = np.asarray(s, dtype=np.float64)
    return s * (0.5 * erfc(-s * _INV_SQRT2))


def col_gelu(X_bits: np.ndarray, A_i_bits: np.ndarray) -> np.ndarray:
    """Column-parallel step: Z_i = bf16(GeLU(X·A_i)), as bfloat16 bits.

    "Megatron-LM deep architecture", column-parallel linear: each rank takes
    the same X and its own column block of the first weight, and applies
    GeLU to its own columns with no exchange.
    """
    S = bf16_decode(X_bits) @ bf16_decode(A_i_bits)
    return bf16_encode(gelu(S))


def col_gelu_bias(X_bits: np.ndarray, A_i_bits: np.ndarray, b_i_bits: np.ndarray) -> np.ndarray:
    """Column-parallel step with the layer's bias: Z_i = bf16(GeLU(X·A_i + b_i)).

    "Megatron-LM deep architecture", code pattern: the column-parallel
    linear holds a bias of its own output width (the rank's block of the
    first bias) and adds it inside the linear, so before the activation that
    the column/row-parallel section applies to the layer's output.  b_i is
    bf16 bits of length F; the sum is taken in float64.
    """
    S = bf16_decode(X_bits) @ bf16_decode(A_i_bits)
    return bf16_encode(gelu(S + bf16_decode(b_i_bits)[None, :]))


def row_partial(Z_bits: np.ndarray, B_i_bits: np.ndarray) -> np.ndarray:
    """Row-parallel step: the partial output Y_i = Z_i·B_i (float64).

    "Megatron-LM deep architecture", row-parallel linear: each rank multiplies
    its local activation by its row block of the second weight.
    """
    return bf16_decode(Z_bits) @ bf16_decode(B_i_bits)


def mlp_shard(X_bits, A_bits, B_bits, N: int, rank: int, return_z: bool = False):
    """Rank `rank`'s partial output Y_i = GeLU(X·A_i)·B_i of an N-way split.

    A is [d, H] and B is [H, d]; the rank's blocks are taken by
    `shard_columns` ("Megatron architecture and 6D parallel guide", §3.1
    forward pass: Y_i = GeLU(X·A_i)·B_i on each GPU).
    """
    H = A_bits.shape[1]
    if B_bits.shape[0] != H or X_bits.shape[1] != A_bits.shape[0] or B_bits.shape[1] != A_bits.shape[0]:
        raise ValueError("shape mismatch")
    lo, hi = shard_columns(H, N, rank)
    Z = col_gelu(X_bits, A_bits[:, lo:hi])
    Y = row_partial(Z, B_bits[lo:hi, :])
    return (Y, Z) if return_z else Y


def partial_sum(parts) -> np.ndarray:
    """Y = Σ_i Y_i, added in rank order 0..N−1 (float64).

    This is the arithmetic of the AllReduce(sum) that ends the block
    ("Megatron-LM deep architecture", eq. for Output).
    """
    parts = list(parts)
    if not parts:
        raise ValueError("no partials")
    acc = np.array(parts[0], dtype=np.float64, copy=True)
    for p in parts[1:]:
        acc += np.asarray(p, dtype=np.float64)
    return acc


def sp_rows(M: int, N: int, rank: int) -> tuple[int, int]:
    """Row range [lo, hi) of the block output that `rank` keeps under
    sequence parallelism.

    "Megatron-LM deep architecture", sequence-parallel section: an
    AllReduce is an AllGather of a ReduceScatter, and after the MLP the
    ReduceScatter leaves each GPU the summed output for its own 1/N slice of
    the sequence.  With tokens stored sequence-major ([S, B, H], rows in
    sequence order) that slice is the contiguous row block
    [rank·M/N, (rank+1)·M/N).  A row count that N does not divide is an
    error.
    """
    if N < 1 or not (0 <= rank < N):
        raise ValueError(f"rank {rank} not in [0, {N})")
    if M % N:
        raise ValueError(f"{M} rows not divisible by N={N}")
    R = M // N
    return rank * R, (rank + 1) * R


def partial_sum_rows(parts, lo: int, hi: int, bias=None) -> np.ndarray:
    """Rows [lo, hi) of Σ_i Y_i (rank order, float64), plus `bias` once.

    The bias of the row-parallel linear is added after the reduction, once
    ("Megatron-LM deep architecture", code pattern of the row-parallel
    linear: all-reduce the local output, then add the bias).  `bias` is a
    float64 vector of the output width, or None.
    """
    parts = [np.asarray(p, dtype=np.float64) for p in parts]
    if not parts:
        raise ValueError("no partials")
    M = parts[0].shape[0]
    if not (0 <= lo <= hi <= M):
        raise ValueError(f"row range [{lo}, {hi}) outside [0, {M})")
    acc = partial_sum([p[lo:hi] for p in parts])
    if bias is not None:
        acc = acc + np.asarray(bias, dtype=np.float64)[None, :]
    return acc


def reduce_scatter_share(parts, rank: int, bias=None) -> np.ndarray:
    """Rank `rank`'s share of the ReduceScatter that replaces the AllReduce
    under sequence parallelism: its row block of Σ_i Y_i, plus the bias."""
    parts = list(parts)
    lo, hi = sp_rows(np.asarray(parts[0]).shape[0], len(parts), rank)
    return partial_sum_rows(parts, lo, hi, bias)


def mlp_unsharded(X_bits, A_bits, B_bits) -> np.ndarray:
    """The unsharded block Y = bf16(GeLU(X·A))·B (Z rounded as in a shard)."""
    return row_partial(col_gelu(X_bits, A_bits), B_bits)


def mlp_shard_bias(X_bits, A_bits, b1_bits, B_bits, N: int, rank: int) -> np.ndarray:
    """Rank `rank`'s partial output with the first layer's bias:
    Y_i = bf16(GeLU(X·A_i + b1_i))·B_i, b1_i the rank's block of b1 (the
    column-parallel layer's bias shard).  The second layer's bias is not in
    any partial: it is added once after the sum (`partial_sum_rows`)."""
    H = A_bits.shape[1]
    if b1_bits.shape != (H,):
        raise ValueError("b1 must have the hidden width")
    lo, hi = shard_columns(H, N, rank)
    return row_partial(col_gelu_bias(X_bits, A_bits[:, lo:hi], b1_bits[lo:hi]), B_bits[lo:hi, :])


def mlp_unsharded_bias(X_bits, A_bits, b1_bits, B_bits, b2_bits) -> np.ndarray:
    """The unsharded block with both biases: bf16(GeLU(X·A + b1))·B + b2."""
    return (row_partial(col_gelu_bias(X_bits, A_bits, b1_bits), B_bits)
            + bf16_decode(b2_bits)[None, :])


# ----------------------------------------------------------------------------
# fp8 e4m3 variant ("Megatron-LM deep architecture", FP8 hybrid precision):
# every tensor is multiplied by a scale S derived from its amax before it is
# cast to E4M3; the GEMM result is divided by the product of the two scales.
# Current scaling is used: each tensor's own amax.
# ----------------------------------------------------------------------------

def amax(T_bits: np.ndarray) -> float:
    """max |T| of a bfloat16 tensor (exact)."""
    if T_bits.size == 0:
        return 0.0
    return float(np.max(np.abs(bf16_decode(T_bits))))


def quant_scale(a: float) -> np.float32:
    """Per-tensor quantisation scale s = 448/amax, an fp32 division (1 if amax = 0)."""
    if a == 0.0:
        return np.float32(1.0)
    return np.float32(np.float32(E4M3_MAX) / np.float32(a))


def quant_e4m3(T_bits: np.ndarray, s: np.float32) -> np.ndarray:
    """e4m3 codes of T·s: the product is taken in fp32 (RNE), clamped to ±448,
    then rounded once to e4m3 (RNE)."""
    t32 = bf16_decode(T_bits).astype(np.float32)
    v = (t32 * np.float32(s)).astype(np.float32)
    v = np.clip(v, -E4M3_MAX, E4M3_MAX)
    return e4m3_encode(v.astype(np.float64))


def quantize_inputs_e4m3(T_bits: np.ndarray):
    """(codes, s) of a bfloat16 tensor under its own amax scale."""
    s = quant_scale(amax(T_bits))
    return quant_e4m3(T_bits, s), s


def col_gelu_e4m3(Xq, sX, Aq_i, sA) -> np.ndarray:
    """Z_i = bf16(GeLU((Xq·Aq_i)/(sX·sA))) as bfloat16 bits."""
    S = (e4m3_decode(Xq) @ e4m3_decode(Aq_i)) / (float(sX) * float(sA))
    return bf16_encode(gelu(S))


def requant_z(Z_bits: np.ndarray):
    """Z_q = e4m3(Z·s_Z) with s_Z = 448/amax(Z); returns (codes, s_Z)."""
    return quantize_inputs_e4m3(Z_bits)


def row_partial_e4m3(Zq, sZ, Bq_i, sB) -> np.ndarray:
    """Y_i = (Zq·Bq_i)/(sZ·sB) in float64 (the GPU stores it as bfloat16)."""
    return (e4m3_decode(Zq) @ e4m3_decode(Bq_i)) / (float(sZ) * float(sB))


def mlp_shard_e4m3(Xq, sX, Aq, sA, Bq, sB, N: int = 1, rank: int = 0, return_all=False):
    """fp8 partial output of rank `rank` from quantised X, A, B (codes + scales)."""
    H = Aq.shape[1]
    lo, hi = shard_columns(H, N, rank)
    Z = col_gelu_e4m3(Xq, sX, Aq[:, lo:hi], sA)
    Zq, sZ = requant_z(Z)
    Y = row_partial_e4m3(Zq, sZ, Bq[lo:hi, :], sB)
    if return_all:
        return Y, Z, Zq, sZ
    return Y


# ----------------------------------------------------------------------------
# fp8 delayed scaling ("Megatron-LM deep architecture", FP8 hybrid precision
# and delayed scaling): the scale a step applies is not taken from the
# tensor's own amax but predicted from the moving average of the amaxes
# recorded in earlier steps, so no amax has to be known before the tensor is
# quantised.  Here it is applied to Z, the one tensor quantised inside the
# path: Z is quantised in the column-parallel GEMM's epilogue with the
# predicted scale, and its amax is recorded for later steps.
# ----------------------------------------------------------------------------

def delayed_scale(history) -> np.float32:
    """Scale from an amax history: s = 448 / mean(history), the mean taken
    over the recorded values (float64), rounded to fp32, and the division done
    in fp32 (1 if the history is empty or its mean is 0)."""
    h = np.asarray(history, dtype=np.float64)
    if h.size == 0:
        return np.float32(1.0)
    mean = np.float32(np.mean(h))
    if mean == 0.0:
        return np.float32(1.0)
    return np.float32(np.float32(E4M3_MAX) / mean)


def amax_history_push(history, amax_value, L: int):
    """Record one step's amax in a window of the last L steps; returns the new
    window (oldest first) and the scale the next step applies."""
    if L < 1:
        raise ValueError("window length must be >= 1")
    h = list(history)[-(L - 1):] if L > 1 else []
    h.append(float(np.float32(amax_value)))
    return h, delayed_scale(h)


def col_gelu_e4m3_delayed(Xq, sX, Aq_i, sA, sZ):
    """Z_q = e4m3(bf16(GeLU((Xq·Aq_i)/(sX·sA)))·sZ) with a given (predicted)
    scale sZ, and amax(Z) of this step.  Z is rounded to bf16 first, exactly
    as in the current-scaling path, so the two agree whenever sZ is the same."""
    Z = col_gelu_e4m3(Xq, sX, Aq_i, sA)
    return quant_e4m3(Z, np.float32(sZ)), amax(Z)


def mlp_shard_e4m3_delayed(Xq, sX, Aq, sA, Bq, sB, sZ, N: int = 1, rank: int = 0):
    """fp8 partial output of rank `rank` with Z quantised by the predicted
    scale sZ; returns (Y_i, Z_q, amax(Z))."""
    H = Aq.shape[1]
    lo, hi = shard_columns(H, N, rank)
    Zq, za = col_gelu_e4m3_delayed(Xq, sX, Aq[:, lo:hi], sA, sZ)
    Y = row_partial_e4m3(Zq, sZ, Bq[lo:hi, :], sB)
    return Y, Zq, za


# ----------------------------------------------------------------------------
# Backward of one rank's shard.  The pages give only its communication: two
# AllReduces in the backward pass ("Megatron-LM" glossary and "Megatron
# architecture and 6D parallel guide", tensor-parallel communication): the
# backward of the row-parallel sum hands every rank the same dY, and the
# backward of the column-parallel (replicated) input sums the ranks' dX_i.
# The formulas are the chain rule through the forward as computed: S_i = X·A_i,
# Z_i = bf16(GeLU(S_i)), Y_i = Z_i·B_i.  S is recomputed (activation
# recomputation); dS is rounded to bf16 once, because the next GEMMs take bf16
# operands; dZ is never stored.
# ----------------------------------------------------------------------------

_INV_SQRT_2PI = 0.3989422804014327  # 1/√(2π)


def gelu_grad(s: np.ndarray) -> np.ndarray:
    """GeLU'(s) = Φ(s) + s·φ(s), φ(s) = e^(−s²/2)/√(2π), the derivative of s·Φ(s)."""
    s = np.asarray(s, dtype=np.float64)
    return 0.5 * erfc(-s * _INV_SQRT2) + s * _INV_SQRT_2PI * np.exp(-0.5 * s * s)


def mlp_shard_backward(X_bits, A_bits, B_bits, dY_bits, N: int, rank: int, rounding: bool = True,
                       b1_bits=None):
    """Gradients of rank `rank`'s shard, given the block's output gradient dY.

    Returns a dict of float64 arrays (dS and Z as bf16 bits when `rounding`):
      S  = X·A_i                       [M, F]  (recomputed)
      Z  = bf16(GeLU(S))               [M, F]  (the forward's stored Z)
      dZ = dY·B_iᵀ                     [M, F]
      dS = bf16(dZ ⊙ GeLU'(S))         [M, F]
      dX = dS·A_iᵀ                     [M, d]  (this rank's part of the input gradient)
      dA = Xᵀ·dS                       [d, F]  (the gradient of A_i, a column block of A's)
      dB = Zᵀ·dY                       [F, d]  (the gradient of B_i, a row block of B's)
    With rounding=False, Z and dS stay in float64 (the exact chain rule of the
    unrounded forward, for checking the formulas against finite differences).

    With b1_bits (bf16 [H], the column-parallel layer's bias, added before
    GeLU as in the pages' code pattern) S = X·A_i + b1_i, and the dict also
    holds the bias gradients: db1 = Σ_m dS[m, :] ([F], this rank's block of
    b1's gradient) and db2 = Σ_m dY[m, :] ([d], the gradient of the row
    layer's bias, added once after the sum, so the same on every rank).
    """
    H = A_bits.shape[1]
    lo, hi = shard_columns(H, N, rank)
    X = bf16_decode(X_bits)
    A_i = bf16_decode(A_bits)[:, lo:hi]
    B_i = bf16_decode(B_bits)[lo:hi, :]
    dY = bf16_decode(dY_bits)
    S = X @ A_i
    if b1_bits is not None:
        if np.shape(b1_bits) != (H,):
            raise ValueError("b1 must have the hidden width")
        S = S + bf16_decode(b1_bits)[lo:hi][None, :]
    G = gelu(S)
    dZ = dY @ B_i.T
    dS = dZ * gelu_grad(S)
    if rounding:
        Z_bits, dS_bits = bf16_encode(G), bf16_encode(dS)
        Z, dSv = bf16_decode(Z_bits), bf16_decode(dS_bits)
    else:
        Z_bits = dS_bits = None
        Z, dSv = G, dS
    g = {"S": S, "Z": Z, "Z_bits": Z_bits, "dZ": dZ, "dS": dSv, "dS_bits": dS_bits,
         "dX": dSv @ A_i.T, "dA": X.T @ dSv, "dB": Z.T @ dY}
    if b1_bits is not None:
        g["db1"] = dSv.sum(axis=0)
        g["db2"] = dY.sum(axis=0)
    return g


# ----------------------------------------------------------------------------
# fp8 backward, hybrid formats ("Megatron-LM deep architecture", FP8 hybrid
# precision section: E4M3 for the forward's activations and weights, E5M2,
# with its wider range, for the gradients of the backward pass).  Every
# tensor is quantised with its own current amax scale (448/amax for e4m3,
# 57344/amax for e5m2, fp32 divisions): X, A and B over the whole tensor as
# in the fp8 forward, dY, and the two tensors the backward produces on the
# way, dS (e5m2) and Z (e4m3, the bf16 Z of the recomputed forward).  Each
# GEMM of two quantised operands is divided by the product of their scales.
# ----------------------------------------------------------------------------

def quant_scale_e5m2(a: float) -> np.float32:
    """Per-tensor scale s = 57344/amax, an fp32 division (1 if amax = 0)."""
    if a == 0.0:
        return np.float32(1.0)
    return np.float32(np.float32(E5M2_MAX) / np.float32(a))


def quant_e5m2(T_bits: np.ndarray, s: np.float32) -> np.ndarray:
    """e5m2 codes of T·s: the product in fp32 (RNE), clamped to ±57344, then
    rounded once to e5m2 (RNE)."""
    t32 = bf16_decode(T_bits).astype(np.float32)
    v = (t32 * np.float32(s)).astype(np.float32)
    v = np.clip(v, -E5M2_MAX, E5M2_MAX)
    return e5m2_encode(v.astype(np.float64))


def quantize_e5m2(T_bits: np.ndarray):
    """(codes, s) of a bfloat16 tensor under its own amax scale, in e5m2."""
    s = quant_scale_e5m2(amax(T_bits))
    return quant_e5m2(T_bits, s), s


def mlp_shard_backward_fp8(X_bits, A_bits, B_bits, dY_bits, N: int, rank: int, b1_bits=None):
    """Gradients of rank `rank`'s shard with fp8 GEMMs in the hybrid formats.

    Returns a dict: the scales sX, sA, sB, sdY, sdS, sZ (float32), the codes
    Xq, Aq_i, Bq_i, dYq (e4m3 / e5m2), S and dZ (float64), dS and Z (bf16
    bits), dSq (e5m2), Zq (e4m3), and the gradients dX, dA, dB (float64):
      S  = (Xq·Aq_i)/(sX·sA)               the recomputed pre-activation
      dZ = (dYq·Bq_iᵀ)/(sdY·sB)
      dS = bf16(dZ ⊙ GeLU'(S)),  Z = bf16(GeLU(S))
      dX = (dSq·Aq_iᵀ)/(sdS·sA),  dA = (Xqᵀ·dSq)/(sX·sdS),  dB = (Zqᵀ·dYq)/(sZ·sdY)
    With b1_bits (bf16 [H], the column layer's bias, not quantised) the rank's
    block is added to the dequantised S, and db1 = Σ_m dS (the bf16 dS, before
    its e5m2 quantisation) and db2 = Σ_m dY (bf16 dY) are returned as well.
    """
    H = A_bits.shape[1]
    lo, hi = shard_columns(H, N, rank)
    Xq, sX = quantize_inputs_e4m3(X_bits)
    Aq, sA = quantize_inputs_e4m3(A_bits)
    Bq, sB = quantize_inputs_e4m3(B_bits)
    dYq, sdY = quantize_e5m2(dY_bits)
    Xv, Av, Bv = e4m3_decode(Xq), e4m3_decode(Aq)[:, lo:hi], e4m3_decode(Bq)[lo:hi, :]
    dYv = e5m2_decode(dYq)
    S = (Xv @ Av) / (float(sX) * float(sA))
    if b1_bits is not None:
        if np.shape(b1_bits) != (H,):
            raise ValueError("b1 must have the hidden width")
        S = S + bf16_decode(b1_bits)[lo:hi][None, :]
    dZ = (dYv @ Bv.T) / (float(sdY) * float(sB))
    dS_bits = bf16_encode(dZ * gelu_grad(S))
    Z_bits = bf16_encode(gelu(S))
    dSq, sdS = quantize_e5m2(dS_bits)
    Zq, sZ = quantize_inputs_e4m3(Z_bits)
    dSv, Zv = e5m2_decode(dSq), e4m3_decode(Zq)
    g = {"sX": sX, "sA": sA, "sB": sB, "sdY": sdY, "sdS": sdS, "sZ": sZ,
         "Xq": Xq, "Aq_i": Aq[:, lo:hi], "Bq_i": Bq[lo:hi, :], "dYq": dYq,
         "S": S, "dZ": dZ, "dS_bits": dS_bits, "Z_bits": Z_bits, "dSq": dSq, "Zq": Zq,
         "dX": (dSv @ Av.T) / (float(sdS) * float(sA)),
         "dA": (Xv.T @ dSv) / (float(sX) * float(sdS)),
         "dB": (Zv.T @ dYv) / (float(sZ) * float(sdY))}
    if b1_bits is not None:
        g["db1"] = bf16_decode(dS_bits).sum(axis=0)
        g["db2"] = bf16_decode(dY_bits).sum(axis=0)
    return g
