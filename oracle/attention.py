"""The tensor-parallel attention shard, step by step, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes, and where the pages define it:

* Head split ("Megatron-LM" glossary, tensor-parallel section, and
  "Megatron architecture and 6D parallel guide", §3.2): with h heads and N
  ranks each rank owns h/N whole heads (32 heads at TP=8: 4 per GPU) and
  computes their attention with no exchange.
* Column-parallel QKV projection (same passages; the glossary lists rank i's
  columns as Q[:, i·d/N:(i+1)·d/N] and likewise for K and V).  The fused
  weight W_qkv [d, 3d] is stored head-major: columns [h·3d_h, (h+1)·3d_h)
  are [W_Q,h | W_K,h | W_V,h], head h's query, key and value columns.  The
  heads of rank i are then one contiguous column block for any N, and one
  rank's projection is one GEMM QKV_i = X·W_qkv[:, i·3F:(i+1)·3F], F = d/N.
* Row-parallel output projection (same passages; "Megatron-LM deep
  architecture", multi-head attention paragraph of the column/row-parallel
  section): rank i holds rows [i·F, (i+1)·F) of W_O [d, d] and produces the
  partial Y_i = O_i·W_O,i; the block's output is Σ_i Y_i (one AllReduce).
* Per head (the pages name attention without writing it out; the standard
  scaled dot-product form): O = softmax(Q·Kᵀ/√d_h)·V over each sequence,
  with the causal mask of a decoder (key j visible to query t iff j <= t)
  or none.

Tokens are stored batch-major: row b·S + t of X is token t of sequence b.
Q, K, V and O are rounded to bfloat16 once each, which models the tensors
the path stores; scores, softmax and the weighted sums are float64.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_decode, bf16_encode


def head_columns(d: int, heads: int, N: int, rank: int) -> tuple[int, int, int]:
    """(F, heads per rank, d_h) of rank `rank`'s share of `heads` heads of width d/heads."""
    if N < 1 or not (0 <= rank < N):
        raise ValueError(f"rank {rank} not in [0, {N})")
    if d % heads or heads % N:
        raise ValueError(f"d={d}, heads={heads}, N={N}: heads must divide d and N divide heads")
    dh = d // heads
    hr = heads // N
    return hr * dh, hr, dh


def qkv_block(Wqkv_bits: np.ndarray, N: int, rank: int) -> np.ndarray:
    """Rank `rank`'s column block of the head-major fused W_qkv: its heads'
    [W_Q,h | W_K,h | W_V,h] groups, in head order."""
    d, three_d = Wqkv_bits.shape
    if three_d != 3 * d or d % N:
        raise ValueError("W_qkv must be [d, 3d] with N dividing d")
    F = d // N
    return Wqkv_bits[:, rank * 3 * F:(rank + 1) * 3 * F]


def qkv_proj(X_bits: np.ndarray, Wqkv_bits: np.ndarray, N: int, rank: int) -> np.ndarray:
    """QKV_i = bf16(X·W_qkv,i) [M, 3F] as bfloat16 bits; local head j's Q, K,
    V are columns [3j·dh, (3j+1)·dh), [(3j+1)·dh, (3j+2)·dh), [(3j+2)·dh, (3j+3)·dh)."""
    return bf16_encode(bf16_decode(X_bits) @ bf16_decode(qkv_block(Wqkv_bits, N, rank)))


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax exp(s − max)/Σ exp(s − max); −inf entries get weight 0."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention_heads(QKV_bits: np.ndarray, B: int, S: int, heads: int, dh: int,
                    causal: bool = True, rounding: bool = True) -> np.ndarray:
    """O [M, heads·dh]: per sequence b and head h,
    O_bh = softmax(Q_bh·K_bhᵀ/√dh (+ causal mask))·V_bh, with Q_bh, K_bh, V_bh
    the rows of sequence b in head h's Q, K and V columns (head-major groups).
    Returns bfloat16 bits when `rounding`, else float64."""
    M = B * S
    F = heads * dh
    if QKV_bits.shape != (M, 3 * F):
        raise ValueError(f"QKV must be [{M}, {3 * F}]")
    qkv = bf16_decode(QKV_bits)
    out = np.empty((M, F), dtype=np.float64)
    scale = 1.0 / np.sqrt(dh)
    mask = np.triu(np.ones((S, S), dtype=bool), k=1) if causal else None
    for b in range(B):
        rows = slice(b * S, (b + 1) * S)
        for h in range(heads):
            c = 3 * h * dh
            q = qkv[rows, c:c + dh]
            k = qkv[rows, c + dh:c + 2 * dh]
            v = qkv[rows, c + 2 * dh:c + 3 * dh]
            s = (q @ k.T) * scale
            if causal:
                s = np.where(mask, -np.inf, s)
            out[rows, h * dh:(h + 1) * dh] = softmax_rows(s) @ v
    return bf16_encode(out) if rounding else out


def out_partial(O_bits: np.ndarray, Wo_bits: np.ndarray, N: int, rank: int) -> np.ndarray:
    """Row-parallel output projection: Y_i = O_i·W_O[i·F:(i+1)·F, :] (float64)."""
    d = Wo_bits.shape[0]
    if Wo_bits.shape != (d, d) or d % N:
        raise ValueError("W_O must be [d, d] with N dividing d")
    F = d // N
    return bf16_decode(O_bits) @ bf16_decode(Wo_bits[rank * F:(rank + 1) * F, :])


def attn_shard(X_bits, Wqkv_bits, Wo_bits, N: int, rank: int, B: int, S: int, heads: int,
               causal: bool = True, return_intermediates: bool = False):
    """Rank `rank`'s partial output of the N-way split attention block."""
    M, d = X_bits.shape
    if M != B * S:
        raise ValueError("X must have B·S rows")
    F, hr, dh = head_columns(d, heads, N, rank)
    QKV = qkv_proj(X_bits, Wqkv_bits, N, rank)
    O = attention_heads(QKV, B, S, hr, dh, causal)
    Y = out_partial(O, Wo_bits, N, rank)
    if return_intermediates:
        return Y, QKV, O
    return Y


def attn_unsharded(X_bits, Wqkv_bits, Wo_bits, B: int, S: int, heads: int,
                   causal: bool = True) -> np.ndarray:
    """The whole block on one device, head by head: Y = Σ_h O_h·W_O[h rows, :],
    with head h's Q, K, V from its own column group of W_qkv and its own dh
    rows of W_O; no rank split is involved."""
    M, d = X_bits.shape
    dh = d // heads
    X = bf16_decode(X_bits)
    W = bf16_decode(Wqkv_bits)
    Wo = bf16_decode(Wo_bits)
    Y = np.zeros((M, d), dtype=np.float64)
    for h in range(heads):
        blk = W[:, h * 3 * dh:(h + 1) * 3 * dh]
        qkv = bf16_decode(bf16_encode(X @ blk))
        O = bf16_decode(attention_heads(bf16_encode(qkv), B, S, 1, dh, causal))
        Y += O @ Wo[h * dh:(h + 1) * dh, :]
    return Y
