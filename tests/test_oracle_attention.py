"""Pins of the oracle's attention shard (CPU): the library routine it reduces
to, an independent loop brute force, closed forms and the sharding identity.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oat
from brute import attention_exact, bf16_round, bf16_value
from workloads import bf16_bits_from_f32, make_attn_inputs, ATTN_WORKLOADS


def _rand_qkv(rng, M, F, sigma=1.0):
    return bf16_bits_from_f32((sigma * rng.standard_normal((M, 3 * F))).astype(np.float32))


def _split(qkv, B, S, heads, dh):
    """[B, heads, S, dh] views of Q, K, V from the head-major layout (float64)."""
    v = oracle.bf16_decode(qkv).reshape(B, S, heads, 3, dh)
    return [np.ascontiguousarray(v[:, :, :, j, :].transpose(0, 2, 1, 3)) for j in range(3)]


@pytest.mark.parametrize("B,S,heads,dh,causal", [(2, 37, 3, 16, True), (1, 64, 2, 128, True),
                                                 (3, 19, 4, 8, False)])
def test_matches_torch_sdpa_in_float64(B, S, heads, dh, causal):
    """softmax(QKᵀ/√dh)·V is exactly what scaled_dot_product_attention computes."""
    rng = np.random.default_rng(B * S + heads)
    qkv = _rand_qkv(rng, B * S, heads * dh)
    O = oat.attention_heads(qkv, B, S, heads, dh, causal, rounding=False)
    q, k, v = (torch.from_numpy(t) for t in _split(qkv, B, S, heads, dh))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
    ref = ref.numpy().transpose(0, 2, 1, 3).reshape(B * S, heads * dh)
    assert np.max(np.abs(O - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("causal", [True, False])
def test_matches_loop_brute_force(causal):
    rng = np.random.default_rng(5)
    B, S, heads, dh = 2, 7, 2, 4
    qkv = _rand_qkv(rng, B * S, heads * dh, sigma=1.5)
    O = oat.attention_heads(qkv, B, S, heads, dh, causal, rounding=False)
    ref = np.array(attention_exact(qkv.tolist(), B, S, heads, dh, causal))
    assert np.max(np.abs(O - ref)) <= 1e-13
    # the stored O is the brute force's value rounded once to bfloat16
    Ob = oat.attention_heads(qkv, B, S, heads, dh, causal)
    exp = np.array([[float(bf16_round(__import__("fractions").Fraction(x))) for x in row] for row in ref])
    assert np.array_equal(oracle.bf16_decode(Ob), exp)


def test_zero_queries_give_prefix_means():
    """Q = 0 makes every visible score equal: causal row t is the mean of V[0..t]."""
    rng = np.random.default_rng(7)
    B, S, heads, dh = 2, 33, 2, 8
    qkv = _rand_qkv(rng, B * S, heads * dh)
    v = qkv.reshape(B * S, heads, 3, dh).copy()
    v[:, :, 0, :] = 0                      # Q columns of every head
    qkv0 = v.reshape(B * S, 3 * heads * dh)
    O = oat.attention_heads(qkv0, B, S, heads, dh, causal=True, rounding=False)
    V = oracle.bf16_decode(v[:, :, 2, :]).reshape(B, S, heads, dh)
    pref = np.cumsum(V, axis=1) / np.arange(1, S + 1)[None, :, None, None]
    assert np.max(np.abs(O.reshape(B, S, heads, dh) - pref)) <= 1e-14
    On = oat.attention_heads(qkv0, B, S, heads, dh, causal=False, rounding=False)
    assert np.max(np.abs(On.reshape(B, S, heads, dh) - V.mean(axis=1, keepdims=True))) <= 1e-14


def test_first_query_copies_first_value_and_dominant_key_is_selected():
    rng = np.random.default_rng(8)
    B, S, heads, dh = 1, 16, 1, 8
    qkv = _rand_qkv(rng, S, dh)
    O = oat.attention_heads(qkv, B, S, heads, dh, causal=True)
    assert np.array_equal(O[0], qkv[0, 2 * dh:3 * dh])      # causal row 0 sees key 0 only
    # one key with a huge score: the weights are one-hot to double precision
    v = qkv.reshape(S, 3, dh).copy()
    v[:, 0, :] = bf16_bits_from_f32(np.full((S, dh), 1.0, np.float32))
    v[:, 1, :] = bf16_bits_from_f32(np.zeros((S, dh), np.float32))
    v[5, 1, :] = bf16_bits_from_f32(np.full(dh, 64.0, np.float32))   # score 64·8/√8 ≈ 181
    On = oat.attention_heads(v.reshape(S, 3 * dh), B, S, heads, dh, causal=False, rounding=False)
    V5 = oracle.bf16_decode(v[5, 2, :])
    assert np.max(np.abs(On - V5[None, :])) <= 1e-60 + 1e-15 * np.max(np.abs(V5))


def test_sequences_are_independent():
    rng = np.random.default_rng(9)
    B, S, heads, dh = 3, 12, 2, 8
    qkv = _rand_qkv(rng, B * S, heads * dh)
    O = oat.attention_heads(qkv, B, S, heads, dh)
    qkv2 = qkv.copy()
    qkv2[S:2 * S] = _rand_qkv(rng, S, heads * dh)          # change sequence 1 only
    O2 = oat.attention_heads(qkv2, B, S, heads, dh)
    assert np.array_equal(O[:S], O2[:S]) and np.array_equal(O[2 * S:], O2[2 * S:])
    assert not np.array_equal(O[S:2 * S], O2[S:2 * S])


@pytest.mark.parametrize("N", [1, 2, 4, 8])
def test_shards_sum_to_the_unsharded_block(N):
    """Σ_i Y_i over the head split equals the block computed head by head on
    one device with the full weights ("Megatron-LM deep architecture": the
    row-parallel output projection needs one AllReduce at the end)."""
    wl = ATTN_WORKLOADS["attn_tiny"]
    X, Wqkv, Wo = make_attn_inputs(wl)
    Yu = oat.attn_unsharded(X, Wqkv, Wo, wl.B, wl.S, wl.heads)
    Ys = sum(oat.attn_shard(X, Wqkv, Wo, N, r, wl.B, wl.S, wl.heads) for r in range(N))
    assert np.max(np.abs(Ys - Yu)) <= 1e-12 * np.max(np.abs(Yu))


def test_qkv_block_follows_the_glossary_listing():
    """Rank i's query columns are columns [i·d/N, (i+1)·d/N) of the unfused Q
    (the glossary's listing), whatever the fused storage."""
    d, heads, N = 64, 8, 4
    dh = d // heads
    # fused head-major matrix whose entries name (kind, unfused column)
    W = np.zeros((d, 3 * d), dtype=np.int64)
    for h in range(heads):
        for j in range(3):
            for e in range(dh):
                W[:, 3 * h * dh + j * dh + e] = 1000 * j + h * dh + e
    for r in range(N):
        blk = oat.qkv_block(W, N, r)[0]
        F = d // N
        qcols = [x for x in blk if x < 1000]
        kcols = [x - 1000 for x in blk if 1000 <= x < 2000]
        vcols = [x - 2000 for x in blk if x >= 2000]
        assert qcols == kcols == vcols == list(range(r * F, (r + 1) * F))
