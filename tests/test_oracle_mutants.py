"""The pins catch plausible mistakes: each test plants one mistake in the
oracle (on the CPU, by monkeypatching) and checks that at least one pin in
test_oracle.py then fails."""
import numpy as np
import pytest
from scipy.special import erfc

import oracle
from oracle import mlp as omlp
from oracle import codecs as ocodecs
import test_oracle as pins


def _pins_fail(fns):
    for fn in fns:
        try:
            fn()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


BF16_PINS = [
    pins.test_gelu_matches_normal_table,
    pins.test_gelu_identities,
    pins.test_tiny_tp2_matches_brute_force,
    lambda: pins.test_random_tiny_matches_brute_force(7, 16, 16, 4, 12),
    lambda: pins.test_random_tiny_matches_brute_force(16, 12, 8, 2, 13),
    pins.test_tiny_tp2_closed_form,
    pins.test_identity_weights_reduce_to_elementwise_gelu,
    pins.test_shard_map_matches_tp2_example,
]


def _gelu_tanh(s):
    s = np.asarray(s, np.float64)
    return 0.5 * s * (1 + np.tanh(np.sqrt(2 / np.pi) * (s + 0.044715 * s ** 3)))


MUTANTS = {
    "gelu_tanh_form": ("gelu", _gelu_tanh),
    "gelu_dropped_half": ("gelu", lambda s: np.asarray(s) * erfc(-np.asarray(s) * omlp._INV_SQRT2)),
    "gelu_sign_flip": ("gelu", lambda s: np.asarray(s) * 0.5 * erfc(np.asarray(s) * omlp._INV_SQRT2)),
    "gelu_identity": ("gelu", lambda s: np.asarray(s, np.float64)),
    "shard_off_by_one": ("shard_columns",
                         lambda H, N, r: ((r + 1) % N * (H // N), ((r + 1) % N + 1) * (H // N))),
    "shard_stride_wrong": ("shard_columns", lambda H, N, r: (r, r + H // N)),
    "row_partial_reversed_rows": ("row_partial",
                                  lambda Z, B: ocodecs.bf16_decode(Z) @ ocodecs.bf16_decode(B)[::-1]),
    "col_gelu_transposed_x": ("col_gelu", lambda X, A: ocodecs.bf16_encode(omlp.gelu(
        (ocodecs.bf16_decode(X)[:, ::-1]) @ ocodecs.bf16_decode(A)))),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bf16_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(omlp, attr, fn)
    monkeypatch.setattr(oracle, attr, fn, raising=False)
    assert _pins_fail(BF16_PINS), f"mutant {name} passed every pin"


def _truncating_bf16_encode(x):
    x = np.asarray(x, np.float64)
    return (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_truncating_rounding_is_caught(monkeypatch):
    monkeypatch.setattr(omlp, "bf16_encode", _truncating_bf16_encode)
    assert _pins_fail(BF16_PINS)


def test_unrounded_z_is_caught(monkeypatch):
    # keep S·GeLU in float64 all the way: Z is not rounded to bf16 before GEMM2
    def col_gelu(X, A):
        return omlp.gelu(ocodecs.bf16_decode(X) @ ocodecs.bf16_decode(A))

    def row_partial(Z, B):
        Zf = Z if Z.dtype == np.float64 else ocodecs.bf16_decode(Z)
        return Zf @ ocodecs.bf16_decode(B)
    monkeypatch.setattr(omlp, "col_gelu", col_gelu)
    monkeypatch.setattr(omlp, "row_partial", row_partial)
    assert _pins_fail([pins.test_tiny_tp2_matches_brute_force,
                       lambda: pins.test_random_tiny_matches_brute_force(7, 16, 16, 4, 12)])


def test_partial_sum_dropping_a_rank_is_caught(monkeypatch):
    monkeypatch.setattr(omlp, "partial_sum", lambda parts: sum(list(parts)[:-1]))
    monkeypatch.setattr(oracle, "partial_sum", omlp.partial_sum)
    assert _pins_fail([pins.test_tiny_tp2_closed_form,
                       lambda: pins.test_sum_of_shards_equals_unsharded(40, 48, 4, 21)])


FP8_PINS = [
    lambda: pins.test_fp8_path_matches_brute_force(4, 16, 8, 30),
    lambda: pins.test_fp8_path_matches_brute_force(6, 32, 16, 31),
    pins.test_quant_scale_and_codes,
    pins.test_quant_matches_torch_float8,
]


def test_fp8_scale_inverted_is_caught(monkeypatch):
    monkeypatch.setattr(omlp, "row_partial_e4m3",
                        lambda Zq, sZ, Bq, sB: (ocodecs.e4m3_decode(Zq) @ ocodecs.e4m3_decode(Bq))
                        * (float(sZ) * float(sB)))
    assert _pins_fail(FP8_PINS)


def test_fp8_no_clamp_rounding_mode_is_caught(monkeypatch):
    # quantising by truncation toward zero instead of RNE
    def quant(T, s):
        v = (ocodecs.bf16_decode(T).astype(np.float32) * np.float32(s)).astype(np.float64)
        pos = ocodecs.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
        idx = np.searchsorted(pos, np.abs(v), side="right") - 1
        return (idx.astype(np.uint8) | np.where(v < 0, 0x80, 0).astype(np.uint8))
    monkeypatch.setattr(omlp, "quant_e4m3", quant)
    assert _pins_fail(FP8_PINS)


SP_PINS = [
    lambda: pins.test_all_gather_of_reduce_scatter_is_all_reduce(4),
    pins.test_reduce_scatter_shares_sum_to_unsharded_output,
    pins.test_bias_added_once_after_the_sum_brute_force,
    pins.test_partial_sum_rows_ranges_and_errors,
]


def test_bias_added_per_partial_is_caught(monkeypatch):
    def rows(parts, lo, hi, bias=None):
        parts = [np.asarray(p, np.float64) for p in parts]
        b = 0.0 if bias is None else np.asarray(bias)[None, :]
        return omlp.partial_sum([p[lo:hi] + b for p in parts])
    monkeypatch.setattr(omlp, "partial_sum_rows", rows)
    monkeypatch.setattr(oracle, "partial_sum_rows", rows)
    assert _pins_fail(SP_PINS)


def test_share_of_the_wrong_rank_is_caught(monkeypatch):
    monkeypatch.setattr(omlp, "sp_rows", lambda M, N, r: (((r + 1) % N) * (M // N), ((r + 1) % N + 1) * (M // N)))
    assert _pins_fail(SP_PINS)


def test_share_rows_interleaved_instead_of_blocked_is_caught(monkeypatch):
    # a strided (batch-major) slice instead of the contiguous sequence block
    def share(parts, rank, bias=None):
        parts = [np.asarray(p, np.float64) for p in parts]
        acc = omlp.partial_sum([p[rank::len(parts)] for p in parts])
        return acc if bias is None else acc + np.asarray(bias)[None, :]
    monkeypatch.setattr(omlp, "reduce_scatter_share", share)
    monkeypatch.setattr(oracle, "reduce_scatter_share", share)
    assert _pins_fail(SP_PINS)


DELAYED_PINS = [
    pins.test_delayed_scale_moving_average_window,
    pins.test_delayed_path_with_the_current_scale_is_the_current_path,
    lambda: pins.test_delayed_path_matches_brute_force_with_a_predicted_scale(3.5),
    lambda: pins.test_delayed_path_matches_brute_force_with_a_predicted_scale(0.37),
]


def test_delayed_scale_from_the_max_instead_of_the_mean_is_caught(monkeypatch):
    def scale(history):
        h = np.asarray(history, np.float64)
        return np.float32(1.0) if h.size == 0 or h.max() == 0 else np.float32(448.0 / h.max())
    monkeypatch.setattr(omlp, "delayed_scale", scale)
    assert _pins_fail(DELAYED_PINS)


def test_delayed_window_off_by_one_is_caught(monkeypatch):
    def push(history, a, L):
        h = list(history)[-L:] + [float(np.float32(a))]
        return h, omlp.delayed_scale(h)
    monkeypatch.setattr(omlp, "amax_history_push", push)
    monkeypatch.setattr(oracle, "amax_history_push", push)
    assert _pins_fail(DELAYED_PINS)


def test_delayed_quantising_unrounded_z_is_caught(monkeypatch):
    # quantise GeLU's value before it is rounded to bf16
    def col(Xq, sX, Aq, sA, sZ):
        S = (ocodecs.e4m3_decode(Xq) @ ocodecs.e4m3_decode(Aq)) / (float(sX) * float(sA))
        Zf = omlp.gelu(S)
        v = np.clip((Zf.astype(np.float32) * np.float32(sZ)), -448, 448)
        return ocodecs.e4m3_encode(v.astype(np.float64)), float(np.max(np.abs(Zf)))
    monkeypatch.setattr(omlp, "col_gelu_e4m3_delayed", col)
    assert _pins_fail(DELAYED_PINS)


BACKWARD_PINS = [
    pins.test_gelu_grad_identities_and_numerical_derivative,
    lambda: pins.test_backward_formulas_match_finite_differences(2, 1),
    lambda: pins.test_backward_matches_brute_force(4, 8, 16, 2, 0, 62),
    pins.test_backward_shards_compose_to_the_unsharded_gradients,
]


def test_gelu_grad_without_the_density_term_is_caught(monkeypatch):
    monkeypatch.setattr(omlp, "gelu_grad", lambda s: 0.5 * erfc(-np.asarray(s, np.float64) * omlp._INV_SQRT2))
    monkeypatch.setattr(oracle, "gelu_grad", omlp.gelu_grad)
    assert _pins_fail(BACKWARD_PINS)


def test_gelu_grad_sign_flip_is_caught(monkeypatch):
    def g(s):
        s = np.asarray(s, np.float64)
        return 0.5 * erfc(-s * omlp._INV_SQRT2) - s * omlp._INV_SQRT_2PI * np.exp(-0.5 * s * s)
    monkeypatch.setattr(omlp, "gelu_grad", g)
    monkeypatch.setattr(oracle, "gelu_grad", g)
    assert _pins_fail(BACKWARD_PINS)


def _backward_variant(change):
    real = omlp.mlp_shard_backward

    def bw(X, A, B, dY, N, rank, rounding=True):
        out = dict(real(X, A, B, dY, N, rank, rounding))
        change(out, X, A, B, dY, N, rank)
        return out
    return bw


def test_backward_weight_gradient_from_unrounded_gelu_is_caught(monkeypatch):
    def change(out, X, A, B, dY, N, rank):
        out["dB"] = omlp.gelu(out["S"]).T @ ocodecs.bf16_decode(dY)
    bw = _backward_variant(change)
    monkeypatch.setattr(omlp, "mlp_shard_backward", bw)
    monkeypatch.setattr(oracle, "mlp_shard_backward", bw)
    assert _pins_fail(BACKWARD_PINS)


def test_backward_input_gradient_from_dz_instead_of_ds_is_caught(monkeypatch):
    def change(out, X, A, B, dY, N, rank):
        lo, hi = omlp.shard_columns(A.shape[1], N, rank)
        out["dX"] = out["dZ"] @ ocodecs.bf16_decode(A)[:, lo:hi].T
    bw = _backward_variant(change)
    monkeypatch.setattr(omlp, "mlp_shard_backward", bw)
    monkeypatch.setattr(oracle, "mlp_shard_backward", bw)
    assert _pins_fail(BACKWARD_PINS)


def test_backward_untransposed_weight_is_caught(monkeypatch):
    def change(out, X, A, B, dY, N, rank):
        lo, hi = omlp.shard_columns(A.shape[1], N, rank)
        Bi = ocodecs.bf16_decode(B)[lo:hi, :]
        if Bi.shape[0] == Bi.shape[1]:
            dZ = ocodecs.bf16_decode(dY) @ Bi
            out["dS"] = ocodecs.bf16_decode(ocodecs.bf16_encode(dZ * omlp.gelu_grad(out["S"])))
            out["dX"] = out["dS"] @ ocodecs.bf16_decode(A)[:, lo:hi].T
    bw = _backward_variant(change)
    monkeypatch.setattr(omlp, "mlp_shard_backward", bw)
    monkeypatch.setattr(oracle, "mlp_shard_backward", bw)
    assert _pins_fail(BACKWARD_PINS)


# ------------------------------------------------------------- attention --

import test_oracle_attention as apins  # noqa: E402
from oracle import attention as oat  # noqa: E402

ATTN_PINS = [
    lambda: apins.test_matches_torch_sdpa_in_float64(2, 37, 3, 16, True),
    lambda: apins.test_matches_torch_sdpa_in_float64(3, 19, 4, 8, False),
    lambda: apins.test_matches_loop_brute_force(True),
    apins.test_zero_queries_give_prefix_means,
    apins.test_first_query_copies_first_value_and_dominant_key_is_selected,
    apins.test_sequences_are_independent,
    lambda: apins.test_shards_sum_to_the_unsharded_block(4),
    apins.test_qkv_block_follows_the_glossary_listing,
]


def _attention_variant(monkeypatch, fn):
    monkeypatch.setattr(oat, "attention_heads", fn)


def _heads_variant(scale_fn=None, mask_shift=1, swap_kv=False, softmax_axis=-1, per_batch=True):
    def attn(QKV_bits, B, S, heads, dh, causal=True, rounding=True):
        M, F = B * S, heads * dh
        qkv = oracle.bf16_decode(QKV_bits)
        out = np.empty((M, F))
        scale = scale_fn(dh) if scale_fn else 1.0 / np.sqrt(dh)
        for b in range(B):
            rows = slice(b * S, (b + 1) * S) if per_batch else slice(0, S)
            for h in range(heads):
                c = 3 * h * dh
                q = qkv[rows, c:c + dh]
                k = qkv[rows, c + dh:c + 2 * dh]
                v = qkv[rows, c + 2 * dh:c + 3 * dh]
                if swap_kv:
                    k, v = v, k
                s = (q @ k.T) * scale
                if causal:
                    s = np.where(np.triu(np.ones((S, S), bool), k=mask_shift), -np.inf, s)
                m = np.max(s, axis=softmax_axis, keepdims=True)
                with np.errstate(invalid="ignore"):   # a mutant's wrong axis meets a fully masked row
                    e = np.exp(s - m)
                p = e / np.sum(e, axis=softmax_axis, keepdims=True)
                out[b * S:(b + 1) * S, h * dh:(h + 1) * dh] = p @ v
        return oracle.bf16_encode(out) if rounding else out
    return attn


@pytest.mark.parametrize("mutant", [
    dict(scale_fn=lambda dh: 1.0),                 # no 1/√dh
    dict(scale_fn=lambda dh: 1.0 / dh),            # 1/dh
    dict(mask_shift=0),                            # mask hides the diagonal too
    dict(mask_shift=2),                            # one future key visible
    dict(swap_kv=True),                            # K and V columns swapped
    dict(softmax_axis=0),                          # normalised over queries
    dict(per_batch=False),                         # every sequence reads sequence 0
])
def test_attention_mutants_are_caught(monkeypatch, mutant):
    _attention_variant(monkeypatch, _heads_variant(**mutant))
    assert _pins_fail(ATTN_PINS)


def test_attention_wrong_head_block_is_caught(monkeypatch):
    real = oat.qkv_block

    def blk(W, N, rank):   # rank-major [Q_i | K_i | V_i] instead of head-major groups
        d = W.shape[0]
        F = d // N
        return np.concatenate([W[:, j * d + rank * F:j * d + (rank + 1) * F] for j in range(3)], 1)
    monkeypatch.setattr(oat, "qkv_block", blk)
    assert _pins_fail(ATTN_PINS)
    monkeypatch.setattr(oat, "qkv_block", real)


def test_attention_output_rows_of_the_wrong_rank_are_caught(monkeypatch):
    real = oat.out_partial

    def op(O_bits, Wo_bits, N, rank):
        return real(O_bits, Wo_bits, N, (rank + 1) % N)
    monkeypatch.setattr(oat, "out_partial", op)
    assert _pins_fail(ATTN_PINS)


# ------------------------------------------------------- fp8 backward -----

FP8_BWD_PINS = [
    lambda: pins.test_fp8_backward_matches_brute_force(4, 16, 32, 2, 1, 70),
    pins.test_fp8_backward_on_exact_inputs_reduces_to_the_bf16_backward,
]


def _fp8_bwd_variant(monkeypatch, change):
    real = omlp.mlp_shard_backward_fp8

    def bw(X, A, B, dY, N, rank):
        return change(dict(real(X, A, B, dY, N, rank)), X, A, B, dY, N, rank)
    monkeypatch.setattr(omlp, "mlp_shard_backward_fp8", bw)
    monkeypatch.setattr(oracle, "mlp_shard_backward_fp8", bw)


def test_fp8_backward_gradient_in_e4m3_is_caught(monkeypatch):
    def change(g, X, A, B, dY, N, rank):
        dSq, sdS = omlp.quantize_inputs_e4m3(g["dS_bits"])    # e4m3 instead of e5m2
        g["dSq"], g["sdS"] = dSq, sdS
        return g
    _fp8_bwd_variant(monkeypatch, change)
    assert _pins_fail(FP8_BWD_PINS)


def test_fp8_backward_swapped_scales_are_caught(monkeypatch):
    def change(g, X, A, B, dY, N, rank):
        g["dB"] = g["dB"] * (float(g["sdY"]) / float(g["sdS"]))   # divided by sZ·sdS
        return g
    _fp8_bwd_variant(monkeypatch, change)
    assert _pins_fail(FP8_BWD_PINS)


def test_fp8_backward_unquantised_dy_is_caught(monkeypatch):
    real_q = omlp.quantize_e5m2

    def q(T):
        codes, s = real_q(T)
        return omlp.e5m2_encode(oracle.bf16_decode(T) * 1.0), np.float32(1.0)  # no scale
    monkeypatch.setattr(omlp, "quantize_e5m2", q)
    assert _pins_fail(FP8_BWD_PINS)
