"""CPU oracle for one tensor-parallel rank's share of the Megatron MLP block.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the GPU path; the only thing the
two sides share is the bit patterns of the seeded inputs.

What it computes, and where the pages define it:

* Shard map ("Megatron architecture and 6D parallel guide", §3.1, TP=2
  example; "Megatron-LM deep architecture", column/row-parallel section):
  rank i holds A_i = A[:, i·F:(i+1)·F] and B_i = B[i·F:(i+1)·F, :], F = 4d/N.
* Column-parallel GEMM + elementwise GeLU (same sections; "Megatron-LM"
  glossary, tensor-parallel FFN table): Z_i = GeLU(X·A_i), no exchange.
* Row-parallel GEMM ("Megatron-LM deep architecture", column/row-parallel
  section): Y_i = Z_i·B_i.
* Closed form of the output (same section, eq. for Output):
  Y = Z·B = Σ_i Z_i·B_i = Σ_i Y_i.
* Bias of the column-parallel linear ("Megatron-LM deep architecture", code
  pattern): rank i's block b1_i of the first bias is added to X·A_i inside
  the linear, before GeLU: Z_i = GeLU(X·A_i + b1_i).
* Sequence-parallel share of the sum and the bias ("Megatron-LM deep
  architecture", sequence-parallel section and the row-parallel code
  pattern): rank j keeps rows [j·M/N, (j+1)·M/N) of Σ_i Y_i, and the bias
  is added once, after the reduction.
* fp8 e4m3 forward GEMMs with amax-derived per-tensor scales
  ("Megatron-LM deep architecture", FP8 hybrid precision section), with the
  current scale (the tensor's own amax) or the delayed one (448 over the
  moving average of the amaxes recorded in earlier steps).
* Attention shard (module `attention`; "Megatron-LM" glossary and
  "Megatron architecture and 6D parallel guide", §3.2): the heads split over
  the ranks, column-parallel QKV projection, per-head softmax attention, and
  the row-parallel output projection whose partials sum to the block output.
* fp8 backward in the hybrid formats ("Megatron-LM deep architecture", FP8
  hybrid precision section): E4M3 for activations and weights, E5M2 for the
  gradients, each with its own amax scale.
* Backward of the shard: the chain rule through the forward as computed,
  dZ = dY·B_iᵀ, dS = bf16(dZ ⊙ GeLU'(S)), dX_i = dS·A_iᵀ, dA_i = Xᵀ·dS,
  dB_i = Z_iᵀ·dY; the ranks' dX_i sum to the input gradient (the backward
  AllReduce).

Everything is float64, on bfloat16 (or e4m3) inputs decoded exactly.  Z is
rounded to bfloat16 once, after GeLU, which models the GPU's stored Z.

Pins (tests marked "not gpu"): an exact rational brute force on tiny shapes,
the closed form Σ_i Y_i = Y, N=1 = unsharded, structured inputs that reduce
the path to an elementwise GeLU, textbook values of the normal CDF, and
exhaustive codec checks against torch's CPU conversions.
"""
from . import attention
from .codecs import (bf16_decode, bf16_encode, e4m3_decode, e4m3_encode, e5m2_decode,
                     e5m2_encode, E4M3_MAX, E5M2_MAX)
from .mlp import (shard_columns, gelu, col_gelu, row_partial, mlp_shard, partial_sum,
                  sp_rows, partial_sum_rows, reduce_scatter_share, mlp_unsharded, amax,
                  quant_scale, quant_e4m3, col_gelu_e4m3, requant_z, row_partial_e4m3,
                  mlp_shard_e4m3, quantize_inputs_e4m3, delayed_scale, amax_history_push,
                  col_gelu_e4m3_delayed, mlp_shard_e4m3_delayed, gelu_grad,
                  mlp_shard_backward, quant_scale_e5m2, quant_e5m2, quantize_e5m2,
                  mlp_shard_backward_fp8, col_gelu_bias, mlp_shard_bias, mlp_unsharded_bias)

__all__ = [
    "bf16_decode", "bf16_encode", "e4m3_decode", "e4m3_encode", "E4M3_MAX",
    "e5m2_decode", "e5m2_encode", "E5M2_MAX", "quant_scale_e5m2", "quant_e5m2", "quantize_e5m2",
    "mlp_shard_backward_fp8",
    "shard_columns", "gelu", "col_gelu", "row_partial", "mlp_shard", "partial_sum",
    "sp_rows", "partial_sum_rows", "reduce_scatter_share", "mlp_unsharded", "amax",
    "quant_scale", "quant_e4m3", "col_gelu_e4m3", "requant_z", "row_partial_e4m3",
    "mlp_shard_e4m3", "quantize_inputs_e4m3", "delayed_scale", "amax_history_push",
    "col_gelu_e4m3_delayed", "mlp_shard_e4m3_delayed", "gelu_grad", "mlp_shard_backward",
    "col_gelu_bias", "mlp_shard_bias", "mlp_unsharded_bias", "attention",
]
