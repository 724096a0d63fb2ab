// Shared device helpers for the gfx950 kernels of the tensor-parallel MLP
// shard: vector types, bf16 rounding, the block-id remap over XCDs, and the
// GeLU evaluation used by the column-parallel epilogues.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;

// float -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}

// GeLU(x) = x·Φ(x), the exact (Gaussian CDF) form, Φ(x) = ½·erfc(−x/√2).
//
// erfc(z), z = |x|/√2 >= 0, is evaluated with the rational approximation of
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26
// (C. Hastings): erfc(z) ≈ (a1·t + a2·t² + a3·t³ + a4·t⁴ + a5·t⁵)·e^(−z²),
// t = 1/(1 + p·z), with |error| ≤ 1.5e-7 on erf. In fp32 (hardware reciprocal
// and 2^x, each within about 1 ulp) the GeLU error is below |x|·3e-7, far
// under half a bf16 ulp of GeLU(x) except where GeLU(x) itself is below
// about 1e-4, i.e. in the far negative tail. About 15 VALU operations.
__device__ __forceinline__ float gelu_as(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
  float p = fmaf(t, 1.061405429f, -1.453152027f);
  p = fmaf(t, p, 1.421413741f);
  p = fmaf(t, p, -0.284496736f);
  p = fmaf(t, p, 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * z * z);  // e^(−z²)
  const float half_erfc = 0.5f * t * p * e;
  return x * (x >= 0.0f ? 1.0f - half_erfc : half_erfc);
}

// Reference evaluation with the device library's erfcf (used where cost does
// not matter).
__device__ __forceinline__ float gelu_erfc(float x) {
  return 0.5f * x * erfcf(-0.70710678118654752f * x);
}

__device__ __forceinline__ float gelu_exact(float x) { return gelu_as(x); }

// Consecutive workgroup ids are dispatched round-robin over the 8 XCDs of
// an MI355X, each of which has its own L2. Renumber so that a run of
// nblocks/8 consecutive logical ids executes on one XCD; tiles that share
// operand panels are then given consecutive logical ids.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  if (nblocks % kXcd != 0) return bid;
  return (bid % kXcd) * (nblocks / kXcd) + bid / kXcd;
}

// Logical block id -> (tile_m, tile_n) in groups of `group_m` tile rows, so
// consecutive ids walk down a short column of tiles before moving right.
__device__ __forceinline__ void grouped_tile(int bid, int tiles_m, int tiles_n, int group_m,
                                             int& tm, int& tn) {
  const int group_size = group_m * tiles_n;
  const int group = bid / group_size;
  const int first_m = group * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int in_group = bid - group * group_size;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

}  // namespace tpmlp
