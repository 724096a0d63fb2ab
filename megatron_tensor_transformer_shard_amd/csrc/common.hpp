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

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;

// Two floats -> two bfloat16 (low half = lo), round to nearest even; a single
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// float -> bfloat16 bits, round to nearest even.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  return pack_bf16x2(f, 0.0f) & 0xFFFFu;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}

// max(x, 0) for finite x as one v_med3_f32 (fmaxf would first quiet a
// signalling NaN in x with a second instruction; with +inf as the upper
// bound the compiler turns the median into exactly that fmaxf).
__device__ __forceinline__ float relu(float x, float big = 3.40282347e38f) {
  return __builtin_amdgcn_fmed3f(x, 0.0f, big);
}

// GeLU(x) = x·Φ(x), the exact (Gaussian CDF) form.
//
// With h = Φ(−|x|) = ½·erfc(|x|/√2): GeLU(x) = x − |x|·h for x >= 0 and
// x·h = −|x|·h for x < 0, i.e. GeLU(x) = max(x, 0) − |x|·h in both cases.
// erfc(z), z = |x|/√2, is evaluated with the rational approximation of
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26
// (C. Hastings): erfc(z) ≈ (a1·t + a2·t² + a3·t³ + a4·t⁴ + a5·t⁵)·e^(−z²),
// t = 1/(1 + p·z), |error| ≤ 1.5e-7 on erf. Here p/√2 and the ½ are folded
// into the constants and e^(−z²) = 2^(−x²·log2(e)/2). In fp32 (hardware
// reciprocal and 2^x, each within about 1 ulp) the GeLU error is below
// |x|·3e-7, far under half a bf16 ulp of GeLU(x) except where GeLU(x) itself
// is below about 1e-4, i.e. in the far negative tail. 11 VALU operations and
// 2 transcendentals.
//
// The constants of gelu_exact. In an epilogue they are held in VGPRs
// (gelu_regs), opaque to the compiler: a VOP3 instruction (every fma here
// whose operands are not all plain registers) cannot encode a literal, and
// the compiler would otherwise move a literal into a register on every call.
struct GeluRegs {
  float p, a5, a4, a3, a2, a1, big;
};

__device__ __forceinline__ GeluRegs gelu_consts() {
  return GeluRegs{0.3275911f * 0.70710678118654752f, 0.5f * 1.061405429f,
                  0.5f * -1.453152027f, 0.5f * 1.421413741f, 0.5f * -0.284496736f,
                  0.5f * 0.254829592f, 3.40282347e38f};
}

__device__ __forceinline__ GeluRegs gelu_regs() {
  GeluRegs k = gelu_consts();
  asm("" : "+v"(k.p), "+v"(k.a5), "+v"(k.a4), "+v"(k.a3), "+v"(k.a2), "+v"(k.a1), "+v"(k.big));
  return k;
}

__device__ __forceinline__ float gelu_exact(float x, const GeluRegs& k) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(k.p, ax, 1.0f));
  float p = fmaf(t, k.a5, k.a4);
  p = fmaf(t, p, k.a3);
  p = fmaf(t, p, k.a2);
  p = fmaf(t, p, k.a1);
  const float e = __builtin_amdgcn_exp2f((x * -0.72134752044448170f) * x);  // e^(−x²/2)
  const float h = (t * p) * e;                                              // Φ(−|x|)
  return fmaf(-ax, h, relu(x, k.big));
}

__device__ __forceinline__ float gelu_exact(float x) { return gelu_exact(x, gelu_consts()); }

// GeLU(x) and GeLU'(x) = Φ(x) + x·φ(x) together, φ(x) = e^(−x²/2)/√(2π), with
// the same erfc evaluation as gelu_exact: h = Φ(−|x|), Φ(x) = 1 − h for x >= 0
// and h for x < 0. The GeLU'(x) error is that of Φ (below 1e-7) plus fp32
// rounding.
__device__ __forceinline__ void gelu_and_grad(float x, float& g, float& dg,
                                              const GeluRegs& k = gelu_consts()) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(k.p, ax, 1.0f));
  float p = fmaf(t, k.a5, k.a4);
  p = fmaf(t, p, k.a3);
  p = fmaf(t, p, k.a2);
  p = fmaf(t, p, k.a1);
  const float e = __builtin_amdgcn_exp2f((x * -0.72134752044448170f) * x);  // e^(−x²/2)
  const float h = (t * p) * e;                                              // Φ(−|x|)
  g = fmaf(-ax, h, relu(x, k.big));
  const float phi = x >= 0.0f ? 1.0f - h : h;
  dg = fmaf(x, e * 0.39894228040143268f, phi);
}

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
