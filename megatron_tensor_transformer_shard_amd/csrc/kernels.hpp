// Internal launch interface between the C ABI (abi.cpp) and the gfx950
// kernels. Every launcher enqueues on `stream` and returns the launch status;
// argument validation has already happened in the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

namespace tpmlp {

// Tile shape named by the environment variable TPMLP_TILE ("<BM>x<BN>", e.g.
// "256x192"). The GEMM launchers take it instead of their own choice when it
// names one of their instantiated shapes, so that tests can run every tile
// shape on shapes small enough to check each output element against the
// oracle. Unset or malformed: false, and the launchers choose as usual.
inline bool tile_override(int& bm, int& bn) {
  const char* s = getenv("TPMLP_TILE");
  if (s == nullptr || *s == '\0') return false;
  int a = 0, b = 0;
  char tail = 0;
  if (sscanf(s, "%dx%d%c", &a, &b, &tail) != 2) return false;
  bm = a;
  bn = b;
  return true;
}

// Epilogues: GeluBf16 = bf16(GeLU(acc)); F32 = acc; Bf16 = bf16(acc);
// GeluE4m3 (fp8 GEMM only): bf16(GeLU(acc)) quantised to e4m3 with a given
// scale, one byte per element; GeluGradBf16 (backward, both engines):
// C = bf16(acc·GeLU'(S)), C2 = bf16(GeLU(S)) with S read from an fp32 [M, N]
// matrix. In the fp8 engine acc is first divided by sP·sQ.
enum class OutKind : int { GeluBf16 = 0, F32 = 1, Bf16 = 2, GeluE4m3 = 3, GeluGradBf16 = 4, GeluBiasBf16 = 5,
                            F32Bias = 6 };

// Operand layouts of the bf16 GEMM C = P·Q: NN = P [M, K] K-contiguous and
// Q [K, N] N-contiguous (the forward); QT = Q stored [N, K] K-contiguous;
// PT = P stored [K, M] M-contiguous.
enum class Layout : int { NN = 0, QT = 1, PT = 2 };

// C[M, N] = epilogue(P[M, K] · Q[K, N]); P rows K-contiguous (stride ldp),
// Q rows N-contiguous (stride ldq), C dense with stride ldc, all bf16 inputs.
// stamps (measurement only, else NULL): 4 clock stamps per workgroup, see
// engine::ClockStamp; room for 4·⌈M/128⌉·⌈N/128⌉ values covers any tile.
hipError_t launch_gemm_bf16(const uint16_t* P, int64_t ldp, const uint16_t* Q, int64_t ldq,
                            void* C, int64_t ldc, int M, int N, int K, OutKind out,
                            hipStream_t stream, uint64_t* stamps = nullptr);

// The same GEMM with another operand layout and the backward's epilogue;
// ldp / ldq are the row strides of P and Q as stored; aux/ldaux (fp32 S) and
// C2 (bf16 Z, row stride ldc) are used by GeluGradBf16 only.
hipError_t launch_gemm_bf16_ex(const uint16_t* P, int64_t ldp, const uint16_t* Q, int64_t ldq,
                               void* C, int64_t ldc, int M, int N, int K, OutKind out, Layout lay,
                               const float* aux, int64_t ldaux, void* C2, hipStream_t stream);

// C = bf16(GeLU(P·Q + bias)) (out GeluBiasBf16, layout NN or QT) or the fp32
// C = P·Q + bias (out F32Bias, layout NN), with bias bf16 [N] added to every row.
hipError_t launch_gemm_bf16_bias(const uint16_t* P, int64_t ldp, const uint16_t* Q, int64_t ldq,
                                 const uint16_t* bias, void* C, int64_t ldc, int M, int N, int K,
                                 OutKind out, Layout lay, hipStream_t stream);

// out[c] = Σ_r G[r, c] in fp32 (bias gradient), G bf16 [rows, cols] with row
// stride ld, cols a multiple of 8; partial holds colsum_row_blocks(rows)·cols
// floats of scratch. Deterministic (no atomics).
int64_t colsum_row_blocks(int64_t rows);
hipError_t launch_colsum_bf16(const uint16_t* G, int64_t ld, int rows, int cols, float* out,
                              float* partial, hipStream_t stream);

// Two independent GEMMs of one layout and epilogue (fp32 or bf16 output) in
// one launch, so that two problems of few tiles each fill the chip together.
struct BfGemm {
  const uint16_t* P; int64_t ldp; const uint16_t* Q; int64_t ldq; void* C; int64_t ldc;
  int M, N, K;
};
hipError_t launch_gemm_bf16_pair(const BfGemm& x, const BfGemm& y, OutKind out, Layout lay,
                                 hipStream_t stream);

// Per-head causal (or full) softmax attention of one rank, head width 128:
// QKV [B·S, ld] bf16 with head j's Q, K, V at columns 3j·128 + {0, 128, 256};
// O [B·S, ldo] bf16 with head j at columns j·128.
hipError_t launch_attention(const uint16_t* QKV, int64_t ld, uint16_t* O, int64_t ldo, int B,
                            int S, int heads, bool causal, hipStream_t stream);

// Y = Σ_i parts[i] in rank order, fp32 accumulation, then + bias[e % d] when
// bias_kind is 1 (fp32 bias) or 2 (bf16 bias); bias_kind 0 adds nothing.
hipError_t launch_partial_sum(const void* const* parts, int nparts, bool parts_bf16, void* Y,
                              bool y_bf16, int64_t numel, const void* bias, int bias_kind,
                              int64_t d, hipStream_t stream);

// fp8 paths (OCP e4m3 forward, e4m3 / e5m2 backward).
// p[0 .. n) = v (n <= 64), one small kernel (no memset: safe under graph capture).
hipError_t launch_fill_f32(float* p, float v, hipStream_t stream, int n = 1);
// *amax = max |T| (zeroed first unless zero is false: then it is max'ed into).
hipError_t launch_amax_bf16(const uint16_t* T, int64_t numel, float* amax, hipStream_t stream,
                            bool zero = true);
// *amax[i] = max(*amax[i], max |T[i]|) for up to four tensors in one launch
// (the slots are not cleared).
hipError_t launch_amax_bf16_multi(const uint16_t* const* T, const int64_t* numel,
                                  float* const* amax, int n, hipStream_t stream);
hipError_t launch_quant_e4m3(const uint16_t* T, int64_t numel, const float* amax, uint8_t* Tq,
                             float* scale, hipStream_t stream);
// C = epilogue((P·Q) / (sP·sQ)); GeluBf16 also folds max|Z| into z_amax when
// z_amax is not NULL; Bf16 stores bf16; GeluE4m3 stores e4m3(bf16(GeLU)·sC[0])
// bytes (ldc in bytes) and folds max|bf16(GeLU)| into z_amax.
// fp8 GEMM C = epilogue((P·Q)/(sP·sQ)) with P [M, K] (row stride ldp) and Q
// [K, N] (row stride ldq) as fp8 codes of formats fp and fq (0 = e4m3, 1 =
// e5m2). z_amax (and z_amax2) are zeroed on the stream first when given.
// Epilogues: GeluBf16 / GeluE4m3 / Bf16 (e4m3 x e4m3, z_amax = max|Z|, sC the
// e4m3 scale of Z), F32 (any of the format pairs used), GeluGradBf16 (e5m2 P x
// e4m3 Q: C = bf16(acc·GeLU'(S)) with S from aux [M, N] fp32, C2 = bf16(GeLU(S)),
// z_amax = max|C|, z_amax2 = max|C2|).
struct Fp8GemmArgs {
  const uint8_t* P; int64_t ldp; const float* sP;
  const uint8_t* Q; int64_t ldq; const float* sQ;
  void* C; int64_t ldc; float* z_amax; const float* sC;
  const float* aux; int64_t ldaux; void* C2; float* z_amax2;
  int M, N, K;
  const uint16_t* bias = nullptr;  // F32Bias: bf16 [N], added to every row after dequantising
  uint64_t* stamps = nullptr;      // measurement only: clock stamps per workgroup (ClockStamp)
};
hipError_t launch_gemm_fp8(const Fp8GemmArgs& a, OutKind out, int fp, int fq,
                           hipStream_t stream, bool zero_amax = true);
// Two independent fp8 GEMMs of one format pair and epilogue in one launch.
hipError_t launch_gemm_fp8_pair(const Fp8GemmArgs& x, const Fp8GemmArgs& y, OutKind out, int fp,
                                int fq, hipStream_t stream);

// Tq = fp8 codes (format fmt) of T·s, s = MAX/amax (448 for e4m3, 57344 for
// e5m2; 1 if amax = 0), clamped to ±MAX, RNE; scale[0] = s. numel % 16 == 0
// handled in vector steps (the caller guarantees it).
hipError_t launch_quant_fp8(int fmt, const uint16_t* T, int64_t numel, const float* amax,
                            uint8_t* Tq, float* scale, hipStream_t stream);
// The same for the block T [R, C] (row stride ldt), written to Tq [R, C]
// (row stride ldq) and/or its transpose TqT [C, R] (row stride ldqt) from one
// read of T; either output may be NULL, not both. R and C multiples of 16.
hipError_t launch_quant_fp8_tile(int fmt, const uint16_t* T, int64_t ldt, int R, int C,
                                 const float* amax, uint8_t* Tq, int64_t ldq, uint8_t* TqT,
                                 int64_t ldqt, float* scale, hipStream_t stream);

hipError_t launch_gemm_e4m3(const uint8_t* P, int64_t ldp, const float* sP, const uint8_t* Q,
                            int64_t ldq, const float* sQ, void* C, int64_t ldc, float* z_amax,
                            const float* sC, int M, int N, int K, OutKind out,
                            hipStream_t stream, uint64_t* stamps = nullptr);
// Delayed scaling: record amax[0] in the ring history[L] at slot count % L,
// advance count, and write next_scale[0] = 448 / mean of the recorded values
// (the last min(count, L)), or 1 when that mean is 0.
hipError_t launch_amax_history_push(float* history, uint32_t* count, int L, const float* amax,
                                    float* next_scale, hipStream_t stream);

}  // namespace tpmlp
