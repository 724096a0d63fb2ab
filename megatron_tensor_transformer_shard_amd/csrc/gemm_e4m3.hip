// fp8 (OCP e4m3) variant of the tensor-parallel MLP shard on gfx950.
//
// "Megatron-LM deep architecture", FP8 hybrid precision section: forward
// activation x weight GEMMs run in E4M3; each tensor is multiplied by a
// scale derived from its amax before the cast, and the product of two
// quantised operands is divided by the product of their scales. Here the
// scale is current (s = 448 / amax of the tensor itself).
//
// Kernels:
//  - amax_bf16:  max |T| of a bf16 tensor -> one float (atomic max on the bits;
//                non-negative floats order like their unsigned bit patterns).
//  - quant_e4m3: s = 448/amax; Tq = e4m3(clamp(T·s, ±448)), RNE (v_cvt_pk_fp8_f32).
//  - gemm_e4m3:  C = epilogue((P·Q)/(sP·sQ)) with v_mfma_scale_f32_16x16x128_f8f6f4
//                (both operands e4m3, unit block scales), the same tile engine
//                as the bf16 GEMM with BK = 128 bytes, and either a GeLU +
//                bf16 + amax(|Z|) epilogue, the same with Z quantised to e4m3
//                by a given (delayed) scale, or a plain bf16 store.
//  - quant_fp8_tile: the same quantisation for a strided block, optionally
//                written transposed (through LDS), in e4m3 or e5m2; the fp8
//                backward needs X, A_i, B_i and Z in the other orientation.
//  - The backward's gradients are e5m2 ("Megatron-LM deep architecture", FP8
//                hybrid precision section: E5M2, with its wider range, for the
//                backward's gradients): s = 57344/amax, v_cvt_pk_bf8_f32, and
//                the GEMM takes the format of each operand as a template
//                argument (the MFMA's A and B format fields).
//  - amax_history_push: delayed scaling ("Megatron-LM deep architecture",
//                FP8 section: the scale a step applies is predicted from the
//                moving average of the amaxes of earlier steps, so it is known
//                before the tensor exists and Z can be quantised inside the
//                GEMM's epilogue). One wave records the step's amax in a ring
//                of L values and derives the next scale from their mean.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "tile_engine.hpp"

namespace tpmlp {
namespace {

constexpr int kThreads = 256;
constexpr float kE4m3Max = 448.0f;
constexpr float kE5m2Max = 57344.0f;

// fp8 formats (the MFMA's format codes): 0 = e4m3, 1 = e5m2.
template <int FMT>
constexpr float fp8_max() { return FMT == 0 ? kE4m3Max : kE5m2Max; }

__global__ void fill_f32_kernel(float* p, int n, float v) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ void atomic_max_nonneg(float* addr, float v) {
  atomicMax(reinterpret_cast<unsigned int*>(addr), __builtin_bit_cast(unsigned int, v));
}

// max |x| of the 8 bf16 values in w: |x| of a bf16 is its bit pattern with
// the sign cleared, and non-negative floats order like their bit patterns.
__device__ __forceinline__ uint32_t absmax_bits8(const u32x4& w) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
  return m;
}

// max |T_i| of up to four bf16 tensors in one launch, max'ed into *amax[i].
// A workgroup reads contiguous chunks of kAmaxUnroll x 1024 vectors (128 KB;
// each thread's eight 16-byte loads in flight together), chunk-strided over
// the grid, one tensor after the other; per tensor, the workgroup's waves
// combine through LDS and issue one atomic, since atomics on one address
// serialise.
constexpr int kAmaxThreads = 1024, kAmaxUnroll = 8, kAmaxMaxTensors = 4;
struct AmaxSet {
  const uint16_t* t[kAmaxMaxTensors];
  int64_t numel[kAmaxMaxTensors];
  float* out[kAmaxMaxTensors];
  int n;
};

__global__ __launch_bounds__(kAmaxThreads) void amax_bf16_kernel(AmaxSet set) {
  __shared__ uint32_t part[kAmaxThreads / 64];
  constexpr int64_t kChunk = (int64_t)kAmaxUnroll * kAmaxThreads;
  for (int i = 0; i < set.n; ++i) {
    const uint16_t* T = set.t[i];
    const int64_t numel = set.numel[i], nvec = numel / 8, nchunk = nvec / kChunk;
    const u32x4* src = reinterpret_cast<const u32x4*>(T);
    uint32_t mb = 0;
    for (int64_t c = blockIdx.x; c < nchunk; c += gridDim.x) {
      const u32x4* p = src + c * kChunk + threadIdx.x;
      u32x4 w[kAmaxUnroll];
#pragma unroll
      for (int j = 0; j < kAmaxUnroll; ++j) w[j] = p[j * kAmaxThreads];
#pragma unroll
      for (int j = 0; j < kAmaxUnroll; ++j) mb = max(mb, absmax_bits8(w[j]));
    }
    // the vectors after the last whole chunk, then the elements after the last vector
    for (int64_t v = nchunk * kChunk + (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x; v < nvec;
         v += (int64_t)gridDim.x * kAmaxThreads)
      mb = max(mb, absmax_bits8(src[v]));
    if (blockIdx.x == 0)
      for (int64_t e = nvec * 8 + threadIdx.x; e < numel; e += kAmaxThreads)
        mb = max(mb, T[e] & 0x7FFFu);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mb = max(mb, (uint32_t)__shfl_xor((int)mb, off, 64));
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = mb;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t b = part[0];
#pragma unroll
      for (int w = 1; w < kAmaxThreads / 64; ++w) b = max(b, part[w]);
      atomic_max_nonneg(set.out[i], bf16_bits_to_f32(b));
    }
    __syncthreads();  // part is rewritten for the next tensor
  }
}

template <int FMT = 0>
__device__ __forceinline__ float quant_scale_of(float amax) {
  return amax == 0.0f ? 1.0f : fp8_max<FMT>() / amax;
}

// Two floats -> two e4m3 codes in the low 16 bits (RNE; inputs within ±448).
__device__ __forceinline__ uint32_t cvt_e4m3x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

__device__ __forceinline__ float clamp448(float x) {
  return fminf(fmaxf(x, -kE4m3Max), kE4m3Max);
}

// Two floats -> two codes of format FMT in the low 16 bits, after the clamp
// to the format's largest finite value (RNE).
template <int FMT>
__device__ __forceinline__ uint32_t cvt_fp8x2(float a, float b) {
  constexpr float top = fp8_max<FMT>();
  a = fminf(fmaxf(a, -top), top);
  b = fminf(fmaxf(b, -top), top);
  if constexpr (FMT == 0) return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
  else return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false) & 0xFFFFu;
}

// One wave: lane l sums ring slots l, l+64, ... (the new amax in place of
// its slot), a butterfly combines the lanes, lane 0 writes the slot, the
// count and the scale. Reads of the ring all precede lane 0's write.
__global__ __launch_bounds__(64) void amax_history_push_kernel(float* __restrict__ hist,
                                                               uint32_t* __restrict__ count, int L,
                                                               const float* __restrict__ amax,
                                                               float* __restrict__ next_scale) {
  const int lane = threadIdx.x;
  const uint32_t c = count[0];
  const uint32_t slot = c % (uint32_t)L;
  const uint32_t n = c < (uint32_t)L ? c + 1u : (uint32_t)L;
  const float a = amax[0];
  float sum = 0.0f;
  for (uint32_t j = lane; j < n; j += 64) sum += (j == slot) ? a : hist[j];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (lane == 0) {
    hist[slot] = a;
    count[0] = c + 1u;
    const float mean = sum / (float)n;
    next_scale[0] = mean > 0.0f ? kE4m3Max / mean : 1.0f;
  }
}

// 16 bf16 values (two 16-byte vectors) -> 16 codes of format FMT.
template <int FMT>
__device__ __forceinline__ u32x4 quant16(const u32x4& w0, const u32x4& w1, float s) {
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4& w = (j < 2) ? w0 : w1;
    const uint32_t x0 = w[(j & 1) * 2], x1 = w[(j & 1) * 2 + 1];
    o[j] = cvt_fp8x2<FMT>(bf16_bits_to_f32(x0 & 0xFFFFu) * s, bf16_bits_to_f32(x0 >> 16) * s) |
           (cvt_fp8x2<FMT>(bf16_bits_to_f32(x1 & 0xFFFFu) * s, bf16_bits_to_f32(x1 >> 16) * s)
            << 16);
  }
  return o;
}

// 16 elements per thread per step (two 16-byte loads, one 16-byte store),
// the loads of four grid-stride steps issued together.
template <int FMT>
__global__ __launch_bounds__(kThreads) void quant_fp8_kernel(const uint16_t* __restrict__ T,
                                                             int64_t numel,
                                                             const float* __restrict__ amax,
                                                             uint8_t* __restrict__ Tq,
                                                             float* __restrict__ scale) {
  constexpr int U = 4;
  const float s = quant_scale_of<FMT>(amax[0]);
  if (blockIdx.x == 0 && threadIdx.x == 0) scale[0] = s;
  const int64_t nvec = numel / 16;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const u32x4* src = reinterpret_cast<const u32x4*>(T);
  u32x4* dst = reinterpret_cast<u32x4*>(Tq);
  int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; v + (U - 1) * stride < nvec; v += U * stride) {
    u32x4 w[2 * U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      w[2 * j] = src[2 * (v + j * stride)];
      w[2 * j + 1] = src[2 * (v + j * stride) + 1];
    }
#pragma unroll
    for (int j = 0; j < U; ++j) dst[v + j * stride] = quant16<FMT>(w[2 * j], w[2 * j + 1], s);
  }
  for (; v < nvec; v += stride) dst[v] = quant16<FMT>(src[2 * v], src[2 * v + 1], s);
}

// Quantise the block T [R, C] (row stride ldt) with the scale of `amax` into
// Tq [R, C] (row stride ldq; MODE bit 0) and/or TqT [C, R] (row stride ldqt;
// MODE bit 1), so a tensor needed in both orientations is read once. One
// workgroup per 64 x 64 tile: thread t loads 16 consecutive elements of row
// t / 4 and converts them; the transposed codes go through LDS ([column][row],
// rows of 80 bytes) and thread t stores 16 consecutive codes of output row
// t / 4. R and C are multiples of 16, so a 16-element chunk is either wholly
// inside or wholly outside the block.
template <int FMT, int MODE>
__global__ __launch_bounds__(kThreads) void quant_fp8_tile_kernel(
    const uint16_t* __restrict__ T, int64_t ldt, int R, int C, const float* __restrict__ amax,
    uint8_t* __restrict__ Tq, int64_t ldq, uint8_t* __restrict__ TqT, int64_t ldqt,
    float* __restrict__ scale) {
  constexpr int kTile = 64, kStride = 80;
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTile * kStride];
  const float s = quant_scale_of<FMT>(amax[0]);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) scale[0] = s;
  const int t = threadIdx.x;
  const int r = t >> 2, cc = (t & 3) * 16;
  const int row = blockIdx.y * kTile + r, col = blockIdx.x * kTile + cc;
  u32x4 o = {0u, 0u, 0u, 0u};
  if (row < R && col < C) {
    const u32x4* src = reinterpret_cast<const u32x4*>(T + (int64_t)row * ldt + col);
    o = quant16<FMT>(src[0], src[1], s);
    if constexpr ((MODE & 1) != 0) *reinterpret_cast<u32x4*>(Tq + (int64_t)row * ldq + col) = o;
  }
  if constexpr ((MODE & 2) != 0) {
#pragma unroll
    for (int j = 0; j < 16; ++j) tile[(cc + j) * kStride + r] = (uint8_t)(o[j >> 2] >> (8 * (j & 3)));
    __syncthreads();
    const int orow = blockIdx.x * kTile + r;   // a column of T
    const int ocol = blockIdx.y * kTile + cc;  // rows of T
    if (orow < C && ocol < R)
      *reinterpret_cast<u32x4*>(TqT + (int64_t)orow * ldqt + ocol) =
          *reinterpret_cast<const u32x4*>(tile + r * kStride + cc);
  }
}

// ---------------------------------------------------------------------------
// e4m3 GEMM on the same tile engine as the bf16 GEMMs (see gemm_bf16.hip).
//  - MFMA v_mfma_scale_f32_16x16x128_f8f6f4 (both operands e4m3, unit block
//    scales): a k-slice is 128 e4m3 values (128-byte P rows) and one MFMA
//    k-step. Lane group g = lane >> 4 holds 32 consecutive k-values,
//    k = 32g .. 32g+31, of one row (B operand, from P) or one column (A
//    operand, from Q); any k order works as long as both operands agree.
//  - A workgroup is 4 waves (2 x 2) with a wave tile of up to 128 x 128
//    (MT x NT fragments of 16). The k-step is split into two halves of MFMAs
//    (fragment columns ni < NT/2, then ni >= NT/2) around the slice's barrier,
//    as the bf16 engine splits a slice into its two k-steps.
//  - P fragment (B operand): two ds_read_b128 (16-byte chunks 2g, 2g+1 of the
//    swizzled 128-byte row). The second half runs mi-major, so P fragment mi
//    is reloaded for the next slice right after its last MFMA.
//  - Q fragment (A operand) from the N-contiguous e4m3 Q tile: four
//    ds_read_b64_tr_b8. In each 16-lane group, lane L addresses k-row
//    32g + 8q + (L >> 1), bytes 8·(L & 1) .. +7 of the fragment's 16-byte
//    column granule, and lane j receives byte column j of the 8 rows: 8
//    k-values of one output column per read. Single-buffered: fragment ni is
//    reloaded for the next slice once its last MFMA of this slice is issued.
//  - Granule g of Q row r is stored at (g + f(r)) mod (BN/16); f depends on
//    bits 0-2 and 5 of r and makes every 32-lane pass of a transposing read
//    hit 64 distinct banks (found by exhaustive search).
//  - Three LDS stages for P and two for Q, one barrier per slice: the first
//    half k-step reads the second-half Q fragments of slice kt and issues the
//    P part of slice kt+2 into the P stage of slice kt-1; wait for slice kt+1
//    and barrier; the second half reads the P fragments and first-half Q
//    fragments of slice kt+1 and issues the Q part of slice kt+2 into the Q
//    stage of slice kt. The main loop is uniform (the DMA reloads the last
//    slice into stages never read again near the end).
//  - When K is not a multiple of 128, the last slice loads k clamped into
//    [k_last, K) and its k >= K part is cleared in LDS after it lands.
// ---------------------------------------------------------------------------
namespace e4 {

using namespace engine;

constexpr int BK = 128;   // k (bytes) per LDS slice
constexpr int NSP = 3, NSQ = 2;

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// Rotation of the granules of Q row r (GR granules of 16 bytes per row).
template <int GR>
__device__ __forceinline__ int q8_rot(int r) {
  if constexpr (GR == 16) return (r & 7) + 8 * ((r >> 5) & 1);
  else if constexpr (GR == 12) return ((r >> 2) & 1) + 2 * ((r >> 5) & 1);
  else return ((r >> 1) & 1) + 2 * ((r >> 2) & 1) + 4 * ((r >> 5) & 1);
}

// FP, FQ: fp8 formats of P and Q (0 = e4m3, 1 = e5m2). Workgroups [0, tiles0)
// compute problem g0, the rest problem g1 (a launch of one problem passes
// tiles0 = its tile count).
// Combine the workgroup's per-lane maxima a (and b) and add them to *pa (and
// *pb) with one atomic each: atomics on one address serialise, so one per
// workgroup rather than one per wave. Called by every wave after the
// epilogue; the first barrier also ensures that no wave still reads the LDS
// stages and that every wave's DMA has landed (each waited for it after its
// main loop), so the stage memory can hold the partial maxima.
__device__ __forceinline__ void block_max_to(uint8_t* smem, int wave, int lane, float a, float b,
                                             float* pa, float* pb) {
  a = wave_max(a);
  b = wave_max(b);
  float* red = reinterpret_cast<float*>(smem);
  barrier();
  if (lane == 0) {
    red[wave] = a;
    red[4 + wave] = b;
  }
  waitcnt<0, 0>();
  barrier();
  if (wave == 0 && lane == 0) {
    atomic_max_nonneg(pa, fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
    if (pb != nullptr) atomic_max_nonneg(pb, fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7])));
  }
}

template <int BM, int BN, int OUT, bool KTAIL, int FP, int FQ, int UNR>
__global__ __launch_bounds__(kThreads) void gemm_e4m3_kernel(Fp8GemmArgs g0, Fp8GemmArgs g1,
                                                             int tiles0, int group_m) {
  constexpr int TM = BM / 2, TN = BN / 2;      // wave tile (2 x 2 waves)
  constexpr int MT = TM / 16, NT = TN / 16;    // 16x16 MFMA tiles per wave
  constexpr int NH = NT / 2;                   // fragment columns of the first half k-step
  constexpr int CH = 8;                        // 16-byte chunks per P row
  constexpr int PROW = BK;                     // bytes per P row
  constexpr int PG = BM * CH;                  // granules in a P slice
  constexpr int QGR = BN / 16;                 // granules per Q row
  constexpr int QG = BK * QGR;                 // granules in a Q slice
  constexpr int P_ROUNDS = PG / kThreads, Q_ROUNDS = QG / kThreads;
  constexpr int ROUNDS = P_ROUNDS + Q_ROUNDS;
  constexpr int P_BYTES = PG * 16, Q_BYTES = QG * 16;
  constexpr int Q_BASE = NSP * P_BYTES;
  static_assert(PG % kThreads == 0 && QG % kThreads == 0, "slices must split over 256 lanes");
  static_assert(NT % 2 == 0, "two half k-steps");
  static_assert(NSP * P_BYTES + NSQ * Q_BYTES <= 163840, "LDS stages");
  constexpr bool GELU = OUT == (int)OutKind::GeluBf16 || OUT == (int)OutKind::GeluE4m3;

  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSP * P_BYTES + NSQ * Q_BYTES];

  int id = xcd_remap(blockIdx.x, gridDim.x);
  const bool second = id >= tiles0;
  const Fp8GemmArgs& g = second ? g1 : g0;
  if (second) id -= tiles0;
  const engine::ClockStamp stamp(g.stamps);
  const uint8_t* const P = g.P;
  const uint8_t* const Q = g.Q;
  const float* const sP = g.sP;
  const float* const sQ = g.sQ;
  void* const C = g.C;
  void* const C2 = g.C2;
  float* const z_amax = g.z_amax;
  float* const z_amax2 = g.z_amax2;
  const float* const sC = g.sC;
  const float* const aux = g.aux;
  const int64_t ldp = g.ldp, ldq = g.ldq, ldc = g.ldc, ldaux = g.ldaux;
  const int M = g.M, N = g.N, K = g.K;

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  grouped_tile(id, tiles_m, tiles_n, group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  const int ktiles = (K + BK - 1) / BK;
  const int last = ktiles - 1;
  const int k_last = last * BK;

  // Per-lane byte offsets (from the slice's wave-uniform base) of the
  // granules this lane copies; rows of P beyond M and columns of Q beyond N
  // are clamped; with KTAIL the last slice's offsets are clamped into
  // [k_last, K) (they only move down, so they stay non-negative).
  const uint8_t* p_base = P + (int64_t)m0 * ldp;
  const uint8_t* q_base = Q + n0;
  uint32_t p_off[P_ROUNDS], q_off[Q_ROUNDS];
  uint32_t p_off_t[KTAIL ? P_ROUNDS : 1], q_off_t[KTAIL ? Q_ROUNDS : 1];
#pragma unroll
  for (int j = 0; j < P_ROUNDS; ++j) {
    const int pos = (j * 4 + wave) * 64 + lane;
    const int r = pos / CH, c = swz_p<CH>(r, pos % CH);
    p_off[j] = (uint32_t)((int64_t)(min(m0 + r, M - 1) - m0) * ldp + c * 16);
    if constexpr (KTAIL) {
      const int keep = min(c * 16, K - 16 - k_last);
      p_off_t[j] = p_off[j] - (uint32_t)(c * 16 - keep);
    }
  }
#pragma unroll
  for (int j = 0; j < Q_ROUNDS; ++j) {
    const int pos = (j * 4 + wave) * 64 + lane;
    const int r = pos / QGR, gp = pos % QGR;
    const int g = (gp + QGR - q8_rot<QGR>(r)) % QGR;  // granule stored at position gp
    q_off[j] = (uint32_t)((int64_t)r * ldq + min(n0 + g * 16, N - 16) - n0);
    if constexpr (KTAIL) {
      const int keep = min(r, K - 1 - k_last);
      q_off_t[j] = q_off[j] - (uint32_t)(r - keep) * (uint32_t)ldq;
    }
  }
  const uint32_t lds0 = lds_addr(smem) + wave * 1024;

  auto issue_p = [&](int kt, int pst, int j) __attribute__((always_inline)) {
    uint32_t off = p_off[j];
    if constexpr (KTAIL) off = kt == last ? p_off_t[j] : off;
    dma16(p_base + (int64_t)kt * BK, off, lds0 + pst * P_BYTES + j * 4096);
  };
  auto issue_q = [&](int kt, int qst, int j) __attribute__((always_inline)) {
    uint32_t off = q_off[j];
    if constexpr (KTAIL) off = kt == last ? q_off_t[j] : off;
    dma16(q_base + (int64_t)kt * BK * ldq, off, lds0 + Q_BASE + qst * Q_BYTES + j * 4096);
  };

  // Clear the k >= K part of the last slice's stages (after its DMA landed).
  auto clear_tail = [&]() {
    uint8_t* sp = smem + (last % NSP) * P_BYTES;
    uint8_t* sq = smem + Q_BASE + (last % NSQ) * Q_BYTES;
    const int kvalid = K - k_last;  // multiple of 16, in (0, BK)
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = t; i < PG; i += kThreads) {
      const int r = i / CH, c = i % CH;
      if (c * 16 >= kvalid) *reinterpret_cast<u32x4*>(sp + r * PROW + swz_p<CH>(r, c) * 16) = z;
    }
    for (int i = t; i < QG; i += kThreads)
      if (i / QGR >= kvalid) *reinterpret_cast<u32x4*>(sq + i * 16) = z;
  };

  // Fragment addressing.
  int p_frag[MT];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) p_frag[mi] = wm * TM + mi * 16 + (lane & 15);
  // Q fragment ni, read q: byte q_addr[ni] + 8q·BN of the Q stage. The row's
  // rotation only depends on the lane (bits 0-2 and 5 of the row).
  const int q_row0 = 32 * (lane >> 4) + ((lane & 15) >> 1);
  int q_addr[NT];
#pragma unroll
  for (int ni = 0; ni < NT; ++ni) {
    const int gq = (wn * TN + ni * 16) >> 4;
    q_addr[ni] = q_row0 * BN + ((gq + q8_rot<QGR>(q_row0)) % QGR) * 16 + 8 * (lane & 1);
  }

  // Both fragment sets are single-buffered: each fragment is reloaded for the
  // next slice once its last MFMA of this slice has been issued.
  i32x8 afr[NT];
  i32x8 bfr[MT];
  auto read_q = [&](int qst, int ni, int q) __attribute__((always_inline)) {
    const uint8_t* sq = smem + Q_BASE + qst * Q_BYTES;
    const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (lds_i32x2*)(sq + q_addr[ni] + 8 * q * BN));
    if (q == 0) afr[ni].s01 = v;
    else if (q == 1) afr[ni].s23 = v;
    else if (q == 2) afr[ni].s45 = v;
    else afr[ni].s67 = v;
  };
  auto read_p = [&](int pst, int mi, int h) __attribute__((always_inline)) {
    const uint8_t* sp = smem + pst * P_BYTES;
    const int r = p_frag[mi];
    const u32x4 v = *reinterpret_cast<const u32x4*>(
        sp + r * PROW + swz_p<CH>(r, 2 * (lane >> 4) + h) * 16);
    const i32x4 vi = __builtin_bit_cast(i32x4, v);
    if (h == 0) bfr[mi].lo = vi; else bfr[mi].hi = vi;
  };

  f32x4 acc[NT][MT];
#pragma unroll
  for (int ni = 0; ni < NT; ++ni)
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) acc[ni][mi] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  constexpr int NMH = NH * MT;     // MFMAs per half k-step
  constexpr int NRA = 4 * NH;      // Q-fragment reads per half
  static_assert(NRA <= NMH && P_ROUNDS <= NMH && Q_ROUNDS <= NMH, "slots for reads and DMA");
  // First half of slice kt: MFMAs of fragment columns ni < NH, ni-major; the
  // reads of Q fragments ni >= NH of slice kt (stage rq), and the P part of
  // slice dkt's DMA into P stage dst.
  auto half0 = [&](int rq, int dkt, int dst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NMH; ++i) {
      const int ni = i / MT, mi = i % MT;
      acc[ni][mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          afr[ni], bfr[mi], acc[ni][mi], FQ, FP, 0, 127, 0, 127);
#pragma unroll
      for (int j = 0; j < NRA; ++j)
        if (j * NMH / NRA == i) read_q(rq, NH + j / 4, j % 4);
#pragma unroll
      for (int j = 0; j < P_ROUNDS; ++j)
        if (j * NMH / P_ROUNDS == i) issue_p(dkt, dst, j);
      SCHED_PIN();
    }
  };
  // Second half: fragment columns ni >= NH, mi-major, so P fragment mi is
  // dead after position mi·NH + NH − 1 and is reloaded there from the next
  // slice (P stage rp); the Q fragments ni < NH of the next slice (stage rq)
  // are read early in the half; the Q part of slice dkt's DMA goes into Q
  // stage dst.
  auto half1 = [&](int rp, int rq, int dkt, int dst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NMH; ++i) {
      const int mi = i / NH, ni = NH + i % NH;
      acc[ni][mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          afr[ni], bfr[mi], acc[ni][mi], FQ, FP, 0, 127, 0, 127);
      if (i % NH == NH - 1) {
        read_p(rp, mi, 0);
        read_p(rp, mi, 1);
      }
#pragma unroll
      for (int j = 0; j < NRA; ++j)
        if (j * NMH / (2 * NRA) == i) read_q(rq, j / 4, j % 4);
#pragma unroll
      for (int j = 0; j < Q_ROUNDS; ++j)
        if (j * NMH / Q_ROUNDS == i) issue_q(dkt, dst, j);
      SCHED_PIN();
    }
  };

  // Prologue: slices 0 and 1 (clamped to the last slice) into P stages 0, 1
  // and Q stages 0, 1; wait for slice 0; read its P fragments and its
  // first-half Q fragments.
#pragma unroll
  for (int j = 0; j < P_ROUNDS; ++j) issue_p(0, 0, j);
#pragma unroll
  for (int j = 0; j < Q_ROUNDS; ++j) issue_q(0, 0, j);
#pragma unroll
  for (int j = 0; j < P_ROUNDS; ++j) issue_p(min(1, last), 1, j);
#pragma unroll
  for (int j = 0; j < Q_ROUNDS; ++j) issue_q(min(1, last), 1, j);
  waitcnt<ROUNDS, 0>();
  barrier();
  if (KTAIL && ktiles == 1) {
    clear_tail();
    waitcnt<63, 0>();
    barrier();
  }
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) {
    read_p(0, mi, 0);
    read_p(0, mi, 1);
  }
#pragma unroll
  for (int j = 0; j < NRA; ++j) read_q(0, j / 4, j % 4);

  // Slice kt: Q stage qs = kt & 1, P stage ps = kt % 3. With six slices per
  // iteration (UNR = 6, a multiple of 6 slices) every stage index is a
  // constant; with two (UNR = 2, an even slice count) the Q stages are, and
  // the P stages come from a phase counter (no division on the loop's
  // critical path).
  // (The first k-step reads no P fragments, so slice kt needs the P stages
  // of slices kt+1 and kt+2 only.)
  auto slice = [&](int kt, int ps1, int ps2, int qs) __attribute__((always_inline)) {
    half0(qs, min(kt + 2, last), ps2);
    waitcnt<P_ROUNDS, 0>();  // slice kt+1 has landed (only the P part of kt+2 may be in flight)
    barrier();               // every wave is done reading the stages of slice kt
    if (KTAIL && kt + 2 == ktiles) {
      clear_tail();
      waitcnt<63, 0>();
      barrier();
    }
    half1(ps1, qs ^ 1, min(kt + 2, last), qs);
  };
  if constexpr (UNR == 6) {
    for (int kt = 0; kt < ktiles; kt += 6) {
#pragma unroll
      for (int u = 0; u < 6; ++u) slice(kt + u, (u + 1) % 3, (u + 2) % 3, u & 1);
    }
  } else if constexpr (UNR == 2) {
    int ph = 0;  // kt % 3
    for (int kt = 0; kt < ktiles; kt += 2) {
      const int p1 = ph == 2 ? 0 : ph + 1, p2 = ph == 0 ? 2 : ph - 1;  // (kt + 1) % 3, (kt + 2) % 3
      slice(kt, p1, p2, 0);
      slice(kt + 1, p2, ph, 1);
      ph = p2;
    }
  } else {
    for (int kt = 0; kt < ktiles; ++kt) slice(kt, (kt + 1) % 3, (kt + 2) % 3, kt & 1);
  }
  waitcnt<0, 0>();  // no DMA may still write LDS when the workgroup ends

  // Epilogue: dequantise by 1/(sP·sQ); GeLU + bf16 + max|Z| (+ e4m3 with the
  // given scale), bf16, fp32, or (backward) dS = bf16(acc·GeLU'(S)) and
  // Z = bf16(GeLU(S)) with max|dS| and max|Z|. Lane holds, for 16x16 tile
  // (ni, mi), C[m][n .. n+3] with m = mi·16 + (lane & 15),
  // n = ni·16 + 4·(lane >> 4) (wave-tile relative). Element offsets are a
  // per-lane base (tile (0, 0)) plus the wave-uniform 16·mi rows and 16·ni
  // columns (row strides are below 2^23, so the latter fits 32 bits); a tile
  // is stored where its row and column are inside. The maxima of bf16 values
  // are taken on their bit patterns with the sign cleared, two at a time
  // (v_pk_max_u16): non-negative floats order like their bit patterns.
  // Tiles are stored row block by row block, as in the bf16 engine, so each
  // 128-byte line of C is completed by consecutive store instructions.
  const float dq = 1.0f / (sP[0] * sQ[0]);
  const int mrow = m0 + wm * TM + (lane & 15), ncol = n0 + wn * TN + 4 * (lane >> 4);
  const int rows_left = M - mrow, cols_left = N - ncol;
  const int64_t c_lane = (int64_t)mrow * ldc + ncol;
  auto c_off = [&](int mi, int ni) __attribute__((always_inline)) {
    return c_lane + (int)(16 * mi * ldc + 16 * ni);
  };
  auto inside = [&](int mi, int ni) __attribute__((always_inline)) {
    return 16 * mi < rows_left && 16 * ni < cols_left;
  };
  auto absmax16x2 = [](u16x2 m, uint32_t w) __attribute__((always_inline)) {
    return __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu));
  };
  auto max_of = [](u16x2 m) __attribute__((always_inline)) {
    return bf16_bits_to_f32(max((uint32_t)m[0], (uint32_t)m[1]));
  };
  if constexpr (OUT == (int)OutKind::F32 || OUT == (int)OutKind::F32Bias) {
    // F32Bias: the lane's four bias values per 16-column group, loaded once
    // from a column clamped into [0, N - 4] (N a multiple of 16, ncol of 4)
    // and kept as packed bf16 pairs; a clamped group is never stored.
    [[maybe_unused]] u32x2 bias2[NT];
    if constexpr (OUT == (int)OutKind::F32Bias) {
      const int col_max = N - 4 - ncol;
#pragma unroll
      for (int ni = 0; ni < NT; ++ni)
        bias2[ni] = *reinterpret_cast<const u32x2*>(g.bias + ncol + min(16 * ni, col_max));
    }
    auto store_all = [&](auto checked) __attribute__((always_inline)) {
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
        for (int ni = 0; ni < NT; ++ni) {
          if (decltype(checked)::value && !inside(mi, ni)) continue;
          f32x4 v = acc[ni][mi];
          asm volatile("" : "+v"(v));
          if constexpr (OUT == (int)OutKind::F32Bias) {
            const u32x2 w = bias2[ni];
            const f32x4 b = {__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xFFFF0000u),
                             __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xFFFF0000u)};
            *reinterpret_cast<f32x4*>(static_cast<float*>(C) + c_off(mi, ni)) = v * dq + b;
          } else {
            *reinterpret_cast<f32x4*>(static_cast<float*>(C) + c_off(mi, ni)) = v * dq;
          }
        }
      }
    };
    if (M - m0 >= BM && N - n0 >= BN) store_all(std::false_type{});
    else store_all(std::true_type{});
    stamp.finish(g.stamps);
    return;
  }
  if constexpr (OUT == (int)OutKind::GeluGradBf16) {
    // The S values of EB tiles are loaded together, LA batches ahead of the
    // batch being computed; loads are clamped to the last row and column
    // group (no branch).
    constexpr int EB = 8, NB = NT * MT / EB, LA = 2;
    static_assert((NT * MT) % EB == 0, "epilogue batches");
    const int row_max = M - 1 - mrow, col_max = N - 4 - ncol;
    const float* aux_lane = aux + (int64_t)mrow * ldaux + ncol;
    u16x2 dsm = {0, 0}, zm = {0, 0};
    f32x4 svb[LA + 1][EB];
    const GeluRegs gk = gelu_regs();
    auto load_batch = [&](int b, int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < EB; ++e) {
        const int mi = (b * EB + e) / NT, ni = (b * EB + e) % NT;
        const int r = min(16 * mi, row_max), c = min(16 * ni, col_max);
        svb[buf][e] = *reinterpret_cast<const f32x4*>(aux_lane + ((int64_t)r * (int)ldaux + c));
      }
    };
    // tiles wholly inside C store without the per-tile row and column checks
    auto run = [&](auto checked) __attribute__((always_inline)) {
#pragma unroll
      for (int b = 0; b < LA && b < NB; ++b) load_batch(b, b);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (b + LA < NB) load_batch(b + LA, (b + LA) % (LA + 1));
#pragma unroll
        for (int e = 0; e < EB; ++e) {
          const int mi = (b * EB + e) / NT, ni = (b * EB + e) % NT;
          f32x4 v = acc[ni][mi];
          asm volatile("" : "+v"(v));
          v *= dq;
          if (!decltype(checked)::value || inside(mi, ni)) {
            const f32x4 sv = svb[b % (LA + 1)][e];
            float gl[4], dg[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) gelu_and_grad(sv[q], gl[q], dg[q], gk);
            const u32x2 o = {pack_bf16x2(v[0] * dg[0], v[1] * dg[1]),
                             pack_bf16x2(v[2] * dg[2], v[3] * dg[3])};
            const u32x2 z = {pack_bf16x2(gl[0], gl[1]), pack_bf16x2(gl[2], gl[3])};
            dsm = absmax16x2(absmax16x2(dsm, o[0]), o[1]);
            zm = absmax16x2(absmax16x2(zm, z[0]), z[1]);
            const int64_t off = c_off(mi, ni);
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(C) + off) = o;
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(C2) + off) = z;
          }
        }
      }
    };
    if (M - m0 >= BM && N - n0 >= BN) run(std::false_type{});
    else run(std::true_type{});
    block_max_to(smem, wave, lane, max_of(dsm), max_of(zm), z_amax, z_amax2);
    stamp.finish(g.stamps);
    return;
  }
  const float sc = OUT == (int)OutKind::GeluE4m3 ? sC[0] : 1.0f;
  [[maybe_unused]] const GeluRegs gk = gelu_regs();
  u16x2 zm = {0, 0};
  // tiles wholly inside C store without the per-tile row and column checks
  auto store_all = [&](auto checked) __attribute__((always_inline)) {
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) {
        if (decltype(checked)::value && !inside(mi, ni)) continue;
        f32x4 v = acc[ni][mi];
        asm volatile("" : "+v"(v));
        v *= dq;
        const u32x2 o = GELU ? u32x2{pack_bf16x2(gelu_exact(v[0], gk), gelu_exact(v[1], gk)),
                                     pack_bf16x2(gelu_exact(v[2], gk), gelu_exact(v[3], gk))}
                             : u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        if (GELU) zm = absmax16x2(absmax16x2(zm, o[0]), o[1]);
        const int64_t off = c_off(mi, ni);
        if constexpr (OUT == (int)OutKind::GeluE4m3) {
          // the bf16 Z times the scale in fp32, clamped to ±448, one RNE rounding
          float q[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            q[e] = clamp448(bf16_bits_to_f32((o[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) * sc);
          const uint32_t qb = cvt_e4m3x2(q[0], q[1]) | (cvt_e4m3x2(q[2], q[3]) << 16);
          *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(C) + off) = qb;
        } else {
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(C) + off) = o;
        }
      }
    }
  };
  if (M - m0 >= BM && N - n0 >= BN) store_all(std::false_type{});
  else store_all(std::true_type{});
  if (GELU && z_amax != nullptr) block_max_to(smem, wave, lane, max_of(zm), 0.0f, z_amax, nullptr);
  stamp.finish(g.stamps);
}

}  // namespace e4

template <int BM, int BN>
int tile_count(const Fp8GemmArgs& a) {
  return ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
}

// One launch over problems a[0 .. n) (n = 1 or 2).
// Six slices per main-loop iteration when every problem has a multiple of 6
// slices, two when they are even, else one; not six at 256 x 256 or with a K
// tail, nor two at 256 x 256 with a K tail (the compiler would move or spill
// accumulators).
template <int BM, int BN, int OUT, bool KTAIL, int FP, int FQ>
hipError_t launch_one(const Fp8GemmArgs* a, int n, hipStream_t stream) {
  const int t0 = tile_count<BM, BN>(a[0]);
  const int tiles = t0 + (n > 1 ? tile_count<BM, BN>(a[1]) : 0);
  const int group_m = 4;
  const Fp8GemmArgs& a1 = n > 1 ? a[1] : a[0];
  const int s0 = (a[0].K + e4::BK - 1) / e4::BK, s1 = (a1.K + e4::BK - 1) / e4::BK;
  constexpr bool big = BM == 256 && BN == 256;
  if constexpr (!big && !KTAIL) {
    if (s0 % 6 == 0 && s1 % 6 == 0) {
      hipLaunchKernelGGL((e4::gemm_e4m3_kernel<BM, BN, OUT, KTAIL, FP, FQ, 6>), dim3(tiles),
                         dim3(kThreads), 0, stream, a[0], a1, t0, group_m);
      return hipGetLastError();
    }
  }
  if constexpr (!(KTAIL && big)) {
    if (s0 % 2 == 0 && s1 % 2 == 0) {
      hipLaunchKernelGGL((e4::gemm_e4m3_kernel<BM, BN, OUT, KTAIL, FP, FQ, 2>), dim3(tiles),
                         dim3(kThreads), 0, stream, a[0], a1, t0, group_m);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((e4::gemm_e4m3_kernel<BM, BN, OUT, KTAIL, FP, FQ, 1>), dim3(tiles),
                     dim3(kThreads), 0, stream, a[0], a1, t0, group_m);
  return hipGetLastError();
}

// The (formats, epilogue) combinations the path uses: e4m3 x e4m3 for the
// forward (GeLU, GeLU + e4m3, bf16) and the backward's recomputed S (fp32,
// with or without the column layer's bias);
// e5m2 P x e4m3 Q for dS (GeLU') and dX_i (fp32); e4m3 P x e5m2 Q for the
// weight gradients (fp32).
template <int BM, int BN, bool KTAIL>
hipError_t launch_cfg(const Fp8GemmArgs* a, int n, OutKind out, int fp, int fq, hipStream_t stream) {
  if (fp == 0 && fq == 0) {
    switch (out) {
      case OutKind::GeluBf16: return launch_one<BM, BN, (int)OutKind::GeluBf16, KTAIL, 0, 0>(a, n, stream);
      case OutKind::GeluE4m3: return launch_one<BM, BN, (int)OutKind::GeluE4m3, KTAIL, 0, 0>(a, n, stream);
      case OutKind::Bf16: return launch_one<BM, BN, (int)OutKind::Bf16, KTAIL, 0, 0>(a, n, stream);
      case OutKind::F32: return launch_one<BM, BN, (int)OutKind::F32, KTAIL, 0, 0>(a, n, stream);
      case OutKind::F32Bias: return launch_one<BM, BN, (int)OutKind::F32Bias, KTAIL, 0, 0>(a, n, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (fp == 1 && fq == 0) {
    switch (out) {
      case OutKind::GeluGradBf16: return launch_one<BM, BN, (int)OutKind::GeluGradBf16, KTAIL, 1, 0>(a, n, stream);
      case OutKind::F32: return launch_one<BM, BN, (int)OutKind::F32, KTAIL, 1, 0>(a, n, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (fp == 0 && fq == 1 && out == OutKind::F32)
    return launch_one<BM, BN, (int)OutKind::F32, KTAIL, 0, 1>(a, n, stream);
  return hipErrorInvalidValue;
}

template <int BM, int BN>
hipError_t launch_tile(const Fp8GemmArgs* a, int n, OutKind out, int fp, int fq,
                       hipStream_t stream) {
  bool tail = false;
  for (int i = 0; i < n; ++i) tail = tail || a[i].K % e4::BK != 0;
  if (!tail) return launch_cfg<BM, BN, false>(a, n, out, fp, fq, stream);
  return launch_cfg<BM, BN, true>(a, n, out, fp, fq, stream);
}

int64_t grid_for(int64_t nvec) {
  int64_t blocks = (nvec + kThreads - 1) / kThreads;
  if (blocks > 256 * 8) blocks = 256 * 8;
  return blocks < 1 ? 1 : blocks;
}

}  // namespace

hipError_t launch_fill_f32(float* p, float v, hipStream_t stream, int n) {
  hipLaunchKernelGGL(fill_f32_kernel, dim3(1), dim3(64), 0, stream, p, n, v);
  return hipGetLastError();
}

hipError_t launch_amax_bf16_multi(const uint16_t* const* T, const int64_t* numel,
                                  float* const* amax, int n, hipStream_t stream) {
  if (n < 1 || n > kAmaxMaxTensors) return hipErrorInvalidValue;
  AmaxSet set{};
  int64_t most = 0;
  set.n = 0;
  for (int i = 0; i < n; ++i) {
    if (numel[i] == 0) continue;
    set.t[set.n] = T[i];
    set.numel[set.n] = numel[i];
    set.out[set.n] = amax[i];
    ++set.n;
    most = numel[i] > most ? numel[i] : most;
  }
  if (set.n == 0) return hipSuccess;
  // one 1024-thread workgroup per CU, or one per chunk of the largest tensor
  int64_t blocks = (most / 8 + kAmaxUnroll * kAmaxThreads - 1) / (kAmaxUnroll * kAmaxThreads);
  blocks = blocks < 1 ? 1 : (blocks > 256 ? 256 : blocks);
  hipLaunchKernelGGL(amax_bf16_kernel, dim3((unsigned)blocks), dim3(kAmaxThreads), 0, stream, set);
  return hipGetLastError();
}

hipError_t launch_amax_bf16(const uint16_t* T, int64_t numel, float* amax, hipStream_t stream,
                            bool zero) {
  hipError_t e = zero ? launch_fill_f32(amax, 0.0f, stream) : hipSuccess;
  if (e != hipSuccess || numel == 0) return e;
  return launch_amax_bf16_multi(&T, &numel, &amax, 1, stream);
}

hipError_t launch_quant_fp8(int fmt, const uint16_t* T, int64_t numel, const float* amax,
                            uint8_t* Tq, float* scale, hipStream_t stream) {
  const dim3 grid((unsigned)grid_for(numel / 16));
  if (fmt == 0)
    hipLaunchKernelGGL(quant_fp8_kernel<0>, grid, dim3(kThreads), 0, stream, T, numel, amax, Tq, scale);
  else
    hipLaunchKernelGGL(quant_fp8_kernel<1>, grid, dim3(kThreads), 0, stream, T, numel, amax, Tq, scale);
  return hipGetLastError();
}

hipError_t launch_quant_e4m3(const uint16_t* T, int64_t numel, const float* amax, uint8_t* Tq,
                             float* scale, hipStream_t stream) {
  return launch_quant_fp8(0, T, numel, amax, Tq, scale, stream);
}

namespace {
template <int FMT, int MODE>
void launch_tile_mode(dim3 grid, const uint16_t* T, int64_t ldt, int R, int C, const float* amax,
                      uint8_t* Tq, int64_t ldq, uint8_t* TqT, int64_t ldqt, float* scale,
                      hipStream_t stream) {
  hipLaunchKernelGGL((quant_fp8_tile_kernel<FMT, MODE>), grid, dim3(kThreads), 0, stream, T, ldt,
                     R, C, amax, Tq, ldq, TqT, ldqt, scale);
}
template <int FMT>
void launch_tile_fmt(int mode, dim3 grid, const uint16_t* T, int64_t ldt, int R, int C,
                     const float* amax, uint8_t* Tq, int64_t ldq, uint8_t* TqT, int64_t ldqt,
                     float* scale, hipStream_t stream) {
  if (mode == 1) launch_tile_mode<FMT, 1>(grid, T, ldt, R, C, amax, Tq, ldq, TqT, ldqt, scale, stream);
  else if (mode == 2) launch_tile_mode<FMT, 2>(grid, T, ldt, R, C, amax, Tq, ldq, TqT, ldqt, scale, stream);
  else launch_tile_mode<FMT, 3>(grid, T, ldt, R, C, amax, Tq, ldq, TqT, ldqt, scale, stream);
}
}  // namespace

hipError_t launch_quant_fp8_tile(int fmt, const uint16_t* T, int64_t ldt, int R, int C,
                                 const float* amax, uint8_t* Tq, int64_t ldq, uint8_t* TqT,
                                 int64_t ldqt, float* scale, hipStream_t stream) {
  const int mode = (Tq != nullptr ? 1 : 0) | (TqT != nullptr ? 2 : 0);
  if (mode == 0) return hipErrorInvalidValue;
  if (R == 0 || C == 0) return hipSuccess;
  const dim3 grid((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64));
  if (fmt == 0) launch_tile_fmt<0>(mode, grid, T, ldt, R, C, amax, Tq, ldq, TqT, ldqt, scale, stream);
  else launch_tile_fmt<1>(mode, grid, T, ldt, R, C, amax, Tq, ldq, TqT, ldqt, scale, stream);
  return hipGetLastError();
}

hipError_t launch_amax_history_push(float* history, uint32_t* count, int L, const float* amax,
                                    float* next_scale, hipStream_t stream) {
  hipLaunchKernelGGL(amax_history_push_kernel, dim3(1), dim3(64), 0, stream, history, count, L,
                     amax, next_scale);
  return hipGetLastError();
}

namespace {
// Zero the amax outputs, then launch problems a[0 .. n) with the tile shape of
// the best estimated time: waves of 256 CUs times a per-tile time relative to
// a 256x256 tile (smaller tiles reuse each LDS byte less, so their cost falls
// slower than their area).
hipError_t launch_group(const Fp8GemmArgs* a, int n, OutKind out, int fp, int fq,
                        hipStream_t stream, bool zero_amax) {
  for (int i = 0; i < n && zero_amax; ++i)
    for (float* am : {a[i].z_amax, a[i].z_amax2})
      if (am != nullptr) {
        hipError_t e = launch_fill_f32(am, 0.0f, stream);
        if (e != hipSuccess) return e;
      }
  static const struct { int bm, bn; double cost; } cands[] = {
      {256, 256, 1.00}, {256, 192, 0.85}, {128, 128, 0.30}};
  double best = 1e300;
  int pick = 0;
  int forced = -1, obm, obn;
  if (tile_override(obm, obn))
    for (int c = 0; c < 3; ++c)
      if (cands[c].bm == obm && cands[c].bn == obn) forced = c;
  for (int c = 0; c < 3; ++c) {
    long tiles = 0;
    for (int i = 0; i < n; ++i)
      tiles += (long)((a[i].M + cands[c].bm - 1) / cands[c].bm) * ((a[i].N + cands[c].bn - 1) / cands[c].bn);
    const double est = (double)((tiles + 255) / 256) * cands[c].cost;
    if (est < best - 1e-9) { best = est; pick = c; }
  }
  if (forced >= 0) pick = forced;
  if (pick == 0) return launch_tile<256, 256>(a, n, out, fp, fq, stream);
  if (pick == 1) return launch_tile<256, 192>(a, n, out, fp, fq, stream);
  return launch_tile<128, 128>(a, n, out, fp, fq, stream);
}
}  // namespace

hipError_t launch_gemm_fp8(const Fp8GemmArgs& a, OutKind out, int fp, int fq,
                           hipStream_t stream, bool zero_amax) {
  if (a.M == 0 || a.N == 0) {
    for (float* am : {a.z_amax, a.z_amax2})
      if (am != nullptr && zero_amax) {
        hipError_t e = launch_fill_f32(am, 0.0f, stream);
        if (e != hipSuccess) return e;
      }
    return hipSuccess;
  }
  return launch_group(&a, 1, out, fp, fq, stream, zero_amax);
}

hipError_t launch_gemm_fp8_pair(const Fp8GemmArgs& x, const Fp8GemmArgs& y, OutKind out, int fp,
                                int fq, hipStream_t stream) {
  Fp8GemmArgs a[2];
  int n = 0;
  for (const Fp8GemmArgs* g : {&x, &y})
    if (g->M > 0 && g->N > 0) a[n++] = *g;
  if (n == 0) return hipSuccess;
  return launch_group(a, n, out, fp, fq, stream, true);
}

hipError_t launch_gemm_e4m3(const uint8_t* P, int64_t ldp, const float* sP, const uint8_t* Q,
                            int64_t ldq, const float* sQ, void* C, int64_t ldc, float* z_amax,
                            const float* sC, int M, int N, int K, OutKind out,
                            hipStream_t stream, uint64_t* stamps) {
  Fp8GemmArgs a{P, ldp, sP, Q, ldq, sQ, C, ldc, z_amax, sC, nullptr, 0, nullptr, nullptr,
                M, N, K};
  a.stamps = stamps;
  return launch_gemm_fp8(a, out, 0, 0, stream, true);
}

}  // namespace tpmlp
