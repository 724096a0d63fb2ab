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
//  - gemm_e4m3:  C = epilogue((P·Q)/(sP·sQ)) with v_mfma_scale_f32_32x32x64_f8f6f4
//                (both operands e4m3, unit block scales), the same tile engine
//                as the bf16 GEMM with BK = 128 bytes, and either a GeLU +
//                bf16 + amax(|Z|) epilogue, the same with Z quantised to e4m3
//                by a given (delayed) scale, or a plain bf16 store.
//  - amax_history_push: delayed scaling ("Megatron-LM deep architecture",
//                FP8 section: the scale a step applies is predicted from the
//                moving average of the amaxes of earlier steps, so it is known
//                before the tensor exists and Z can be quantised inside the
//                GEMM's epilogue). One wave records the step's amax in a ring
//                of L values and derives the next scale from their mean.
#include "common.hpp"
#include "kernels.hpp"
#include "tile_engine.hpp"

namespace tpmlp {
namespace {

constexpr int kThreads = 256;
constexpr float kE4m3Max = 448.0f;

__global__ void fill_f32_kernel(float* p, float v) { *p = v; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ void atomic_max_nonneg(float* addr, float v) {
  atomicMax(reinterpret_cast<unsigned int*>(addr), __builtin_bit_cast(unsigned int, v));
}

__global__ __launch_bounds__(kThreads) void amax_bf16_kernel(const uint16_t* __restrict__ T,
                                                             int64_t numel, float* amax) {
  float m = 0.0f;
  const int64_t nvec = numel / 8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < nvec; v += stride) {
    const u32x4 w = reinterpret_cast<const u32x4*>(T)[v];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = fmaxf(m, fabsf(bf16_bits_to_f32(w[j] & 0xFFFFu)));
      m = fmaxf(m, fabsf(bf16_bits_to_f32(w[j] >> 16)));
    }
  }
  if (blockIdx.x == 0)
    for (int64_t e = nvec * 8 + threadIdx.x; e < numel; e += kThreads)
      m = fmaxf(m, fabsf(bf16_bits_to_f32(T[e])));
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) atomic_max_nonneg(amax, m);
}

__device__ __forceinline__ float quant_scale_of(float amax) {
  return amax == 0.0f ? 1.0f : kE4m3Max / amax;
}

// Two floats -> two e4m3 codes in the low 16 bits (RNE; inputs within ±448).
__device__ __forceinline__ uint32_t cvt_e4m3x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

__device__ __forceinline__ float clamp448(float x) {
  return fminf(fmaxf(x, -kE4m3Max), kE4m3Max);
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

// 16 elements per thread per step: 2 x 16-byte bf16 loads, one 16-byte store.
__global__ __launch_bounds__(kThreads) void quant_e4m3_kernel(const uint16_t* __restrict__ T,
                                                              int64_t numel,
                                                              const float* __restrict__ amax,
                                                              uint8_t* __restrict__ Tq,
                                                              float* __restrict__ scale) {
  const float s = quant_scale_of(amax[0]);
  if (blockIdx.x == 0 && threadIdx.x == 0) scale[0] = s;
  const int64_t nvec = numel / 16;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < nvec; v += stride) {
    const u32x4 w0 = reinterpret_cast<const u32x4*>(T)[2 * v];
    const u32x4 w1 = reinterpret_cast<const u32x4*>(T)[2 * v + 1];
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4& w = (j < 2) ? w0 : w1;
      const uint32_t x0 = w[(j & 1) * 2], x1 = w[(j & 1) * 2 + 1];
      const float f0 = clamp448(bf16_bits_to_f32(x0 & 0xFFFFu) * s);
      const float f1 = clamp448(bf16_bits_to_f32(x0 >> 16) * s);
      const float f2 = clamp448(bf16_bits_to_f32(x1 & 0xFFFFu) * s);
      const float f3 = clamp448(bf16_bits_to_f32(x1 >> 16) * s);
      o[j] = cvt_e4m3x2(f0, f1) | (cvt_e4m3x2(f2, f3) << 16);
    }
    reinterpret_cast<u32x4*>(Tq)[v] = o;
  }
}

// ---------------------------------------------------------------------------
// e4m3 GEMM on the same tile engine as the bf16 GEMMs (see gemm_bf16.hip): a
// k-slice is 128 e4m3 values (BK bytes = 128, the same 128-byte P rows), two
// LDS stages filled by global_load_lds_dwordx4, one barrier per slice, and one
// fragment read and one DMA instruction interleaved after each MFMA.
//  - MFMA v_mfma_scale_f32_32x32x64_f8f6f4 (both operands e4m3, unit block
//    scales): each lane holds 32 k-values of one row (A) or column (B); lane
//    half h = lane >> 5 holds k = 64s + 32h .. +31 of k-step s.
//  - P fragment (B operand): two ds_read_b128 (16-byte chunks 4s+2h, 4s+2h+1).
//  - Q fragment (A operand) from the N-contiguous e4m3 Q tile: four
//    ds_read_b64_tr_b8. In each 16-lane group, lane L addresses row L>>1,
//    bytes 8·(L&1)..+7 of an 8-row x 16-byte block, and lane j receives byte
//    column j of the 8 rows: 8 k-values of one output column per read.
//  - Q rows are BN bytes; granule g of row r is rotated so that the 8 rows x 2
//    granules one read instruction touches per lane half fall in distinct
//    16-byte bank groups (rotations found by exhaustive search over
//    f(r) = a·(r&1) + b·((r>>1)&1) + c·((r>>2)&1)).
// ---------------------------------------------------------------------------
namespace e4 {

using namespace engine;

constexpr int BK = 128, NS = 2, KS = BK / 64;

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

template <int GR>
__device__ __forceinline__ int rot_q8(int r, int g) {
  if constexpr (GR == 16) return (g + 2 * (r & 7)) & 15;
  else if constexpr (GR == 12) return (g + 2 * ((r >> 2) & 1)) % 12;
  else return (g + 2 * ((r >> 1) & 1) + 4 * ((r >> 2) & 1)) % GR;
}

template <int BM, int BN, int OUT>
__global__ __launch_bounds__(kThreads) void gemm_e4m3_kernel(
    const uint8_t* __restrict__ P, int64_t ldp, const float* __restrict__ sP,
    const uint8_t* __restrict__ Q, int64_t ldq, const float* __restrict__ sQ,
    void* __restrict__ C, int64_t ldc, float* __restrict__ z_amax, const float* __restrict__ sC,
    int M, int N, int K, int group_m) {
  constexpr int TM = BM / 2, TN = BN / 2;
  constexpr int MT = TM / 32, NT = TN / 32;
  constexpr int CH = 8, PROW = BK;            // 16-byte chunks / bytes per P row
  constexpr int PG = BM * CH;
  constexpr int QGR = BN / 16;                // granules per Q row
  constexpr int QG = BK * QGR;
  constexpr int P_ROUNDS = PG / kThreads, Q_ROUNDS = QG / kThreads;
  constexpr int ROUNDS = P_ROUNDS + Q_ROUNDS;
  constexpr int P_BYTES = PG * 16, STAGE = (PG + QG) * 16;
  static_assert(PG % kThreads == 0 && QG % kThreads == 0, "slices must split over 256 lanes");
  static_assert(NS * STAGE <= 163840, "LDS stages");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE];

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  grouped_tile(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  const uint8_t* p_base = P + (int64_t)m0 * ldp;
  const uint8_t* q_base = Q + n0;
  uint32_t p_off[P_ROUNDS], q_off[Q_ROUNDS];
  int p_chunk[P_ROUNDS], q_row[Q_ROUNDS];
#pragma unroll
  for (int j = 0; j < P_ROUNDS; ++j) {
    const int pos = (j * 4 + wave) * 64 + lane;
    const int r = pos / CH, c = swz_p<CH>(r, pos % CH);
    p_chunk[j] = c;
    p_off[j] = (uint32_t)((int64_t)(min(m0 + r, M - 1) - m0) * ldp + c * 16);
  }
#pragma unroll
  for (int j = 0; j < Q_ROUNDS; ++j) {
    const int pos = (j * 4 + wave) * 64 + lane;
    const int r = pos / QGR, gp = pos % QGR;
    int g = 0;  // the granule stored at position gp of row r
#pragma unroll
    for (int c = 0; c < QGR; ++c)
      if (rot_q8<QGR>(r, c) == gp) g = c;
    q_row[j] = r;
    q_off[j] = (uint32_t)((int64_t)r * ldq + min(n0 + g * 16, N - 16) - n0);
  }

  const int ktiles = (K + BK - 1) / BK;
  const bool k_tail = (K % BK) != 0;
  const uint32_t lds0 = lds_addr(smem) + wave * 1024;

  struct SliceDma {
    const uint8_t* pb;
    const uint8_t* qb;
    uint32_t lp;
  };
  auto slice_dma = [&](int kt) {
    SliceDma d;
    d.pb = p_base + kt * BK;
    d.qb = q_base + (int64_t)(kt * BK) * ldq;
    d.lp = lds0 + (kt % NS) * STAGE;
    return d;
  };
  auto issue_one = [&](const SliceDma& d, int j) {
    if (j < P_ROUNDS) dma16(d.pb, p_off[j], d.lp + j * 4096);
    else dma16(d.qb, q_off[j - P_ROUNDS], d.lp + P_BYTES + (j - P_ROUNDS) * 4096);
  };
  auto issue_slice = [&](int kt) {
    const SliceDma d = slice_dma(kt);
    if (!(k_tail && kt + 1 == ktiles)) {
#pragma unroll
      for (int j = 0; j < ROUNDS; ++j) issue_one(d, j);
      return;
    }
    const int k0 = kt * BK;
#pragma unroll
    for (int j = 0; j < P_ROUNDS; ++j) {
      const int cc = p_chunk[j] * 16, keep = min(cc, K - 16 - k0);
      dma16(d.pb, p_off[j] - (uint32_t)(cc - keep), d.lp + j * 4096);
    }
#pragma unroll
    for (int j = 0; j < Q_ROUNDS; ++j) {
      const int r = q_row[j], keep = min(r, K - 1 - k0);
      dma16(d.qb, q_off[j] - (uint32_t)(r - keep) * (uint32_t)ldq, d.lp + P_BYTES + j * 4096);
    }
  };
  auto clear_tail = [&](int kt) {
    uint8_t* sp = smem + (kt % NS) * STAGE;
    uint8_t* sq = sp + P_BYTES;
    const int kvalid = K - kt * BK;  // multiple of 16, in (0, BK)
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
  for (int mi = 0; mi < MT; ++mi) p_frag[mi] = wm * TM + mi * 32 + (lane & 31);
  const int q_rsub = 32 * (lane >> 5) + ((lane & 15) >> 1);   // + 64s + 8q
  const int q_byte = 8 * (lane & 1);
  int q_gran[NT];
#pragma unroll
  for (int ni = 0; ni < NT; ++ni) q_gran[ni] = (wn * TN + ni * 32 + 16 * ((lane >> 4) & 1)) >> 4;

  i32x8 afr[2][NT], bfr[2][MT];
  constexpr int NREADS = 2 * MT + 4 * NT;
  // idx-th fragment read of k-step s of slice kt: first the 4 reads of A
  // fragment 0, then the B fragments, then the other A fragments.
  auto read_one = [&](int kt, int s, int buf, int idx) {
    const uint8_t* sp = smem + (kt % NS) * STAGE;
    const uint8_t* sq = sp + P_BYTES;
    auto read_a = [&](int ni, int q) {
      const int r = 64 * s + q_rsub + 8 * q;
      const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (lds_i32x2*)(sq + r * BN + rot_q8<QGR>(r, q_gran[ni]) * 16 + q_byte));
      if (q == 0) afr[buf][ni].s01 = v;
      else if (q == 1) afr[buf][ni].s23 = v;
      else if (q == 2) afr[buf][ni].s45 = v;
      else afr[buf][ni].s67 = v;
    };
    if (idx < 4) {
      read_a(0, idx);
    } else if (idx < 4 + 2 * MT) {
      const int mi = (idx - 4) / 2, half = (idx - 4) % 2, r = p_frag[mi];
      const int chunk = 4 * s + 2 * (lane >> 5) + half;
      const u32x4 v = *reinterpret_cast<const u32x4*>(sp + r * PROW + swz_p<CH>(r, chunk) * 16);
      const i32x4 vi = __builtin_bit_cast(i32x4, v);
      if (half == 0) bfr[buf][mi].lo = vi; else bfr[buf][mi].hi = vi;
    } else {
      const int j = idx - 4 - 2 * MT;
      read_a(1 + j / 4, j % 4);
    }
  };

  f32x16 acc[NT][MT];
#pragma unroll
  for (int ni = 0; ni < NT; ++ni)
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[ni][mi][v] = 0.0f;

  constexpr int NMFMA = NT * MT;
  auto kstep = [&](int cur, bool reads, int rkt, int rs, bool dma, const SliceDma& dd) {
#pragma unroll
    for (int i = 0; i < NMFMA; ++i) {
      const int ni = i / MT, mi = i % MT;
      acc[ni][mi] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          afr[cur][ni], bfr[cur][mi], acc[ni][mi], 0, 0, 0, 127, 0, 127);
      if (reads) {
#pragma unroll
        for (int j = 0; j < NREADS; ++j)
          if ((NREADS <= NMFMA ? j : j * NMFMA / NREADS) == i) read_one(rkt, rs, cur ^ 1, j);
      }
      if (dma) {
#pragma unroll
        for (int j = 0; j < ROUNDS; ++j)
          if ((ROUNDS <= NMFMA ? j : j * NMFMA / ROUNDS) == i) issue_one(dd, j);
      }
      SCHED_PIN();
    }
  };

  const int pre = min(NS, ktiles);
  for (int kt = 0; kt < pre; ++kt) issue_slice(kt);
  wait_dma<ROUNDS, NS - 1>(pre - 1);
  barrier();
  if (k_tail && ktiles == 1) {
    clear_tail(0);
    waitcnt<0, 0>();
    barrier();
  }
#pragma unroll
  for (int i = 0; i < NREADS; ++i) read_one(0, 0, 0, i);

  auto sync_next = [&](int kt) {
    wait_dma<ROUNDS, NS - 2>(min(kt + NS, ktiles) - (kt + 2));
    barrier();
    if (k_tail && kt + 2 == ktiles) {
      clear_tail(kt + 1);
      waitcnt<0, 0>();
      barrier();
    }
  };
  const SliceDma none{};
  const int steady_end = ktiles - NS - (k_tail ? 1 : 0);
  int kt = 0;
  for (; kt < steady_end; ++kt) {
#pragma unroll
    for (int s = 0; s + 1 < KS; ++s) kstep(s & 1, true, kt, s + 1, false, none);
    sync_next(kt);
    kstep((KS - 1) & 1, true, kt + 1, 0, true, slice_dma(kt + NS));
  }
  for (; kt < ktiles; ++kt) {
#pragma unroll
    for (int s = 0; s + 1 < KS; ++s) kstep(s & 1, true, kt, s + 1, false, none);
    const bool more = kt + 1 < ktiles;
    if (more) {
      sync_next(kt);
      if (kt + NS < ktiles) issue_slice(kt + NS);
    }
    kstep((KS - 1) & 1, more, kt + 1, 0, false, none);
  }

  // Epilogue: dequantise by 1/(sP·sQ); GeLU + bf16 + max|Z| (+ e4m3 with the
  // given scale), or bf16.
  constexpr bool GELU = OUT == (int)OutKind::GeluBf16 || OUT == (int)OutKind::GeluE4m3;
  const float dq = 1.0f / (sP[0] * sQ[0]);
  const float sc = OUT == (int)OutKind::GeluE4m3 ? sC[0] : 1.0f;
  float zmax = 0.0f;
#pragma unroll
  for (int ni = 0; ni < NT; ++ni) {
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      const int m = m0 + wm * TM + mi * 32 + (lane & 31);
      if (m >= M) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * TN + ni * 32 + 8 * g + 4 * (lane >> 5);
        if (n >= N) continue;
        uint32_t bits[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = acc[ni][mi][4 * g + e] * dq;
          const float z = GELU ? gelu_exact(v) : v;
          bits[e] = f32_to_bf16_rne(z);
          if (GELU) zmax = fmaxf(zmax, fabsf(bf16_bits_to_f32(bits[e])));
        }
        if constexpr (OUT == (int)OutKind::GeluE4m3) {
          // the bf16 Z times the scale in fp32, clamped to ±448, one RNE rounding
          float q[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) q[e] = clamp448(bf16_bits_to_f32(bits[e]) * sc);
          const uint32_t o = cvt_e4m3x2(q[0], q[1]) | (cvt_e4m3x2(q[2], q[3]) << 16);
          *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(C) + (int64_t)m * ldc + n) = o;
        } else {
          u32x2 o = {bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16)};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(C) + (int64_t)m * ldc + n) = o;
        }
      }
    }
  }
  if (GELU && z_amax != nullptr) {
    zmax = wave_max(zmax);
    if (lane == 0) atomic_max_nonneg(z_amax, zmax);
  }
}

}  // namespace e4

template <int BM, int BN>
hipError_t launch_cfg(const uint8_t* P, int64_t ldp, const float* sP, const uint8_t* Q,
                      int64_t ldq, const float* sQ, void* C, int64_t ldc, float* z_amax,
                      const float* sC, int M, int N, int K, OutKind out, hipStream_t stream) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int group_m = 4;
  if (out == OutKind::GeluBf16)
    hipLaunchKernelGGL((e4::gemm_e4m3_kernel<BM, BN, (int)OutKind::GeluBf16>), dim3(tiles),
                       dim3(kThreads), 0, stream, P, ldp, sP, Q, ldq, sQ, C, ldc, z_amax, sC, M,
                       N, K, group_m);
  else if (out == OutKind::GeluE4m3)
    hipLaunchKernelGGL((e4::gemm_e4m3_kernel<BM, BN, (int)OutKind::GeluE4m3>), dim3(tiles),
                       dim3(kThreads), 0, stream, P, ldp, sP, Q, ldq, sQ, C, ldc, z_amax, sC, M,
                       N, K, group_m);
  else
    hipLaunchKernelGGL((e4::gemm_e4m3_kernel<BM, BN, (int)OutKind::Bf16>), dim3(tiles),
                       dim3(kThreads), 0, stream, P, ldp, sP, Q, ldq, sQ, C, ldc, z_amax, sC, M,
                       N, K, group_m);
  return hipGetLastError();
}

int64_t grid_for(int64_t nvec) {
  int64_t blocks = (nvec + kThreads - 1) / kThreads;
  if (blocks > 256 * 8) blocks = 256 * 8;
  return blocks < 1 ? 1 : blocks;
}

}  // namespace

hipError_t launch_fill_f32(float* p, float v, hipStream_t stream) {
  hipLaunchKernelGGL(fill_f32_kernel, dim3(1), dim3(1), 0, stream, p, v);
  return hipGetLastError();
}

hipError_t launch_amax_bf16(const uint16_t* T, int64_t numel, float* amax, hipStream_t stream) {
  hipError_t e = launch_fill_f32(amax, 0.0f, stream);
  if (e != hipSuccess || numel == 0) return e;
  hipLaunchKernelGGL(amax_bf16_kernel, dim3((unsigned)grid_for(numel / 8)), dim3(kThreads), 0,
                     stream, T, numel, amax);
  return hipGetLastError();
}

hipError_t launch_quant_e4m3(const uint16_t* T, int64_t numel, const float* amax, uint8_t* Tq,
                             float* scale, hipStream_t stream) {
  hipLaunchKernelGGL(quant_e4m3_kernel, dim3((unsigned)grid_for(numel / 16)), dim3(kThreads), 0,
                     stream, T, numel, amax, Tq, scale);
  return hipGetLastError();
}

hipError_t launch_amax_history_push(float* history, uint32_t* count, int L, const float* amax,
                                    float* next_scale, hipStream_t stream) {
  hipLaunchKernelGGL(amax_history_push_kernel, dim3(1), dim3(64), 0, stream, history, count, L,
                     amax, next_scale);
  return hipGetLastError();
}

hipError_t launch_gemm_e4m3(const uint8_t* P, int64_t ldp, const float* sP, const uint8_t* Q,
                            int64_t ldq, const float* sQ, void* C, int64_t ldc, float* z_amax,
                            const float* sC, int M, int N, int K, OutKind out,
                            hipStream_t stream) {
  if (z_amax != nullptr) {
    hipError_t e = launch_fill_f32(z_amax, 0.0f, stream);
    if (e != hipSuccess) return e;
  }
  if (M == 0 || N == 0) return hipSuccess;
  // Tile shape with the best estimated time: waves of 256 CUs times a
  // per-tile cost that grows for smaller tiles. (A 256x256 e4m3 tile would
  // need more than the 512 registers a lane has.)
  static const struct { int bm, bn; double cost; } cands[] = {{256, 192, 1.00}, {128, 128, 0.38}};
  double best = 1e300;
  int pick = 0;
  for (int i = 0; i < 2; ++i) {
    const long tiles = (long)((M + cands[i].bm - 1) / cands[i].bm) * ((N + cands[i].bn - 1) / cands[i].bn);
    const double est = (double)((tiles + 255) / 256) * cands[i].cost;
    if (est < best - 1e-9) { best = est; pick = i; }
  }
  if (pick == 0)
    return launch_cfg<256, 192>(P, ldp, sP, Q, ldq, sQ, C, ldc, z_amax, sC, M, N, K, out, stream);
  return launch_cfg<128, 128>(P, ldp, sP, Q, ldq, sQ, C, ldc, z_amax, sC, M, N, K, out, stream);
}

}  // namespace tpmlp
