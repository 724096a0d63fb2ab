// bf16 MFMA GEMMs of the tensor-parallel MLP shard on gfx950.
//
//   column-parallel step:  Z_i = bf16(GeLU(X·A_i))      (GeLU fused in the epilogue)
//   row-parallel step:     Y_i = Z_i·B_i                 (fp32 or bf16 partial)
//
// ("Megatron-LM deep architecture", column/row-parallel section.) Both are
// C = P·Q with P [M, K] K-contiguous (X or Z_i) and Q [K, N] N-contiguous
// (A_i or B_i in the pages' math layout), so one tile engine serves both.
//
// Tile engine (one workgroup = 4 waves = 256 threads, tile BM x BN, waves 2 x 2):
//  - k advances in slices of BK = 64. Both operand slices go HBM -> LDS with
//    global_load_lds_dwordx4 (no staging registers): each wave instruction
//    fills 1 KB of LDS contiguously, and each lane picks the 16-byte granule
//    of HBM that belongs at its LDS position, which is how the LDS swizzles
//    below are realised.
//  - The P slice is stored K-contiguous, 128-byte rows, 16-byte chunk c of row
//    r at c ^ ((r & 7) ^ ((r >> 3) & 1)), so the 8 or 16 lanes served per LDS
//    cycle by a ds_read_b128 of 32 consecutive rows hit distinct banks.
//  - The Q slice stays N-contiguous as in HBM (rows of 2·BN bytes); granule g
//    of row r is stored at (g + 4·(r & 3)) mod (BN/8), a rotation by 64 bytes
//    per row, so the 4 rows read together by a transposing read land in
//    distinct 64-byte bank groups.
//  - MFMA v_mfma_f32_32x32x16_bf16. The Q fragment is the A operand and is read
//    with ds_read_b64_tr_b16: in each 16-lane group, lane L addresses row
//    L>>2, columns 4·(L&3)..+3 of a 4 x 16 block, and lane j receives column j
//    of the 4 rows. Two such reads give the 8 k-values of one output column.
//    The P fragment (B operand) is one ds_read_b128. Each lane ends with 4
//    consecutive output columns per 32x32 tile (8- or 16-byte stores).
//  - Two LDS stages, one barrier per slice: the next slice's data is awaited
//    and the barrier taken before the last k-step's MFMAs, the DMA for the
//    slice after next is issued right after the barrier, and the first
//    fragments of the next slice are read while those MFMAs run.
//  - Rows of P beyond M and columns of Q beyond N are loaded from clamped
//    addresses (their outputs are discarded). In a last partial slice, the
//    k >= K part of both LDS tiles is cleared after the DMA lands.
//  - Workgroup ids are remapped so the tiles of one XCD share P and Q panels
//    in that XCD's L2.
#include "common.hpp"
#include "kernels.hpp"
#include "tile_engine.hpp"

namespace tpmlp {
namespace {

constexpr int kThreads = 256;

using namespace engine;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int BM, int BN, int BK, int NS, int OUT>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(
    const uint16_t* __restrict__ P, int64_t ldp, const uint16_t* __restrict__ Q, int64_t ldq,
    void* __restrict__ C, int64_t ldc, int M, int N, int K, int group_m) {
  constexpr int TM = BM / 2, TN = BN / 2;      // wave tile (2 x 2 waves)
  constexpr int MT = TM / 32, NT = TN / 32;    // 32x32 MFMA tiles per wave
  constexpr int CH = BK / 8;                   // 16-byte chunks per P row
  constexpr int PROW = BK * 2;                 // bytes per P row
  constexpr int PG = BM * CH;                  // granules in a P slice
  constexpr int QGR = BN / 8;                  // granules per Q row
  constexpr int QG = BK * QGR;                 // granules in a Q slice
  constexpr int P_ROUNDS = PG / kThreads, Q_ROUNDS = QG / kThreads;
  constexpr int ROUNDS = P_ROUNDS + Q_ROUNDS;  // DMA instructions per wave per slice
  constexpr int P_BYTES = PG * 16, STAGE = (PG + QG) * 16;
  constexpr int KS = BK / 16;                  // MFMA k-steps per slice
  static_assert(CH == 4 || CH == 8, "BK must be 32 or 64");
  static_assert(PG % kThreads == 0 && QG % kThreads == 0, "slices must split over 256 lanes");
  static_assert(QGR % 4 == 0, "Q rows must hold a multiple of 4 granules");
  static_assert(NS >= 2 && NS <= 5 && NS * STAGE <= 163840, "LDS stages");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE];

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  grouped_tile(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // Per-lane byte offsets (from the tile's wave-uniform base) of the granules
  // this lane copies; rows of P beyond M and columns of Q beyond N are clamped.
  const uint16_t* p_base = P + (int64_t)m0 * ldp;
  const uint16_t* q_base = Q + n0;
  uint32_t p_off[P_ROUNDS], q_off[Q_ROUNDS];
  int p_chunk[P_ROUNDS], q_row[Q_ROUNDS];
#pragma unroll
  for (int j = 0; j < P_ROUNDS; ++j) {
    const int pos = (j * 4 + wave) * 64 + lane;
    const int r = pos / CH, c = swz_p<CH>(r, pos % CH);
    p_chunk[j] = c;
    p_off[j] = (uint32_t)(((int64_t)(min(m0 + r, M - 1) - m0) * ldp + c * 8) * 2);
  }
#pragma unroll
  for (int j = 0; j < Q_ROUNDS; ++j) {
    const int pos = (j * 4 + wave) * 64 + lane;
    const int r = pos / QGR, gp = pos % QGR;
    const int g = (gp + QGR - 4 * (r & 3)) % QGR;
    q_row[j] = r;
    q_off[j] = (uint32_t)(((int64_t)r * ldq + min(n0 + g * 8, N - 8) - n0) * 2);
  }

  const int ktiles = (K + BK - 1) / BK;
  const bool k_tail = (K % BK) != 0;
  const uint32_t lds0 = lds_addr(smem) + wave * 1024;

  // DMA of slice kt into stage kt % NS: the wave-uniform HBM bases and LDS
  // address of the slice, and the j-th of its ROUNDS instructions.
  struct SliceDma {
    const uint16_t* pb;
    const uint16_t* qb;
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
  // Whole slice at once; the last, partial slice clamps k into [k0, K) (the
  // excess is cleared after it lands) and offsets only move down.
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
      const int cc = p_chunk[j] * 8, keep = min(cc, K - 8 - k0);
      dma16(d.pb, p_off[j] - 2u * (uint32_t)(cc - keep), d.lp + j * 4096);
    }
#pragma unroll
    for (int j = 0; j < Q_ROUNDS; ++j) {
      const int r = q_row[j], keep = min(r, K - 1 - k0);
      dma16(d.qb, q_off[j] - 2u * (uint32_t)(r - keep) * (uint32_t)ldq,
            d.lp + P_BYTES + j * 4096);
    }
  };

  // Clear the k >= K part of the last, partial slice (after its DMA landed).
  auto clear_tail = [&](int kt) {
    uint8_t* sp = smem + (kt % NS) * STAGE;
    uint8_t* sq = sp + P_BYTES;
    const int kvalid = K - kt * BK;  // multiple of 8, in (0, BK)
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = t; i < PG; i += kThreads) {
      const int r = i / CH, c = i % CH;
      if (c * 8 >= kvalid) *reinterpret_cast<u32x4*>(sp + r * PROW + swz_p<CH>(r, c) * 16) = z;
    }
    for (int i = t; i < QG; i += kThreads) {
      if (i / QGR >= kvalid) *reinterpret_cast<u32x4*>(sq + i * 16) = z;
    }
  };

  // Fragment addressing (byte offsets within a stage).
  // P (B operand): row m, 16-byte chunk 2s + (lane >> 5).
  int p_frag[MT];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) p_frag[mi] = wm * TM + mi * 32 + (lane & 31);
  // Q (A operand): rows k = 16s + 8(lane>>5) + 4h + ((lane&15)>>2),
  // columns n = wn*TN + ni*32 + 16((lane>>4)&1) + 4(lane&3); the row & 3 of
  // every row a lane reads is (lane&15)>>2, so its rotated granule is fixed.
  const int q_rsub = 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int q_byte = 8 * (lane & 1);
  int q_pos[NT];
#pragma unroll
  for (int ni = 0; ni < NT; ++ni)
    q_pos[ni] = rot_q<QGR>(q_rsub,
                           (wn * TN + ni * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) >> 3) *
                    16 + q_byte;

  // Fragment registers, double-buffered across k-steps. A fragments are two
  // 8-byte halves (one transposing read each).
  s16x8 afr[2][NT];
  bf16x8 bfr[2][MT];
  constexpr int NREADS = MT + 2 * NT;
  // idx-th fragment read of k-step s of slice kt into buffer buf; ordered so
  // that the next k-step's first MFMAs (A fragment 0 with every B fragment)
  // find their operands first.
  auto read_one = [&](int kt, int s, int buf, int idx) {
    const uint8_t* sp = smem + (kt % NS) * STAGE;
    const uint8_t* sq = sp + P_BYTES;
    const int r0 = 16 * s + q_rsub;
    if (idx < 2) {
      const uint8_t* a = sq + (r0 + 4 * idx) * (2 * BN) + q_pos[0];
      const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a);
      if (idx == 0) afr[buf][0].lo = v; else afr[buf][0].hi = v;
    } else if (idx < 2 + MT) {
      const int mi = idx - 2, r = p_frag[mi];
      bfr[buf][mi] = *reinterpret_cast<const bf16x8*>(
          sp + r * PROW + swz_p<CH>(r, 2 * s + (lane >> 5)) * 16);
    } else {
      const int ni = 1 + (idx - 2 - MT) / 2, h = (idx - 2 - MT) % 2;
      const uint8_t* a = sq + (r0 + 4 * h) * (2 * BN) + q_pos[ni];
      const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a);
      if (h == 0) afr[buf][ni].lo = v; else afr[buf][ni].hi = v;
    }
  };

  f32x16 acc[NT][MT];
#pragma unroll
  for (int ni = 0; ni < NT; ++ni)
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[ni][mi][v] = 0.0f;

  // One k-step: the NT x MT MFMAs on buffer `cur`; after MFMA i the i-th
  // fragment read for the next k-step (into cur ^ 1) and, when `dma`, the
  // i-th DMA instruction of slice dkt are issued, so that neither LDS nor
  // global-load issue ever stalls the MFMA pipe for long.
  // (With fewer MFMAs than reads or DMA instructions, slot i takes every
  // j with j·NMFMA/count == i.)
  constexpr int NMFMA = NT * MT;
  auto kstep = [&](int cur, bool reads, int rkt, int rs, bool dma, const SliceDma& dd) {
#pragma unroll
    for (int i = 0; i < NMFMA; ++i) {
      const int ni = i / MT, mi = i % MT;
      acc[ni][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8, afr[cur][ni]), bfr[cur][mi], acc[ni][mi], 0, 0, 0);
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

  // Prologue: the first NS slices in flight; wait for slice 0.
  const int pre = min(NS, ktiles);
  for (int kt = 0; kt < pre; ++kt) issue_slice(kt);
  wait_dma<ROUNDS, NS - 1 < 3 ? NS - 1 : 3>(pre - 1);
  barrier();
  if (k_tail && ktiles == 1) {
    clear_tail(0);
    waitcnt<0, 0>();
    barrier();
  }
#pragma unroll
  for (int i = 0; i < NREADS; ++i) read_one(0, 0, 0, i);

  // Slice kt is read from stage kt % NS. Before its last k-step: wait until
  // slice kt+1 has landed (slices kt+2 .. kt+NS-1 may still be in flight),
  // barrier (every wave has finished reading stage kt % NS), then, during
  // the last k-step, issue slice kt+NS into that stage and read the first
  // fragments of slice kt+1.
  auto sync_next = [&](int kt) {
    wait_dma<ROUNDS, NS - 2 < 3 ? NS - 2 : 3>(min(kt + NS, ktiles) - (kt + 2));
    barrier();
    if (k_tail && kt + 2 == ktiles) {
      clear_tail(kt + 1);
      waitcnt<0, 0>();
      barrier();
    }
  };
  const SliceDma none{};

  // Steady state: every slice issues a full slice kt+NS, interleaved with its
  // last k-step's MFMAs. (One MFMA sequence per call site keeps the
  // accumulators in place.)
  const int steady_end = ktiles - NS - (k_tail ? 1 : 0);
  int kt = 0;
  for (; kt < steady_end; ++kt) {
#pragma unroll
    for (int s = 0; s + 1 < KS; ++s) kstep(s & 1, true, kt, s + 1, false, none);
    sync_next(kt);
    kstep((KS - 1) & 1, true, kt + 1, 0, true, slice_dma(kt + NS));
  }
  // Drain: the remaining slices; a DMA still due (possibly the partial last
  // slice) is issued whole.
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

  // Epilogue. Lane holds, for 32x32 tile (ni, mi) and group g = 0..3,
  // C[m][n .. n+3] with m = (lane & 31), n = 8g + 4·(lane >> 5) (tile-relative).
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
        const float v0 = acc[ni][mi][4 * g + 0], v1 = acc[ni][mi][4 * g + 1];
        const float v2 = acc[ni][mi][4 * g + 2], v3 = acc[ni][mi][4 * g + 3];
        if constexpr (OUT == (int)OutKind::F32) {
          f32x4 o = {v0, v1, v2, v3};
          *reinterpret_cast<f32x4*>(static_cast<float*>(C) + (int64_t)m * ldc + n) = o;
        } else if constexpr (OUT == (int)OutKind::GeluBf16) {
          u32x2 o = {pack_bf16x2(gelu_exact(v0), gelu_exact(v1)),
                     pack_bf16x2(gelu_exact(v2), gelu_exact(v3))};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(C) + (int64_t)m * ldc + n) = o;
        } else {
          u32x2 o = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(C) + (int64_t)m * ldc + n) = o;
        }
      }
    }
  }
}

constexpr int kBK = 64, kStages = 2;

template <int BM, int BN>
hipError_t launch_cfg(const uint16_t* P, int64_t ldp, const uint16_t* Q, int64_t ldq, void* C,
                      int64_t ldc, int M, int N, int K, OutKind out, hipStream_t stream) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int group_m = 4;
  switch (out) {
    case OutKind::GeluBf16:
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, kBK, kStages, (int)OutKind::GeluBf16>), dim3(tiles),
                         dim3(kThreads), 0, stream, P, ldp, Q, ldq, C, ldc, M, N, K, group_m);
      break;
    case OutKind::F32:
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, kBK, kStages, (int)OutKind::F32>), dim3(tiles),
                         dim3(kThreads), 0, stream, P, ldp, Q, ldq, C, ldc, M, N, K, group_m);
      break;
    case OutKind::Bf16:
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, kBK, kStages, (int)OutKind::Bf16>), dim3(tiles),
                         dim3(kThreads), 0, stream, P, ldp, Q, ldq, C, ldc, M, N, K, group_m);
      break;
  }
  return hipGetLastError();
}

struct TileChoice { int bm, bn; };

// Pick the tile shape with the best estimated time: waves of 256 CUs times a
// per-tile cost that grows for smaller tiles (less reuse per LDS byte).
TileChoice choose_tile(int M, int N) {
  static const struct { int bm, bn; double cost; } cands[] = {
      {256, 256, 1.00}, {256, 192, 0.78}, {256, 128, 0.54}, {128, 128, 0.30},
  };
  constexpr int kCus = 256;
  double best = 1e300;
  TileChoice choice{256, 256};
  for (const auto& c : cands) {
    const long tiles = (long)((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
    const long waves = (tiles + kCus - 1) / kCus;
    const double est = waves * c.cost;
    if (est < best - 1e-9) { best = est; choice = {c.bm, c.bn}; }
  }
  return choice;
}

}  // namespace

hipError_t launch_gemm_bf16(const uint16_t* P, int64_t ldp, const uint16_t* Q, int64_t ldq,
                            void* C, int64_t ldc, int M, int N, int K, OutKind out,
                            hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const TileChoice tc = choose_tile(M, N);
  if (tc.bm == 256 && tc.bn == 256) return launch_cfg<256, 256>(P, ldp, Q, ldq, C, ldc, M, N, K, out, stream);
  if (tc.bm == 256 && tc.bn == 192) return launch_cfg<256, 192>(P, ldp, Q, ldq, C, ldc, M, N, K, out, stream);
  if (tc.bm == 256 && tc.bn == 128) return launch_cfg<256, 128>(P, ldp, Q, ldq, C, ldc, M, N, K, out, stream);
  return launch_cfg<128, 128>(P, ldp, Q, ldq, C, ldc, M, N, K, out, stream);
}

}  // namespace tpmlp
