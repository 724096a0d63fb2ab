// bf16 MFMA GEMMs of the tensor-parallel MLP shard on gfx950.
//
//   column-parallel step:  Z_i = bf16(GeLU(X·A_i))      (GeLU fused in the epilogue)
//                          or bf16(GeLU(X·A_i + b1_i)) with the layer's bias
//   row-parallel step:     Y_i = Z_i·B_i                 (fp32 or bf16 partial)
//
// ("Megatron-LM deep architecture", column/row-parallel section.) Both are
// C = P·Q with P [M, K] K-contiguous (X or Z_i) and Q [K, N] N-contiguous
// (A_i or B_i in the pages' math layout), so one tile engine serves both.
//
// Tile engine (one workgroup = 4 waves = 256 threads, tile BM x BN, waves 2 x 2,
// wave tile up to 128 x 128):
//  - MFMA v_mfma_f32_16x16x32_bf16. With random operands the chip's power
//    limit holds a 16x16x32 stream at a markedly higher clock than the
//    32x32x16 one (fewer accumulator reads and writes per flop), which is
//    what bounds a dense bf16 GEMM on MI355X.
//  - k advances in slices of BK = 64 (two MFMA k-steps of 32). Both operand
//    slices go HBM -> LDS with global_load_lds_dwordx4 (no staging
//    registers): each wave instruction fills 1 KB of LDS contiguously, and
//    each lane picks the 16-byte granule of HBM that belongs at its LDS
//    position, which is how the LDS layouts below are realised.
//  - The MFMA's k order: in k-step s (of 2 per slice) lane group
//    g = lane >> 4 holds slice k-values 16g + 8s .. 16g + 8s + 7 of its row
//    or column (any k order is valid when both operands use it). Taking
//    16-byte chunk 2g + s rather than 4s + g keeps the two 16-lane groups of
//    each 32-lane half of a ds_read_b128 on different chunks of rows four
//    apart, which share banks: with chunk 4s + g the P reads stalled 4 cycles
//    each on bank conflicts (SQ_LDS_BANK_CONFLICT on MI355X).
//  - P slice: K-contiguous 128-byte rows, 16-byte chunk c of row r stored at
//    c ^ ((r & 7) ^ ((r >> 3) & 1)). B-operand fragment (16 rows x 32 k):
//    one ds_read_b128 per lane (row = lane & 15, chunk 2(lane >> 4) + s).
//  - Q slice: N-contiguous rows as in HBM; granule g of row r stored at
//    (g + rot(r)) mod (BN/8), a row-dependent rotation that spreads the 8
//    rows a 32-lane half of a transposing read touches over distinct banks.
//    A-operand fragment (16 columns x 32 k): two ds_read_b64_tr_b16 per lane;
//    in each 16-lane group lane L addresses k-row 16g + 8s + 4h + (L >> 2) at
//    columns 4(L & 3) .. +3 and receives column L of the 4 rows.
//  - Three LDS stages for P and two for Q (3 x 32 + 2 x 32 KB = 160 KB for a
//    256 x 256 tile), one barrier per slice. Slice kt: k-step 0 (reads the
//    fragments of k-step 1 and issues the P part of slice kt+2 into the P
//    stage of slice kt-1); wait for slice kt+1 and barrier; k-step 1 (reads
//    the first fragments of slice kt+1 and issues the Q part of slice kt+2
//    into the Q stage just released). Fragment reads and DMA instructions are
//    interleaved one by one with the MFMAs. A DMA instruction whose address
//    unit is busy stalls the wave's in-order issue, so splitting a slice's
//    DMA over both k-steps halves the burst each k-step carries.
//  - The main loop has no tail: past the last slice the DMA reloads the last
//    slice into stages that are not read again. Its stage indices cost
//    instructions on the loop's critical path, so they are kept out of it
//    where the slice count allows: six slices per iteration when it is a
//    multiple of 6 (every stage index a constant), two when it is even (the
//    Q stages constants, the P stages from a phase counter kept mod 3), else
//    one (both from a counter kept mod 6, no division); the K-major reads add
//    immediate offsets to one VGPR base per k-step. Six per iteration is not
//    used at 256 x 256, where the compiler then stops keeping the
//    accumulators in place (see launch_one). (Measured on MI355X: a loop
//    whose stage indices were all constants took about 300 of its 2600
//    cycles per slice fewer.)
//  - Rows of P beyond M and columns of Q beyond N are loaded from clamped
//    addresses (their outputs are discarded). When K is not a multiple of 64
//    (KTAIL), the last slice loads k clamped into [k_last, K) and the k >= K
//    part of its LDS stage is cleared after it lands.
//  - Workgroup ids are remapped so the tiles of one XCD share P and Q panels
//    in that XCD's L2.
//
// The backward of the shard needs the other two operand layouts: Q stored
// K-contiguous ([N, K], QT: the transposed weights of dZ = dY·B_iᵀ and
// dX_i = dS·A_iᵀ) and P stored M-contiguous ([K, M], PT: the transposed
// activations of dB_i = Z_iᵀ·dY and dA_i = Xᵀ·dS). Each operand is either
// "K-major" (LDS rows are its m or n index, 128-byte K-contiguous rows,
// fragments by one ds_read_b128, as P above) or "MN-major" (LDS rows are k,
// fragments by two ds_read_b64_tr_b16, as Q above); an MFMA operand fragment
// has the same register layout either way (index lane & 15, k group lane >> 4).
// The GeluGradBf16 epilogue of the backward reads the recomputed S (fp32) and
// writes dS = bf16(acc·GeLU'(S)) and Z = bf16(GeLU(S)).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "tile_engine.hpp"

namespace tpmlp {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;   // k per LDS slice
constexpr int kNSP = 3;   // LDS stages of the P operand
constexpr int kNSQ = 2;   // LDS stages of the Q operand

using namespace engine;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Granule rotation of Q row `row` (GR granules of 16 bytes per row). A
// 32-lane half of a ds_read_b64_tr_b16 reads 2 adjacent granules of rows
// {0,1,2,3, 16,17,18,19} (+ a multiple of 4); with 512- or 256-byte rows
// (GR = 32, 16) every row starts at bank 0, so those rows are spread by
// 32 bytes each; with 384-byte rows (GR = 24) odd rows already start half a
// bank row later, so rows are only spread by 32 bytes per row pair.
template <int GR>
__device__ __forceinline__ int q_rot(int row) {
  if constexpr (GR % 16 == 0) return 2 * (row & 3) + 8 * ((row >> 4) & 1);
  else return 2 * ((row >> 1) & 1) + 4 * ((row >> 4) & 1);
}

// One operand's slice in LDS and its DMA, tail clearing and fragment reads.
// W = tile width of the operand (BM for P, BN for Q); KMAJ: LDS rows are the
// operand's m/n index (128-byte K-contiguous rows), else rows are k (W
// elements each). A stage is W·128 bytes either way.
template <int W, bool KMAJ, bool KTAIL>
struct Operand {
  static constexpr int BK = kBK;
  static constexpr int CH = BK / 8;         // 16-byte chunks per K-major row
  static constexpr int GR = W / 8;          // granules per MN-major row
  static constexpr int G = W * CH;          // granules in a slice
  static constexpr int ROUNDS = G / kThreads;
  static constexpr int BYTES = G * 16;
  static constexpr int READS = KMAJ ? 1 : 2;  // LDS instructions per fragment
  static_assert(G % kThreads == 0, "slices must split over 256 lanes");
  static_assert(KMAJ || GR % 8 == 0, "MN-major rows must hold a multiple of 8 granules");

  const uint16_t* base;
  int64_t ld;
  uint32_t off[ROUNDS];
  uint32_t off_t[KTAIL ? ROUNDS : 1];

  // x0: first m/n of the tile, X: extent of that index; K, k_last: as in the kernel.
  __device__ __forceinline__ void init(const uint16_t* ptr, int64_t ld_, int x0, int X, int K,
                                       int k_last, int wave, int lane) {
    ld = ld_;
    base = KMAJ ? ptr + (int64_t)x0 * ld : ptr + x0;
#pragma unroll
    for (int j = 0; j < ROUNDS; ++j) {
      const int pos = (j * 4 + wave) * 64 + lane;
      if constexpr (KMAJ) {
        const int r = pos / CH, c = swz_p<CH>(r, pos % CH);
        off[j] = (uint32_t)(((int64_t)(min(x0 + r, X - 1) - x0) * ld + c * 8) * 2);
        if constexpr (KTAIL) {
          const int keep = min(c * 8, K - 8 - k_last);
          off_t[j] = off[j] - 2u * (uint32_t)(c * 8 - keep);
        }
      } else {
        const int r = pos / GR, gp = pos % GR;
        const int g = (gp + GR - q_rot<GR>(r)) % GR;  // granule stored at position gp
        off[j] = (uint32_t)(((int64_t)r * ld + min(x0 + g * 8, X - 8) - x0) * 2);
        if constexpr (KTAIL) {
          const int keep = min(r, K - 1 - k_last);
          off_t[j] = off[j] - 2u * (uint32_t)(r - keep) * (uint32_t)ld;
        }
      }
    }
  }
  // DMA instruction j of slice kt into the stage at LDS byte address `stage`
  // (+ the wave's 1 KB lane block, already in `stage`).
  __device__ __forceinline__ void issue(int kt, int last, uint32_t stage, int j) const {
    uint32_t o = off[j];
    if constexpr (KTAIL) o = kt == last ? off_t[j] : o;
    const uint16_t* b = KMAJ ? base + (int64_t)kt * BK : base + (int64_t)kt * BK * ld;
    dma16(b, o, stage + j * 4096);
  }
  // Zero the k >= kvalid part of a stage.
  __device__ __forceinline__ void clear(uint8_t* sp, int kvalid, int t) const {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = t; i < G; i += kThreads) {
      if constexpr (KMAJ) {
        const int r = i / CH, c = i % CH;
        if (c * 8 >= kvalid) *reinterpret_cast<u32x4*>(sp + r * (BK * 2) + swz_p<CH>(r, c) * 16) = z;
      } else {
        if (i / GR >= kvalid) *reinterpret_cast<u32x4*>(sp + i * 16) = z;
      }
    }
  }
};

// Fragment addressing. K-major: `fa` is the fragment's first row fb (a
// multiple of 16), and the lane reads row fb + (lane & 15) at chunk
// 4s + (lane >> 4); as fb is a multiple of 16 the chunk swizzle of that row
// depends on the lane only, so the lane's byte offset is one value per k-step
// plus fb·128 (an immediate once the wave's base is folded in). MN-major:
// `fa` is the byte offset of the lane's first 8-byte piece at k-step 0.
template <int W, bool KMAJ>
__device__ __forceinline__ int frag_addr(int fb, int lane) {
  if constexpr (KMAJ) {
    return fb;
  } else {
    constexpr int GR = W / 8;
    // every k-row a lane reads is 8s + 4h + rsub, whose rotation (bits 0, 1
    // and 4 of the row) equals that of rsub
    const int rsub = 16 * (lane >> 4) + ((lane & 15) >> 2);
    return rsub * (2 * W) + ((((fb + 4 * (lane & 3)) >> 3) + q_rot<GR>(rsub)) % GR) * 16 +
           8 * (lane & 1);
  }
}

// Lane part of a K-major fragment address for k-step s: row lane & 15 of the
// fragment, chunk swz_p(row, 2(lane >> 4) + s).
__device__ __forceinline__ int kmaj_lane_off(int lane, int s) {
  return (lane & 15) * (kBK * 2) + swz_p<kBK / 8>(lane & 15, 2 * (lane >> 4) + s) * 16;
}

// Piece h (of Operand::READS) of the fragment at `fa` (from frag_addr) for
// k-step s of stage sp: K-major, one ds_read_b128; MN-major, k-rows
// 8s + 4h + rsub by a transposing read.
template <int W, bool KMAJ>
__device__ __forceinline__ void read_frag(const uint8_t* sp, int fa, int s, int h, int lane,
                                          s16x8& f) {
  if constexpr (KMAJ) {
    f = *reinterpret_cast<const s16x8*>(sp + fa * (kBK * 2) + kmaj_lane_off(lane, s));
  } else {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(sp + fa + (8 * s + 4 * h) * (2 * W)));
    if (h == 0) f.lo = v; else f.hi = v;
  }
}

// One GEMM problem: C = P·Q with the operands as stored (row strides ldp,
// ldq), C [M, N] with row stride ldc; aux/ldaux and C2 for GeluGradBf16.
struct GemmArgs {
  const uint16_t* P; int64_t ldp; const uint16_t* Q; int64_t ldq; void* C; int64_t ldc;
  const float* aux; int64_t ldaux; void* C2; int M, N, K;
  const uint16_t* bias;  // GeluBiasBf16: bf16 [N], added to every row before GeLU
  uint64_t* stamps;      // measurement only, else NULL: clock stamps per workgroup
};

// Workgroups [0, tiles0) compute problem g0, the rest problem g1 (a launch
// of one problem passes tiles0 = its tile count). Both share the template
// arguments (tile, epilogue, layouts, KTAIL).
template <int BM, int BN, int OUT, bool KTAIL, bool PT, bool QT, int UNR>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(GemmArgs g0, GemmArgs g1,
                                                             int tiles0, int group_m) {
  constexpr int BK = kBK, NSP = kNSP, NSQ = kNSQ;
  constexpr int TM = BM / 2, TN = BN / 2;      // wave tile (2 x 2 waves)
  constexpr int MT = TM / 16, NT = TN / 16;    // 16x16 MFMA tiles per wave
  using OpP = Operand<BM, !PT, KTAIL>;
  using OpQ = Operand<BN, QT, KTAIL>;
  constexpr int P_ROUNDS = OpP::ROUNDS, Q_ROUNDS = OpQ::ROUNDS;
  constexpr int ROUNDS = P_ROUNDS + Q_ROUNDS;  // DMA instructions per wave per slice
  constexpr int P_BYTES = OpP::BYTES, Q_BYTES = OpQ::BYTES;  // one stage of each operand
  constexpr int Q_BASE = NSP * P_BYTES;                      // Q stages follow the P stages
  static_assert(NSP * P_BYTES + NSQ * Q_BYTES <= 163840, "LDS stages");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSP * P_BYTES + NSQ * Q_BYTES];

  int id = xcd_remap(blockIdx.x, gridDim.x);
  const bool second = id >= tiles0;
  const GemmArgs& g = second ? g1 : g0;
  if (second) id -= tiles0;
  const ClockStamp stamp(g.stamps);
  const uint16_t* const P = g.P;
  const uint16_t* const Q = g.Q;
  void* const C = g.C;
  void* const C2 = g.C2;
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
  const int k_last = last * BK;  // first k of the last slice

  // Per-lane byte offsets of the granules this lane copies; rows/columns
  // beyond M or N are clamped, and with KTAIL the last slice's k is clamped
  // into [k_last, K) (the offsets only move down, so they stay non-negative).
  OpP op_p;
  OpQ op_q;
  op_p.init(P, ldp, m0, M, K, k_last, wave, lane);
  op_q.init(Q, ldq, n0, N, K, k_last, wave, lane);
  const uint32_t lds0 = lds_addr(smem) + wave * 1024;

  auto issue_p = [&](int kt, int pst, int j) __attribute__((always_inline)) {
    op_p.issue(kt, last, lds0 + pst * P_BYTES, j);
  };
  auto issue_q = [&](int kt, int qst, int j) __attribute__((always_inline)) {
    op_q.issue(kt, last, lds0 + Q_BASE + qst * Q_BYTES, j);
  };
  // Clear the k >= K part of the last slice's stages (after its DMA landed).
  auto clear_tail = [&]() {
    op_p.clear(smem + (last % NSP) * P_BYTES, K - k_last, t);
    op_q.clear(smem + Q_BASE + (last % NSQ) * Q_BYTES, K - k_last, t);
  };

  // Fragment addressing (in k-step s lane group g = lane >> 4 holds slice
  // k-values 16g + 8s .. 16g + 8s + 7 of its row or column).
  int p_addr[MT], q_addr[NT];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) p_addr[mi] = frag_addr<BM, !PT>(wm * TM + mi * 16, lane);
#pragma unroll
  for (int ni = 0; ni < NT; ++ni) q_addr[ni] = frag_addr<BN, QT>(wn * TN + ni * 16, lane);

  s16x8 afr[2][NT];  // Q fragments (MFMA A operand)
  s16x8 bfr[2][MT];  // P fragments (MFMA B operand)
  constexpr int RQ = OpQ::READS, RP = OpP::READS;
  constexpr int NREADS = NT * RQ + MT * RP;
  // idx-th fragment read of k-step s of the slice in stages (pst, qst) into
  // buffer buf; ordered so that the next k-step's first MFMAs (Q fragment 0
  // with every P fragment) find their operands first.
  // A K-major operand's fragment reads share one VGPR base per k-step: the
  // stage's LDS offset, the wave's first row and the lane's row and chunk;
  // each fragment adds its rows as an immediate offset. (Formed opaquely, so
  // that the compiler does not fold the wave's rows into a per-fragment
  // scalar and re-add it with a VALU op before every read.)
  auto kmaj_base = [&](uint32_t stage_off, int wrow0, int s) __attribute__((always_inline)) {
    uint32_t o = stage_off + (uint32_t)(wrow0 * (kBK * 2) + kmaj_lane_off(lane, s));
    asm("" : "+v"(o));
    return smem + o;
  };
  auto read_one = [&](int pst, int qst, int s, int buf, int idx, const uint8_t* pk,
                      const uint8_t* qk) __attribute__((always_inline)) {
    const uint8_t* sp = smem + pst * P_BYTES;
    const uint8_t* sq = smem + Q_BASE + qst * Q_BYTES;
    auto read_q = [&](int ni, int h) __attribute__((always_inline)) {
      if constexpr (QT) {
        afr[buf][ni] = *reinterpret_cast<const s16x8*>(qk + ni * 16 * (kBK * 2));
      } else {
        read_frag<BN, false>(sq, q_addr[ni], s, h, lane, afr[buf][ni]);
      }
    };
    if (idx < RQ) {
      read_q(0, idx);
    } else if (idx < RQ + MT * RP) {
      const int j = idx - RQ, mi = j / RP;
      if constexpr (!PT) {
        bfr[buf][mi] = *reinterpret_cast<const s16x8*>(pk + mi * 16 * (kBK * 2));
      } else {
        read_frag<BM, false>(sp, p_addr[mi], s, j % RP, lane, bfr[buf][mi]);
      }
    } else {
      const int j = idx - RQ - MT * RP, ni = 1 + j / RQ;
      read_q(ni, j % RQ);
    }
  };
  auto read_bases = [&](int pst, int qst, int s, const uint8_t*& pk, const uint8_t*& qk)
                        __attribute__((always_inline)) {
    pk = PT ? nullptr : kmaj_base(pst * P_BYTES, wm * TM, s);
    qk = QT ? kmaj_base(Q_BASE + qst * Q_BYTES, wn * TN, s) : nullptr;
  };

  f32x4 acc[NT][MT];
#pragma unroll
  for (int ni = 0; ni < NT; ++ni)
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) acc[ni][mi] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // One k-step: the NT x MT MFMAs on buffer `cur`, each followed by its
  // share of the fragment reads for the next k-step (P stage rp, Q stage rq,
  // k-step rs, into cur ^ 1) and of the DMA instructions of one operand of
  // slice dkt (the P part into P stage dst when dq is false, else the Q
  // part into Q stage dst).
  constexpr int NMFMA = NT * MT;
  static_assert(NREADS <= NMFMA && P_ROUNDS <= NMFMA && Q_ROUNDS <= NMFMA,
                "one MFMA slot per read and DMA");
  auto kstep = [&](int cur, int rp, int rq, int rs, bool dq, int dkt, int dst)
                   __attribute__((always_inline)) {
    const uint8_t *pk, *qk;
    read_bases(rp, rq, rs, pk, qk);
#pragma unroll
    for (int i = 0; i < NMFMA; ++i) {
      const int ni = i / MT, mi = i % MT;
      acc[ni][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, afr[cur][ni]), __builtin_bit_cast(bf16x8, bfr[cur][mi]),
          acc[ni][mi], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < NREADS; ++j)
        if (j * NMFMA / NREADS == i) read_one(rp, rq, rs, cur ^ 1, j, pk, qk);
      if (!dq) {
#pragma unroll
        for (int j = 0; j < P_ROUNDS; ++j)
          if (j * NMFMA / P_ROUNDS == i) issue_p(dkt, dst, j);
      } else {
#pragma unroll
        for (int j = 0; j < Q_ROUNDS; ++j)
          if (j * NMFMA / Q_ROUNDS == i) issue_q(dkt, dst, j);
      }
      SCHED_PIN();
    }
  };

  // Prologue: slices 0 and 1 into P stages 0, 1 and Q stages 0, 1 (slice
  // indices past the end are clamped to the last slice: a reload into a
  // stage whose contents are never used); wait for slice 0.
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
  {
    const uint8_t *pk, *qk;
    read_bases(0, 0, 0, pk, qk);
#pragma unroll
    for (int i = 0; i < NREADS; ++i) read_one(0, 0, 0, 0, i, pk, qk);
  }

  // Slice kt lives in P stage kt % 3 and Q stage kt % 2. Its fragments are
  // all read by the end of its first k-step. The P part of slice kt+2 is
  // copied during the first k-step, into the P stage of slice kt-1 (free
  // since the previous iteration's barrier); the Q part during the second
  // k-step, into the Q stage of slice kt (free once this iteration's barrier
  // has passed). So each k-step carries half of a slice's DMA instructions.
  // Near the end the DMA reloads the last slice into stages that are never
  // read again.
  auto slice = [&](int kt, int ps, int qs) __attribute__((always_inline)) {
    const int ps1 = ps == 2 ? 0 : ps + 1, ps2 = ps == 0 ? 2 : ps - 1;
    kstep(0, ps, qs, 1, false, min(kt + 2, last), ps2);
    waitcnt<P_ROUNDS, 0>();  // slice kt+1 has landed (only the P part of kt+2 may be in flight)
    barrier();               // every wave is done reading the stages of slice kt
    if (KTAIL && kt + 2 == ktiles) {
      clear_tail();
      waitcnt<63, 0>();
      barrier();
    }
    kstep(1, ps1, qs ^ 1, 0, true, min(kt + 2, last), qs);
  };
  if constexpr (UNR == 6) {
    // Six slices per iteration (ktiles is a multiple of 6): every stage
    // index of every read and DMA is a constant.
    for (int kt = 0; kt < ktiles; kt += 6) {
#pragma unroll
      for (int u = 0; u < 6; ++u) slice(kt + u, u % 3, u & 1);
    }
  } else if constexpr (UNR == 2) {
    // Two slices per iteration (ktiles is even), so that the Q stage of
    // every read and DMA is a constant; ph = kt % 3.
    int ph = 0;
    for (int kt = 0; kt < ktiles; kt += 2) {
      slice(kt, ph, 0);
      slice(kt + 1, ph == 2 ? 0 : ph + 1, 1);
      ph = ph == 0 ? 2 : ph - 1;
    }
  } else {
    int ph = 0;  // kt % 6
    for (int kt = 0; kt < ktiles; ++kt) {
      slice(kt, ph >= 3 ? ph - 3 : ph, ph & 1);
      ph = ph == 5 ? 0 : ph + 1;
    }
  }
  waitcnt<0, 0>();  // no DMA may still write LDS when the workgroup ends

  // Epilogue. Lane holds, for 16x16 tile (ni, mi), C[m][n .. n+3] with
  // m = mi·16 + (lane & 15), n = ni·16 + 4·(lane >> 4) (wave-tile relative).
  // Element offsets are a per-lane base (tile (0, 0)) plus the wave-uniform
  // 16·mi rows and 16·ni columns (row strides are below 2^23, so the latter
  // fits 32 bits); a tile is stored where its row and column are inside.
  // Tiles go out row block by row block (mi outer, ni inner), so the pieces
  // of each 128-byte line of C come from consecutive store instructions:
  // with the column groups outer, lines reached HBM in parts (WRITE_SIZE
  // 1.26-1.77 times the output bytes with 256x192 tiles, measured on MI355X;
  // exactly the output bytes in this order, and the GEMMs 2-3% faster).
  const int mrow = m0 + wm * TM + (lane & 15), ncol = n0 + wn * TN + 4 * (lane >> 4);
  const int rows_left = M - mrow, cols_left = N - ncol;
  const int64_t c_lane = (int64_t)mrow * ldc + ncol;
  auto c_off = [&](int mi, int ni) __attribute__((always_inline)) {
    return c_lane + (int)(16 * mi * ldc + 16 * ni);
  };
  auto inside = [&](int mi, int ni) __attribute__((always_inline)) {
    return 16 * mi < rows_left && 16 * ni < cols_left;
  };
  if constexpr (OUT == (int)OutKind::GeluGradBf16) {
    // dS = bf16(dZ·GeLU'(S)) into C, Z = bf16(GeLU(S)) into C2. The S values
    // of EB tiles are loaded together, LA batches ahead of the batch being
    // computed, so their latency hides under the GeLU work of one wave per
    // SIMD. Loads are clamped to the last row and column group (no branch).
    constexpr int EB = 8, NB = NT * MT / EB, LA = 2;
    static_assert((NT * MT) % EB == 0, "epilogue batches");
    const int row_max = M - 1 - mrow, col_max = N - 4 - ncol;
    const float* aux_lane = aux + (int64_t)mrow * ldaux + ncol;
    f32x4 sv[LA + 1][EB];
    const GeluRegs gk = gelu_regs();
    auto load_batch = [&](int b, int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < EB; ++e) {
        const int mi = (b * EB + e) / NT, ni = (b * EB + e) % NT;
        const int r = min(16 * mi, row_max), c = min(16 * ni, col_max);
        sv[buf][e] = *reinterpret_cast<const f32x4*>(aux_lane + ((int64_t)r * (int)ldaux + c));
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
          const f32x4 x = sv[b % (LA + 1)][e];
          float gl[4], dg[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) gelu_and_grad(x[q], gl[q], dg[q], gk);
          if (!decltype(checked)::value || inside(mi, ni)) {
            const int64_t o = c_off(mi, ni);
            const u32x2 d2 = {pack_bf16x2(v[0] * dg[0], v[1] * dg[1]),
                              pack_bf16x2(v[2] * dg[2], v[3] * dg[3])};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(C) + o) = d2;
            const u32x2 z = {pack_bf16x2(gl[0], gl[1]), pack_bf16x2(gl[2], gl[3])};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(C2) + o) = z;
          }
        }
      }
    };
    if (M - m0 >= BM && N - n0 >= BN) run(std::false_type{});
    else run(std::true_type{});
    stamp.finish(g.stamps);
    return;
  }
  // GeluBiasBf16: the bias of the lane's four columns in each 16-column
  // group, loaded once per tile from a column clamped into [0, N - 4] (N is
  // a multiple of 8 and ncol of 4, so the load is whole and 8-byte aligned;
  // a clamped group is never stored).
  // Kept as packed bf16 pairs and widened where used.
  [[maybe_unused]] u32x2 bias2[NT];
  if constexpr (OUT == (int)OutKind::GeluBiasBf16 || OUT == (int)OutKind::F32Bias) {
    const int col_max = N - 4 - ncol;
#pragma unroll
    for (int ni = 0; ni < NT; ++ni)
      bias2[ni] = *reinterpret_cast<const u32x2*>(g.bias + ncol + min(16 * ni, col_max));
  }
  [[maybe_unused]] const GeluRegs gk = gelu_regs();
  // Every store of a tile wholly inside C takes the path without the
  // per-tile row and column checks (the checks cost each 16x16 tile a few
  // scalar instructions and two branches).
  auto store_all = [&](auto checked) __attribute__((always_inline)) {
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) {
        if (decltype(checked)::value && !inside(mi, ni)) continue;
        const int64_t o = c_off(mi, ni);
        f32x4 v = acc[ni][mi];
        // Read the accumulator into VGPRs here, as the GeLU epilogue does; a
        // store straight from AGPRs lets the register allocator split the
        // accumulators between the two files and copy them inside the loop.
        asm volatile("" : "+v"(v));
        if constexpr (OUT == (int)OutKind::F32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(C) + o) = v;
        } else if constexpr (OUT == (int)OutKind::F32Bias) {
          const u32x2 w = bias2[ni];
          const f32x4 b = {__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xFFFF0000u),
                           __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xFFFF0000u)};
          *reinterpret_cast<f32x4*>(static_cast<float*>(C) + o) = v + b;
        } else if constexpr (OUT == (int)OutKind::GeluBf16) {
          const u32x2 g = {pack_bf16x2(gelu_exact(v[0], gk), gelu_exact(v[1], gk)),
                           pack_bf16x2(gelu_exact(v[2], gk), gelu_exact(v[3], gk))};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(C) + o) = g;
        } else if constexpr (OUT == (int)OutKind::GeluBiasBf16) {
          const u32x2 w = bias2[ni];
          const f32x4 b = {__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xFFFF0000u),
                           __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xFFFF0000u)};
          const u32x2 g = {pack_bf16x2(gelu_exact(v[0] + b[0], gk), gelu_exact(v[1] + b[1], gk)),
                           pack_bf16x2(gelu_exact(v[2] + b[2], gk), gelu_exact(v[3] + b[3], gk))};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(C) + o) = g;
        } else {
          const u32x2 g = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(C) + o) = g;
        }
      }
    }
  };
  if (M - m0 >= BM && N - n0 >= BN) store_all(std::false_type{});
  else store_all(std::true_type{});
  stamp.finish(g.stamps);
}

template <int BM, int BN>
int tile_count(const GemmArgs& a) {
  return ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
}

// One launch over problems a[0 .. n) (n = 1 or 2).
// The main loop takes six slices per iteration when every problem of the
// launch has a multiple of 6 slices, two when they are even, else one. Not
// six at 256 x 256, nor two or six with the M-major P operand, nor at
// 256 x 256 with a K tail: there the compiler no longer keeps the
// accumulators in place (it moves them through VGPRs inside the loop, or
// spills).
template <int BM, int BN, int OUT, bool KTAIL, bool PT, bool QT>
hipError_t launch_one(const GemmArgs* a, int n, hipStream_t stream) {
  const int t0 = tile_count<BM, BN>(a[0]);
  const int tiles = t0 + (n > 1 ? tile_count<BM, BN>(a[1]) : 0);
  const int group_m = 4;
  const GemmArgs& a1 = n > 1 ? a[1] : a[0];
  const int s0 = (a[0].K + kBK - 1) / kBK, s1 = (a1.K + kBK - 1) / kBK;
  constexpr bool big = BM == 256 && BN == 256;
  if constexpr (!PT && !big) {
    if (s0 % 6 == 0 && s1 % 6 == 0) {
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, OUT, KTAIL, PT, QT, 6>), dim3(tiles),
                         dim3(kThreads), 0, stream, a[0], a1, t0, group_m);
      return hipGetLastError();
    }
  }
  if constexpr (!PT && !(KTAIL && big)) {
    if (s0 % 2 == 0 && s1 % 2 == 0) {
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, OUT, KTAIL, PT, QT, 2>), dim3(tiles),
                         dim3(kThreads), 0, stream, a[0], a1, t0, group_m);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, OUT, KTAIL, PT, QT, 1>), dim3(tiles),
                     dim3(kThreads), 0, stream, a[0], a1, t0, group_m);
  return hipGetLastError();
}

// The (layout, epilogue) combinations the path uses: the forward's
// K-major P / N-major Q with GeLU (with or without a bias), fp32 (with or
// without a bias: the backward's recomputed S) or bf16 output; K-major Q with the same four (the forward with weights stored
// transposed) or the GeLU-gradient epilogue; M-major P with fp32 output.
template <int BM, int BN, bool KTAIL>
hipError_t launch_cfg(const GemmArgs* a, int n, OutKind out, Layout lay, hipStream_t stream) {
  if (lay == Layout::NN) {
    switch (out) {
      case OutKind::GeluBf16: return launch_one<BM, BN, (int)OutKind::GeluBf16, KTAIL, false, false>(a, n, stream);
      case OutKind::F32: return launch_one<BM, BN, (int)OutKind::F32, KTAIL, false, false>(a, n, stream);
      case OutKind::Bf16: return launch_one<BM, BN, (int)OutKind::Bf16, KTAIL, false, false>(a, n, stream);
      case OutKind::GeluBiasBf16: return launch_one<BM, BN, (int)OutKind::GeluBiasBf16, KTAIL, false, false>(a, n, stream);
      case OutKind::F32Bias: return launch_one<BM, BN, (int)OutKind::F32Bias, KTAIL, false, false>(a, n, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (lay == Layout::QT) {
    switch (out) {
      case OutKind::GeluGradBf16: return launch_one<BM, BN, (int)OutKind::GeluGradBf16, KTAIL, false, true>(a, n, stream);
      case OutKind::F32: return launch_one<BM, BN, (int)OutKind::F32, KTAIL, false, true>(a, n, stream);
      case OutKind::GeluBf16: return launch_one<BM, BN, (int)OutKind::GeluBf16, KTAIL, false, true>(a, n, stream);
      case OutKind::Bf16: return launch_one<BM, BN, (int)OutKind::Bf16, KTAIL, false, true>(a, n, stream);
      case OutKind::GeluBiasBf16: return launch_one<BM, BN, (int)OutKind::GeluBiasBf16, KTAIL, false, true>(a, n, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (out == OutKind::F32) return launch_one<BM, BN, (int)OutKind::F32, KTAIL, true, false>(a, n, stream);
  return hipErrorInvalidValue;
}

template <int BM, int BN>
hipError_t launch_tile(const GemmArgs* a, int n, OutKind out, Layout lay, hipStream_t stream) {
  bool tail = false;
  for (int i = 0; i < n; ++i) tail = tail || a[i].K % kBK != 0;
  if (!tail) return launch_cfg<BM, BN, false>(a, n, out, lay, stream);
  return launch_cfg<BM, BN, true>(a, n, out, lay, stream);
}

struct TileChoice { int bm, bn; };

// Pick the tile shape with the best estimated time: waves of 256 CUs times a
// per-tile time relative to a 256x256 tile, measured on MI355X (smaller
// tiles reuse each LDS byte less, so their cost falls slower than their area).
// 128x192 is for GEMMs whose short N leaves the other shapes too few tiles
// (GPT-2-small's row GEMM, 8192 x 768: 256 tiles, 40 us against 45 us with
// 128x128); its entry sits between the bounds measured on MI355X, below the
// 0.6 at which it would lose there and above the 0.43 at which it would
// displace 256x192 on the 175B-class GEMMs, where it is 40-50% slower.
TileChoice choose_tile(const GemmArgs* a, int n) {
  static const struct { int bm, bn; double cost; } cands[] = {
      {256, 256, 1.00}, {256, 192, 0.85}, {256, 128, 0.62}, {128, 192, 0.55}, {128, 128, 0.30},
  };
  constexpr int kCus = 256;
  int obm, obn;
  if (tile_override(obm, obn))
    for (const auto& c : cands)
      if (c.bm == obm && c.bn == obn) return {obm, obn};
  double best = 1e300;
  TileChoice choice{256, 256};
  for (const auto& c : cands) {
    long tiles = 0;
    for (int i = 0; i < n; ++i)
      tiles += (long)((a[i].M + c.bm - 1) / c.bm) * ((a[i].N + c.bn - 1) / c.bn);
    const long waves = (tiles + kCus - 1) / kCus;
    const double est = waves * c.cost;
    if (est < best - 1e-9) { best = est; choice = {c.bm, c.bn}; }
  }
  return choice;
}

hipError_t launch_group(const GemmArgs* a, int n, OutKind out, Layout lay, hipStream_t stream) {
  const TileChoice tc = choose_tile(a, n);
  if (tc.bm == 256 && tc.bn == 256) return launch_tile<256, 256>(a, n, out, lay, stream);
  if (tc.bm == 256 && tc.bn == 192) return launch_tile<256, 192>(a, n, out, lay, stream);
  if (tc.bm == 256 && tc.bn == 128) return launch_tile<256, 128>(a, n, out, lay, stream);
  if (tc.bm == 128 && tc.bn == 192) return launch_tile<128, 192>(a, n, out, lay, stream);
  return launch_tile<128, 128>(a, n, out, lay, stream);
}

}  // namespace

hipError_t launch_gemm_bf16_ex(const uint16_t* P, int64_t ldp, const uint16_t* Q, int64_t ldq,
                               void* C, int64_t ldc, int M, int N, int K, OutKind out, Layout lay,
                               const float* aux, int64_t ldaux, void* C2, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const GemmArgs a{P, ldp, Q, ldq, C, ldc, aux, ldaux, C2, M, N, K};
  return launch_group(&a, 1, out, lay, stream);
}

hipError_t launch_gemm_bf16_bias(const uint16_t* P, int64_t ldp, const uint16_t* Q, int64_t ldq,
                                 const uint16_t* bias, void* C, int64_t ldc, int M, int N, int K,
                                 OutKind out, Layout lay, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const bool ok = (out == OutKind::GeluBiasBf16 && (lay == Layout::NN || lay == Layout::QT)) ||
                  (out == OutKind::F32Bias && lay == Layout::NN);
  if (!ok) return hipErrorInvalidValue;
  GemmArgs a{P, ldp, Q, ldq, C, ldc, nullptr, 0, nullptr, M, N, K};
  a.bias = bias;
  return launch_group(&a, 1, out, lay, stream);
}

hipError_t launch_gemm_bf16_pair(const BfGemm& x, const BfGemm& y, OutKind out, Layout lay,
                                 hipStream_t stream) {
  GemmArgs a[2];
  int n = 0;
  for (const BfGemm* g : {&x, &y})
    if (g->M > 0 && g->N > 0)
      a[n++] = GemmArgs{g->P, g->ldp, g->Q, g->ldq, g->C, g->ldc, nullptr, 0, nullptr, g->M, g->N,
                        g->K};
  if (n == 0) return hipSuccess;
  return launch_group(a, n, out, lay, stream);
}

hipError_t launch_gemm_bf16(const uint16_t* P, int64_t ldp, const uint16_t* Q, int64_t ldq,
                            void* C, int64_t ldc, int M, int N, int K, OutKind out,
                            hipStream_t stream, uint64_t* stamps) {
  if (M == 0 || N == 0) return hipSuccess;
  GemmArgs a{P, ldp, Q, ldq, C, ldc, nullptr, 0, nullptr, M, N, K};
  a.stamps = stamps;
  return launch_group(&a, 1, out, Layout::NN, stream);
}

}  // namespace tpmlp
