// Per-head attention of one tensor-parallel rank on gfx950 (flash-attention
// style forward: scores, online softmax and the weighted sum of values per
// block of keys, with nothing but the output written to HBM).
//
// Each rank owns whole heads and computes their attention with no exchange
// ("Megatron-LM" glossary, tensor-parallel section; "Megatron architecture
// and 6D parallel guide", §3.2: 32 heads at TP=8 give 4 per GPU). For
// sequence b and head j: O = softmax(Q·Kᵀ/√dh, causal mask)·V.
//
// Layout. QKV [B·S, ld] bf16 (row b·S + t = token t of sequence b); local
// head j's query, key and value columns are [3j·dh, 3j·dh + dh),
// [.. + dh, .. + 2dh), [.. + 2dh, .. + 3dh). O [B·S, ldo] bf16, head j at
// columns [j·dh, (j+1)·dh). dh = 128.
//
// Workgroup = one head of one sequence and 128 queries, as SPLIT
// groups of 128/(16·MT) waves; a wave owns 16·MT queries. The groups split the
// key blocks (64 keys each) round-robin, each double-buffering its own blocks
// in LDS by global_load_lds_dwordx4 (K 16 KB + V 16 KB per stage), and merge
// their partial results through LDS at the end. The shipped configuration is
// MT = 1, SPLIT = 2 (16 waves, 4 per SIMD): the softmax is VALU work that only
// other waves' MFMAs and LDS reads can hide, and splitting the keys halves
// the longest workgroup's chain. Under the causal mask a workgroup holds two
// blocks of 64 queries, an early and a late one (block p and block n-1-p of
// the n in the sequence), so all workgroups have the same number of query-key
// block pairs.
//
//  - Scores: D = K·Qᵀ with v_mfma_f32_16x16x32_bf16 (A = 16 keys x 32 dh of
//    K, B = 32 dh x 16 queries of Q, the Q fragments held in registers for
//    the whole kernel). A lane then holds, for its query (lane & 15), 4 keys
//    of each 16-key tile. The K fragment rows are permuted: row i of key
//    tile nt is key 32·(nt/2) + 8·(i/4) + 4·(nt%2) + i%4, so that across the
//    tile pair (2c, 2c+1) lane group g = lane >> 4 holds keys
//    32c + 8g .. 32c + 8g + 7, exactly the k slots of an MFMA B operand.
//  - Softmax in the exp2 domain on the fp32 scores, online over key blocks
//    (running max per query row reduced over the 4 lane groups with the
//    gfx950 lane swaps, raised lazily; the running sum kept per lane and
//    reduced once at the end).
//  - P·V: D = V'·P' with A = 16 dh x 32 keys of V (two transposing
//    ds_read_b64_tr_b16 per lane from V rows stored as in HBM, granules
//    rotated per row as in the GEMM engine's N-major operand) and B = the
//    bf16-rounded probabilities straight from the score registers.
//  - K rows (256 bytes, 16 chunks) store chunk c of key row r at position
//    c ^ f(r), f(r) = (r & 3) | ((r >> 3) & 1) << 2 | ((r >> 4) & 1) << 3;
//    for the permuted rows a 16-lane group reads, f(row) = lane & 15, so the
//    16 reads of a group fall on 16 distinct 16-byte bank groups.
#include "common.hpp"
#include "kernels.hpp"
#include "tile_engine.hpp"

namespace tpmlp {
namespace {

using namespace engine;

constexpr int kDh = 128;       // head width
constexpr int kBQ = 128;       // queries per workgroup
constexpr int kBKV = 64;       // keys per block
constexpr int kRowBytes = kDh * 2;                 // one K or V row in LDS
constexpr int kStageBytes = kBKV * kRowBytes;      // 16 KB
constexpr int kGranules = kStageBytes / 16;        // 1024 per K or V stage
constexpr float kLazy = 8.0f;  // log2-domain headroom before the running max is raised

constexpr int kMT = 1;     // 16-row query tiles per wave
constexpr int kSplit = 2;  // key-block groups per workgroup

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ int k_swz(int r) {
  return (r & 3) | (((r >> 3) & 1) << 2) | (((r >> 4) & 1) << 3);
}

// Granule rotation of V row r (16 granules per row), as the GEMM engine's
// N-major operand with 256-byte rows.
__device__ __forceinline__ int v_rot(int r) { return 2 * (r & 3) + 8 * ((r >> 3) & 1); }

// Max / sum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups
// holding one query row), with the gfx950 lane-swap instructions: swapping a
// register with itself across 32-lane (16-lane) halves hands every lane the
// value of lane l ^ 32 (l ^ 16) in one of the two results.
__device__ __forceinline__ float xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                                  __builtin_bit_cast(uint32_t, v), false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ float xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                                  __builtin_bit_cast(uint32_t, v), false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 16) ? r[0] : r[1]);
}

__device__ __forceinline__ float wave_max4(float v) {
  v = fmaxf(v, xor16(v));
  return fmaxf(v, xor32(v));
}

__device__ __forceinline__ float wave_sum4(float v) {
  v += xor16(v);
  return v + xor32(v);
}

// MT: 16-row query tiles per wave. SPLIT: groups of kBQ / (16·MT) waves that
// each take every SPLIT-th key block of the same queries (group h the blocks
// kb ≡ h mod SPLIT, in its own LDS stages); their partial results are merged
// through LDS at the end.
template <bool CAUSAL, int MT, int SPLIT>
__global__ __launch_bounds__(64 * SPLIT * kBQ / (16 * MT)) void attn_fwd_kernel(
    const uint16_t* __restrict__ QKV, int64_t ld, uint16_t* __restrict__ O, int64_t ldo, int B,
    int S, int heads, float scale_log2) {
  constexpr int kWaves = kBQ / (16 * MT);        // waves per group
  constexpr int kThreads = 64 * kWaves;          // threads per group
  constexpr int kRounds = kGranules / kThreads;  // DMA instructions per wave per K or V block
  constexpr int kRows = 16 * MT;                 // queries per wave
  // K stages (group h, buffer st) at (2h + st)·16 KB, V stages after all K stages
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * SPLIT * kStageBytes];

  const int bh_count = B * heads;
  const int bid = blockIdx.x;
  const int bh = bid % bh_count;
  const int b = bh / heads, j = bh % heads;

  const int lane = threadIdx.x & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave_all / kWaves;             // key-block group
  const int wave = wave_all % kWaves;            // wave within the group (its query rows)
  const int g = lane >> 4, L = lane & 15;

  const uint16_t* seq = QKV + (int64_t)b * S * ld;   // row 0 of the sequence
  const int qcol = 3 * j * kDh, kcol = qcol + kDh, vcol = qcol + 2 * kDh;
  // q0w: first query of this wave (S for a wave with no queries); last_q: the
  // workgroup's last query. Without the mask a workgroup is kBQ consecutive
  // queries. With it, query block h (of kBQ/2) needs h+1 key blocks, so
  // workgroup p pairs block p (first half of each group's waves) with block
  // nhb-1-p (second half): every workgroup then has about the same work, and
  // the kernel no longer waits on the one that holds the last queries.
  int q0w, last_q;
  if constexpr (CAUSAL) {
    constexpr int kHalf = kBQ / 2;
    static_assert(kRows * (kWaves / 2) == kHalf, "half of a group's waves hold one block");
    const int nhb = (S + kHalf - 1) / kHalf, p = bid / bh_count;
    const int hb = nhb - 1 - p;                      // the later block; hb == p: none
    const bool first = wave < kWaves / 2;
    const int q0 = (first ? p : hb) * kHalf + kRows * (wave % (kWaves / 2));
    q0w = (first || hb > p) ? q0 : S;
    last_q = min(S - 1, max(p, hb) * kHalf + kHalf - 1);
  } else {
    const int qb = bid / bh_count;
    q0w = qb * kBQ + kRows * wave;
    last_q = min(S - 1, qb * kBQ + kBQ - 1);
  }
  const bool idle = q0w >= S;

  // Q fragments: query q0w + 16mi + L, dh 32s + 8g .. +7 (clamped rows beyond S).
  s16x8 qf[MT][4];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) {
    const int q = min(q0w + 16 * mi + L, S - 1);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qf[mi][s] = *reinterpret_cast<const s16x8*>(seq + (int64_t)q * ld + qcol + 32 * s + 8 * g);
  }

  const int last_key = CAUSAL ? last_q : S - 1;
  const int nkb = last_key / kBKV + 1;

  // DMA of key block kb into the group's buffer st: granule
  // pos = (round·waves + wave)·64 + lane.
  const uint32_t lds0 = lds_addr(smem) + wave * 1024;
  const int kst0 = 2 * grp, vst0 = 2 * SPLIT + 2 * grp;  // the group's first K and V stage
  auto issue = [&](int kb, int st) {
    const int kv0 = kb * kBKV;
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int pos = (r * kWaves + wave) * 64 + lane;
      const int row = pos >> 4, p = pos & 15;
      const int key = min(kv0 + row, S - 1);
      const uint32_t kc = (uint32_t)(((int64_t)key * ld + kcol + (p ^ k_swz(row)) * 8) * 2);
      const uint32_t vc =
          (uint32_t)(((int64_t)key * ld + vcol + ((p + 16 - v_rot(row)) & 15) * 8) * 2);
      dma16(seq, kc, lds0 + (kst0 + st) * kStageBytes + r * kThreads * 16);
      dma16(seq, vc, lds0 + (vst0 + st) * kStageBytes + r * kThreads * 16);
    }
  };

  // Fragment addressing (lane parts).
  // K: row 8·(L>>2) + (L&3) (+ 32c + 4e per tile), chunk (4s + g) ^ L.
  const int k_row = 8 * (L >> 2) + (L & 3);
  // V: as the GEMM engine's A operand from an N-major stage of 128 columns.
  const int rsub = 8 * g + (L >> 2);
  int v_addr[8];
#pragma unroll
  for (int nd = 0; nd < 8; ++nd)
    v_addr[nd] = rsub * kRowBytes + ((((16 * nd + 4 * (lane & 3)) >> 3) + v_rot(rsub)) & 15) * 16 +
                 8 * (lane & 1);

  f32x4 o[8][MT];
  float m_run[MT], l_run[MT];  // running max (log2 domain) and this lane's running sum
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
    for (int nd = 0; nd < 8; ++nd) o[nd][mi] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[mi] = -INFINITY;
    l_run[mi] = 0.f;
  }

  if (grp < nkb) issue(grp, 0);
  const int iters = (nkb + SPLIT - 1) / SPLIT;
  for (int it = 0; it < iters; ++it) {
    const int st = it & 1;
    const int kb = it * SPLIT + grp;
    waitcnt<0, 0>();
    barrier();  // block kb is in LDS; every wave is done with the group's previous block
    if (kb + SPLIT < nkb) issue(kb + SPLIT, st ^ 1);
    const int kv0 = kb * kBKV;
    // no queries, past the last block, or (causal) every query of the wave
    // precedes the block
    if (idle || kb >= nkb || (CAUSAL && kv0 > q0w + kRows - 1)) continue;

    const uint8_t* sk = smem + (kst0 + st) * kStageBytes;
    const uint8_t* sv = smem + (vst0 + st) * kStageBytes;
    // scores
    f32x4 sc[4][MT];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) sc[nt][mi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int row = k_row + 32 * (nt >> 1) + 4 * (nt & 1);
        const s16x8 kf =
            *reinterpret_cast<const s16x8*>(sk + row * kRowBytes + (((4 * s + g) ^ L) * 16));
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
          sc[nt][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, kf), __builtin_bit_cast(bf16x8, qf[mi][s]), sc[nt][mi],
              0, 0, 0);
      }
    }

    // Mask (diagonal blocks and the ragged tail only; a wave-uniform branch):
    // element (nt, r) of row mi is key kv0 + 8g + 32(nt/2) + 4(nt%2) + r, and
    // visible keys are <= min(query, S - 1).
    if ((CAUSAL && kv0 + kBKV - 1 > q0w) || kv0 + kBKV > S) {
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        const int q = q0w + 16 * mi + L;
        const int lim = (CAUSAL ? min(q, S - 1) : S - 1) - kv0 - 8 * g;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (32 * (nt >> 1) + 4 * (nt & 1) + r > lim) sc[nt][mi][r] = -INFINITY;
      }
    }

    // online softmax. The running max m (log2 domain) is raised lazily: only
    // when some row's block max exceeds it by more than kLazy are O and the
    // sums rescaled, so the probabilities exp2(s·c − m) stay below 2^kLazy
    // and most blocks cost one FMA, one exp2 and one add per score.
    s16x8 pf[MT][2];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      float mx = -INFINITY;  // the scale is positive: take the max of the raw scores
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[nt][mi][r]);
      mx = wave_max4(mx) * scale_log2;
      if (__any(mx > m_run[mi] + kLazy)) {
        const float m_new = fmaxf(m_run[mi], mx);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[mi] - m_new);
        l_run[mi] *= alpha;
#pragma unroll
        for (int nd = 0; nd < 8; ++nd) o[nd][mi] *= alpha;
        m_run[mi] = m_new;
      }
      const float neg_m = m_run[mi] == -INFINITY ? 0.f : -m_run[mi];
      float ls = 0.f;
      uint32_t pk[4][2];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        float pv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pv[r] = __builtin_amdgcn_exp2f(fmaf(sc[nt][mi][r], scale_log2, neg_m));
          ls += pv[r];
        }
        pk[nt][0] = pack_bf16x2(pv[0], pv[1]);
        pk[nt][1] = pack_bf16x2(pv[2], pv[3]);
      }
      l_run[mi] += ls;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const u32x4 w = {pk[2 * c][0], pk[2 * c][1], pk[2 * c + 1][0], pk[2 * c + 1][1]};
        pf[mi][c] = __builtin_bit_cast(s16x8, w);
      }
    }

    // O += P·V
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int nd = 0; nd < 8; ++nd) {
        s16x8 vf;
        vf.lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(sv + v_addr[nd] + (32 * c) * kRowBytes));
        vf.hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(sv + v_addr[nd] + (32 * c + 4) * kRowBytes));
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
          o[nd][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, vf), __builtin_bit_cast(bf16x8, pf[mi][c]), o[nd][mi],
              0, 0, 0);
      }
    }
  }
  waitcnt<0, 0>();

  if constexpr (SPLIT == 2) {
    // Group 1 hands its running max, partial sums and unnormalised O to the
    // group-0 wave with the same queries (same lane, same elements), which
    // rescales both to the common max and adds them.
    constexpr int kE = 8 * MT * 4 + 2 * MT;  // floats per lane
    static_assert(kE * kThreads * 4 <= 4 * SPLIT * kStageBytes, "merge buffer");
    float* xch = reinterpret_cast<float*>(smem);
    const int slot = wave * 64 + lane;
    barrier();  // every wave is done reading the stages
    if (grp == 1) {
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
        for (int nd = 0; nd < 8; ++nd)
#pragma unroll
          for (int r = 0; r < 4; ++r) xch[((mi * 8 + nd) * 4 + r) * kThreads + slot] = o[nd][mi][r];
        xch[(32 * MT + 2 * mi) * kThreads + slot] = m_run[mi];
        xch[(32 * MT + 2 * mi + 1) * kThreads + slot] = l_run[mi];
      }
    }
    barrier();
    if (grp == 1) return;
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      const float m1 = xch[(32 * MT + 2 * mi) * kThreads + slot];
      const float l1 = xch[(32 * MT + 2 * mi + 1) * kThreads + slot];
      const float m = fmaxf(m_run[mi], m1);
      const float mu = m == -INFINITY ? 0.f : m;
      const float a0 = __builtin_amdgcn_exp2f(m_run[mi] - mu);
      const float a1 = __builtin_amdgcn_exp2f(m1 - mu);
      l_run[mi] = l_run[mi] * a0 + l1 * a1;
#pragma unroll
      for (int nd = 0; nd < 8; ++nd)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          o[nd][mi][r] = o[nd][mi][r] * a0 + xch[((mi * 8 + nd) * 4 + r) * kThreads + slot] * a1;
    }
  }

  // O = acc / l; lane holds O[query q][dh 16nd + 4g .. +3]
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) {
    const int q = q0w + 16 * mi + L;
    const float inv = 1.0f / wave_sum4(l_run[mi]);
    if (q >= S) continue;
    uint16_t* orow = O + ((int64_t)b * S + q) * ldo + j * kDh;
#pragma unroll
    for (int nd = 0; nd < 8; ++nd) {
      const f32x4 v = o[nd][mi] * inv;
      const u32x2 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      *reinterpret_cast<u32x2*>(orow + 16 * nd + 4 * g) = w;
    }
  }
}

}  // namespace

hipError_t launch_attention(const uint16_t* QKV, int64_t ld, uint16_t* O, int64_t ldo, int B,
                            int S, int heads, bool causal, hipStream_t stream) {
  if (B == 0 || S == 0 || heads == 0) return hipSuccess;
  const int nqb = (S + kBQ - 1) / kBQ;
  const dim3 grid(nqb * B * heads);
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)kDh);
  constexpr int MT = kMT, SPLIT = kSplit;
  const dim3 block(64 * SPLIT * kBQ / (16 * MT));
  if (causal)
    hipLaunchKernelGGL((attn_fwd_kernel<true, MT, SPLIT>), grid, block, 0, stream, QKV, ld, O, ldo,
                       B, S, heads, scale_log2);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<false, MT, SPLIT>), grid, block, 0, stream, QKV, ld, O,
                       ldo, B, S, heads, scale_log2);
  return hipGetLastError();
}

}  // namespace tpmlp
