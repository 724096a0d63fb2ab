// bf16 MFMA GEMMs of the tensor-parallel MLP shard on gfx950.
//
//   column-parallel step:  Z_i = bf16(GeLU(X·A_i))      (GeLU fused in the epilogue)
//   row-parallel step:     Y_i = Z_i·B_i                 (fp32 or bf16 partial)
//
// ("Megatron-LM deep architecture", column/row-parallel section.) Both are
// C = P·Q with P [M, K] K-contiguous (X or Z_i) and Q [K, N] N-contiguous
// (A_i or B_i in the pages' math layout), so one tile engine serves both.
//
// Tile engine (one workgroup = 4 waves = 256 threads, one tile BM x BN):
//  - k advances in slices of BK = 64 (128 bytes of bf16 per LDS row).
//  - P slices are copied HBM -> registers -> LDS with 128-bit loads/stores,
//    stored K-contiguous. Q slices are loaded as 8x8 (k x n) blocks with
//    128-bit loads, transposed in registers, and stored K-contiguous, so every
//    MFMA operand is one 128-bit LDS read.
//  - LDS rows are 128 bytes; the 16-byte chunk index is XOR-swizzled with the
//    row so that the 8 (or 16) lanes served per LDS cycle hit distinct banks
//    both when MFMA fragments are read and when tiles are written.
//  - Two LDS stages: slice k+1 is fetched into registers before the MFMAs of
//    slice k are issued, and written to the other stage after them; one
//    barrier per slice.
//  - v_mfma_f32_32x32x16_bf16 with the Q fragment as the A operand and the P
//    fragment as the B operand, so each lane ends with 4 consecutive output
//    columns per 32x32 tile (8- or 16-byte stores in the epilogue).
//  - Workgroup ids are remapped so the tiles of one XCD share P and Q panels
//    in that XCD's L2.
#include "common.hpp"
#include "kernels.hpp"

namespace tpmlp {
namespace {

constexpr int kThreads = 256;
constexpr int BK = 64;

// Position of 16-byte chunk `chunk` in LDS row `row`: rows r and r+8 get
// different XOR patterns so 16 consecutive rows also spread over 64 banks.
__device__ __forceinline__ int swz(int row, int chunk) {
  return chunk ^ ((row & 7) ^ ((row >> 3) & 1));
}

template <int BM, int BN, int OUT>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(
    const uint16_t* __restrict__ P, int64_t ldp, const uint16_t* __restrict__ Q, int64_t ldq,
    void* __restrict__ C, int64_t ldc, int M, int N, int K, int group_m) {
  constexpr int TM = BM / 2, TN = BN / 2;      // wave tile (2 x 2 waves)
  constexpr int MT = TM / 32, NT = TN / 32;    // 32x32 MFMA tiles per wave
  constexpr int P_CHUNKS = BM * (BK / 8);      // 16-byte chunks in a P slice
  constexpr int P_PER_THREAD = (P_CHUNKS + kThreads - 1) / kThreads;
  constexpr int Q_BLOCKS = (BK / 8) * (BN / 8);  // 8x8 blocks in a Q slice
  constexpr int Q_PER_THREAD = (Q_BLOCKS + kThreads - 1) / kThreads;
  constexpr int STAGE = (BM + BN) * BK;          // uint16 elements per LDS stage
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  grouped_tile(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  u32x4 preg[P_PER_THREAD];
  u32x4 qreg[Q_PER_THREAD][8];

  auto load_global = [&](int k0) {
#pragma unroll
    for (int j = 0; j < P_PER_THREAD; ++j) {
      const int i = t + j * kThreads;
      const int r = i >> 3, c = i & 7;
      const int gm = m0 + r, gk = k0 + c * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if ((P_CHUNKS % kThreads == 0 || i < P_CHUNKS) && gm < M && gk < K)
        v = *reinterpret_cast<const u32x4*>(P + (int64_t)gm * ldp + gk);
      preg[j] = v;
    }
#pragma unroll
    for (int j = 0; j < Q_PER_THREAD; ++j) {
      const int i = t + j * kThreads;
      const int kb = i & 7, nb = i >> 3;
      const int gn = n0 + nb * 8;
      const bool ok = (Q_BLOCKS % kThreads == 0 || i < Q_BLOCKS) && gn < N;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int gk = k0 + kb * 8 + r;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (ok && gk < K) v = *reinterpret_cast<const u32x4*>(Q + (int64_t)gk * ldq + gn);
        qreg[j][r] = v;
      }
    }
  };

  auto store_lds = [&](int buf) {
    uint16_t* sP = smem + buf * STAGE;
    uint16_t* sQ = sP + BM * BK;
#pragma unroll
    for (int j = 0; j < P_PER_THREAD; ++j) {
      const int i = t + j * kThreads;
      if (P_CHUNKS % kThreads == 0 || i < P_CHUNKS) {
        const int r = i >> 3, c = i & 7;
        *reinterpret_cast<u32x4*>(sP + r * BK + swz(r, c) * 8) = preg[j];
      }
    }
#pragma unroll
    for (int j = 0; j < Q_PER_THREAD; ++j) {
      const int i = t + j * kThreads;
      if (Q_BLOCKS % kThreads == 0 || i < Q_BLOCKS) {
        const int kb = i & 7, nb = i >> 3;
        // qreg[j][r] holds row k = kb*8 + r, columns nb*8 .. nb*8+7; dword p
        // holds columns 2p (low half) and 2p+1 (high half). Column jn of the
        // block becomes one K-contiguous 16-byte chunk.
#pragma unroll
        for (int jn = 0; jn < 8; ++jn) {
          const int p = jn >> 1;
          u32x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t x = qreg[j][2 * q][p], y = qreg[j][2 * q + 1][p];
            o[q] = (jn & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
          }
          const int n = nb * 8 + jn;
          *reinterpret_cast<u32x4*>(sQ + n * BK + swz(n, kb) * 8) = o;
        }
      }
    }
  };

  f32x16 acc[NT][MT];
#pragma unroll
  for (int ni = 0; ni < NT; ++ni)
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[ni][mi][v] = 0.0f;

  const int ktiles = (K + BK - 1) / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();

  for (int kt = 0; kt < ktiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ktiles) load_global((kt + 1) * BK);

    const uint16_t* sP = smem + buf * STAGE;
    const uint16_t* sQ = sP + BM * BK;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int chunk = 2 * s + (lane >> 5);
      bf16x8 a[NT], b[MT];
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) {
        const int n = wn * TN + ni * 32 + (lane & 31);
        a[ni] = *reinterpret_cast<const bf16x8*>(sQ + n * BK + swz(n, chunk) * 8);
      }
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        const int m = wm * TM + mi * 32 + (lane & 31);
        b[mi] = *reinterpret_cast<const bf16x8*>(sP + m * BK + swz(m, chunk) * 8);
      }
#pragma unroll
      for (int ni = 0; ni < NT; ++ni)
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
          acc[ni][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ni], b[mi], acc[ni][mi], 0, 0, 0);
    }

    if (kt + 1 < ktiles) store_lds(buf ^ 1);
    __syncthreads();
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

template <int BM, int BN>
hipError_t launch_cfg(const uint16_t* P, int64_t ldp, const uint16_t* Q, int64_t ldq, void* C,
                      int64_t ldc, int M, int N, int K, OutKind out, hipStream_t stream) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int group_m = 4;
  switch (out) {
    case OutKind::GeluBf16:
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, (int)OutKind::GeluBf16>), dim3(tiles),
                         dim3(kThreads), 0, stream, P, ldp, Q, ldq, C, ldc, M, N, K, group_m);
      break;
    case OutKind::F32:
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, (int)OutKind::F32>), dim3(tiles),
                         dim3(kThreads), 0, stream, P, ldp, Q, ldq, C, ldc, M, N, K, group_m);
      break;
    case OutKind::Bf16:
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, (int)OutKind::Bf16>), dim3(tiles),
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
