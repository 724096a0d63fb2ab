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
//                bf16 + amax(|Z|) epilogue or a plain bf16 store.
#include "common.hpp"
#include "kernels.hpp"

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
// e4m3 GEMM tile engine. LDS rows are 128 bytes (BK = 128 e4m3 values), with
// the same 16-byte chunk swizzle as the bf16 engine.
// ---------------------------------------------------------------------------
constexpr int BK = 128;

__device__ __forceinline__ int swz(int row, int chunk) {
  return chunk ^ ((row & 7) ^ ((row >> 3) & 1));
}

// byte lanes: perm(hi, lo, sel) picks result byte i from {lo[0..3], hi[0..3]} by sel byte i.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

template <int BM, int BN, int OUT>
__global__ __launch_bounds__(kThreads) void gemm_e4m3_kernel(
    const uint8_t* __restrict__ P, int64_t ldp, const float* __restrict__ sP,
    const uint8_t* __restrict__ Q, int64_t ldq, const float* __restrict__ sQ,
    uint16_t* __restrict__ C, int64_t ldc, float* __restrict__ z_amax, int M, int N, int K,
    int group_m) {
  constexpr int TM = BM / 2, TN = BN / 2;
  constexpr int MT = TM / 32, NT = TN / 32;
  constexpr int P_CHUNKS = BM * (BK / 16);          // 16-byte chunks in a P slice
  constexpr int P_PER_THREAD = (P_CHUNKS + kThreads - 1) / kThreads;
  constexpr int Q_BLOCKS = (BK / 8) * (BN / 16);    // 8(k) x 16(n) byte blocks
  constexpr int Q_PER_THREAD = (Q_BLOCKS + kThreads - 1) / kThreads;
  constexpr int STAGE = (BM + BN) * BK;             // bytes per LDS stage

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

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
      const int gm = m0 + r, gk = k0 + c * 16;
      u32x4 v = {0u, 0u, 0u, 0u};
      if ((P_CHUNKS % kThreads == 0 || i < P_CHUNKS) && gm < M && gk < K)
        v = *reinterpret_cast<const u32x4*>(P + (int64_t)gm * ldp + gk);
      preg[j] = v;
    }
#pragma unroll
    for (int j = 0; j < Q_PER_THREAD; ++j) {
      const int i = t + j * kThreads;
      const int kb = i & 15, nb = i >> 4;   // 16 k-blocks of 8 rows; n-chunks of 16 bytes
      const int gn = n0 + nb * 16;
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
    uint8_t* sPl = smem + buf * STAGE;
    uint8_t* sQl = sPl + BM * BK;
#pragma unroll
    for (int j = 0; j < P_PER_THREAD; ++j) {
      const int i = t + j * kThreads;
      if (P_CHUNKS % kThreads == 0 || i < P_CHUNKS) {
        const int r = i >> 3, c = i & 7;
        *reinterpret_cast<u32x4*>(sPl + r * BK + swz(r, c) * 16) = preg[j];
      }
    }
#pragma unroll
    for (int j = 0; j < Q_PER_THREAD; ++j) {
      const int i = t + j * kThreads;
      if (Q_BLOCKS % kThreads == 0 || i < Q_BLOCKS) {
        const int kb = i & 15, nb = i >> 4;
        // qreg[j][r] = row k = kb*8 + r, bytes n = nb*16 .. +15 (dword c holds n = 4c..4c+3).
        // Output for column n: 8 bytes, k = kb*8 .. +7 (two dwords).
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint32_t out[2][4];   // [k half][n within the dword]
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t a = qreg[j][4 * h + 0][c], b = qreg[j][4 * h + 1][c];
            const uint32_t cc = qreg[j][4 * h + 2][c], d = qreg[j][4 * h + 3][c];
            const uint32_t t0 = perm(b, a, 0x05010400u);   // a0 b0 a1 b1
            const uint32_t t1 = perm(b, a, 0x07030602u);   // a2 b2 a3 b3
            const uint32_t t2 = perm(d, cc, 0x05010400u);  // c0 d0 c1 d1
            const uint32_t t3 = perm(d, cc, 0x07030602u);  // c2 d2 c3 d3
            out[h][0] = perm(t2, t0, 0x05040100u);         // a0 b0 c0 d0
            out[h][1] = perm(t2, t0, 0x07060302u);         // a1 b1 c1 d1
            out[h][2] = perm(t3, t1, 0x05040100u);         // a2 b2 c2 d2
            out[h][3] = perm(t3, t1, 0x07060302u);         // a3 b3 c3 d3
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int n = nb * 16 + 4 * c + e;
            const int c16 = kb >> 1, half = kb & 1;
            u32x2 o = {out[0][e], out[1][e]};
            *reinterpret_cast<u32x2*>(sQl + n * BK + swz(n, c16) * 16 + half * 8) = o;
          }
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
    const uint8_t* sPl = smem + buf * STAGE;
    const uint8_t* sQl = sPl + BM * BK;
#pragma unroll
    for (int s = 0; s < BK / 64; ++s) {
      // lane half h holds k = s*64 + h*32 .. +31: 16-byte chunks 4s+2h, 4s+2h+1
      const int c0 = 4 * s + 2 * (lane >> 5);
      i32x8 a[NT], b[MT];
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) {
        const int n = wn * TN + ni * 32 + (lane & 31);
        const u32x4 lo = *reinterpret_cast<const u32x4*>(sQl + n * BK + swz(n, c0) * 16);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(sQl + n * BK + swz(n, c0 + 1) * 16);
        a[ni] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        const int m = wm * TM + mi * 32 + (lane & 31);
        const u32x4 lo = *reinterpret_cast<const u32x4*>(sPl + m * BK + swz(m, c0) * 16);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(sPl + m * BK + swz(m, c0 + 1) * 16);
        b[mi] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int ni = 0; ni < NT; ++ni)
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
          acc[ni][mi] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              a[ni], b[mi], acc[ni][mi], 0, 0, 0, 127, 0, 127);
    }
    if (kt + 1 < ktiles) store_lds(buf ^ 1);
    __syncthreads();
  }

  const float dq = 1.0f / (sP[0] * sQ[0]);
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
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[ni][mi][4 * g + e] * dq;
        uint32_t bits[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float z = (OUT == (int)OutKind::GeluBf16) ? gelu_exact(v[e]) : v[e];
          bits[e] = f32_to_bf16_rne(z);
          if (OUT == (int)OutKind::GeluBf16) zmax = fmaxf(zmax, fabsf(bf16_bits_to_f32(bits[e])));
        }
        u32x2 o = {bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16)};
        *reinterpret_cast<u32x2*>(C + (int64_t)m * ldc + n) = o;
      }
    }
  }
  if (OUT == (int)OutKind::GeluBf16 && z_amax != nullptr) {
    zmax = wave_max(zmax);
    if (lane == 0) atomic_max_nonneg(z_amax, zmax);
  }
}

template <int BM, int BN>
hipError_t launch_cfg(const uint8_t* P, int64_t ldp, const float* sP, const uint8_t* Q,
                      int64_t ldq, const float* sQ, uint16_t* C, int64_t ldc, float* z_amax,
                      int M, int N, int K, OutKind out, hipStream_t stream) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int group_m = 4;
  if (out == OutKind::GeluBf16)
    hipLaunchKernelGGL((gemm_e4m3_kernel<BM, BN, (int)OutKind::GeluBf16>), dim3(tiles),
                       dim3(kThreads), 0, stream, P, ldp, sP, Q, ldq, sQ, C, ldc, z_amax, M, N,
                       K, group_m);
  else
    hipLaunchKernelGGL((gemm_e4m3_kernel<BM, BN, (int)OutKind::Bf16>), dim3(tiles),
                       dim3(kThreads), 0, stream, P, ldp, sP, Q, ldq, sQ, C, ldc, z_amax, M, N,
                       K, group_m);
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

hipError_t launch_gemm_e4m3(const uint8_t* P, int64_t ldp, const float* sP, const uint8_t* Q,
                            int64_t ldq, const float* sQ, uint16_t* C, int64_t ldc, float* z_amax,
                            int M, int N, int K, OutKind out, hipStream_t stream) {
  if (z_amax != nullptr) {
    hipError_t e = launch_fill_f32(z_amax, 0.0f, stream);
    if (e != hipSuccess) return e;
  }
  if (M == 0 || N == 0) return hipSuccess;
  // 256x256 e4m3 tiles exceed the register budget (the byte transpose needs
  // more live registers than the bf16 one), so the widest tile is 256x192.
  const long tiles192 = (long)((M + 255) / 256) * ((N + 191) / 192);
  const long tiles128 = (long)((M + 127) / 128) * ((N + 127) / 128);
  const double w192 = (double)((tiles192 + 255) / 256);
  const double w128 = (double)((tiles128 + 255) / 256) * 0.40;
  if (w128 < w192 - 1e-9)
    return launch_cfg<128, 128>(P, ldp, sP, Q, ldq, sQ, C, ldc, z_amax, M, N, K, out, stream);
  return launch_cfg<256, 192>(P, ldp, sP, Q, ldq, sQ, C, ldc, z_amax, M, N, K, out, stream);
}

}  // namespace tpmlp
