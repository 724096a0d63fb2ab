// Sum of the tensor-parallel partial outputs, Y = Σ_i Y_i, on one GPU.
//
// This is the arithmetic of the AllReduce(sum) that ends the MLP block
// ("Megatron-LM deep architecture", eq. for Output: Output = Σ_i Y_i). It is
// HBM-bound: N reads and one write per element, each touched once, so loads
// and stores are non-temporal (they bypass the caches' normal retention; a
// sweep on MI355X gave ~5.8-6.1 TB/s this way against ~5.0 with temporal
// stores). A lane owns 16-byte chunks of the partials (4 fp32 or 8 bf16
// elements), four of them per pass, 4 KB apart, so that a workgroup reads
// 16 KB of each partial per pass (about 6.1 TB/s for eight fp32 partials of
// the 7B-class shard, the rate of a plain copy, against 5.8 TB/s with one
// chunk per lane), and adds strictly in rank order in fp32, so the result
// does not depend on the launch shape.
//
// An optional bias (fp32 or bf16, one value per output column) is added once,
// after the sum, as the row-parallel linear of the pages' code pattern does
// after its all-reduce. Under sequence parallelism the all-reduce becomes a
// reduce-scatter and a rank keeps only its block of rows of the sum
// ("Megatron-LM deep architecture", sequence-parallel section); the host
// offsets the partial pointers to the first row, so the kernel always sums a
// contiguous range. Rows are d elements, d a multiple of the chunk, so a
// chunk never straddles two rows.
#include "common.hpp"
#include "kernels.hpp"

namespace tpmlp {
namespace {

constexpr int kMaxParts = 64;
constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // chunks per lane per pass

struct PartPtrs {
  const void* p[kMaxParts];
};

// Elements per 16-byte chunk of a partial.
template <bool IN_BF16>
constexpr int kVec = IN_BF16 ? 8 : 4;

template <bool IN_BF16>
__device__ __forceinline__ void load_chunk(const void* base, int64_t v, float (&x)[kVec<IN_BF16>]) {
  if constexpr (IN_BF16) {
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + v);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
      x[2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
    }
  } else {
    const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(base) + v);
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = w[j];
  }
}

// Bias (once, after the whole sum) and store of one chunk: element offset
// v·V, bias_kind 0 none, 1 fp32, 2 bf16; d = row length (the bias period).
template <bool OUT_BF16, int V>
__device__ __forceinline__ void finish_chunk(float (&acc)[V], void* Y, int64_t v, const void* bias,
                                             int bias_kind, int64_t d) {
  if (bias_kind != 0) {
    const int64_t c0 = (v * V) % d;
#pragma unroll
    for (int e = 0; e < V; ++e)
      acc[e] += bias_kind == 1 ? static_cast<const float*>(bias)[c0 + e]
                               : bf16_bits_to_f32(static_cast<const uint16_t*>(bias)[c0 + e]);
  }
  if constexpr (OUT_BF16) {
    if constexpr (V == 8) {
      const u32x4 o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                       pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(Y) + v);
    } else {
      const u32x2 o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
      __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(Y) + v);
    }
  } else {
    f32x4* q = reinterpret_cast<f32x4*>(Y) + (V / 4) * v;
    __builtin_nontemporal_store(f32x4{acc[0], acc[1], acc[2], acc[3]}, q);
    if constexpr (V == 8) __builtin_nontemporal_store(f32x4{acc[4], acc[5], acc[6], acc[7]}, q + 1);
  }
}

// The chunks v0 + u·kThreads, u < U, of every partial, summed in rank order.
template <bool IN_BF16, bool OUT_BF16, int U>
__device__ __forceinline__ void sum_chunks(const PartPtrs& parts, int nparts, void* Y, int64_t v0,
                                           const void* bias, int bias_kind, int64_t d) {
  constexpr int V = kVec<IN_BF16>;
  float acc[U][V];
#pragma unroll
  for (int u = 0; u < U; ++u) load_chunk<IN_BF16>(parts.p[0], v0 + u * kThreads, acc[u]);
  for (int i = 1; i < nparts; ++i) {
    float x[U][V];
#pragma unroll
    for (int u = 0; u < U; ++u) load_chunk<IN_BF16>(parts.p[i], v0 + u * kThreads, x[u]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < V; ++e) acc[u][e] += x[u][e];
  }
#pragma unroll
  for (int u = 0; u < U; ++u) finish_chunk<OUT_BF16, V>(acc[u], Y, v0 + u * kThreads, bias, bias_kind, d);
}

// A workgroup takes groups of kUnroll·kThreads consecutive chunks (16 KB of
// an fp32 partial per pass, each lane loading kUnroll chunks kThreads apart),
// grid-stride; then the chunks after the last whole group one per lane; then
// the elements after the last chunk.
template <bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void partial_sum_kernel(PartPtrs parts, int nparts,
                                                               void* __restrict__ Y, int64_t nvec,
                                                               int64_t numel,
                                                               const void* __restrict__ bias,
                                                               int bias_kind, int64_t d) {
  constexpr int V = kVec<IN_BF16>;
  constexpr int64_t kGroup = (int64_t)kUnroll * kThreads;
  const int64_t ngroups = nvec / kGroup;
  for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x)
    sum_chunks<IN_BF16, OUT_BF16, kUnroll>(parts, nparts, Y, g * kGroup + threadIdx.x, bias,
                                           bias_kind, d);
  for (int64_t v = ngroups * kGroup + (int64_t)blockIdx.x * kThreads + threadIdx.x; v < nvec;
       v += (int64_t)gridDim.x * kThreads)
    sum_chunks<IN_BF16, OUT_BF16, 1>(parts, nparts, Y, v, bias, bias_kind, d);
  // Scalar tail (numel not a multiple of the chunk), handled by the first block.
  if (blockIdx.x == 0) {
    for (int64_t e = nvec * V + threadIdx.x; e < numel; e += kThreads) {
      float a = 0.0f;
      for (int i = 0; i < nparts; ++i) {
        const float x = IN_BF16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(parts.p[i])[e])
                                : static_cast<const float*>(parts.p[i])[e];
        a = (i == 0) ? x : a + x;
      }
      if (bias_kind != 0)
        a += bias_kind == 1 ? static_cast<const float*>(bias)[e % d]
                            : bf16_bits_to_f32(static_cast<const uint16_t*>(bias)[e % d]);
      if constexpr (OUT_BF16)
        static_cast<uint16_t*>(Y)[e] = (uint16_t)f32_to_bf16_rne(a);
      else
        static_cast<float*>(Y)[e] = a;
    }
  }
}

}  // namespace

hipError_t launch_partial_sum(const void* const* parts, int nparts, bool parts_bf16, void* Y,
                              bool y_bf16, int64_t numel, const void* bias, int bias_kind,
                              int64_t d, hipStream_t stream) {
  if (numel == 0) return hipSuccess;
  PartPtrs pp{};
  for (int i = 0; i < nparts; ++i) pp.p[i] = parts[i];
  const int64_t nvec = numel / (parts_bf16 ? 8 : 4);
  // one group per workgroup up to 32 workgroups per CU (measured on MI355X
  // against 4 to 64 per CU and 1 to 4 chunks per lane), grid-stride beyond
  int64_t blocks = (nvec + (int64_t)kUnroll * kThreads - 1) / ((int64_t)kUnroll * kThreads);
  const int64_t max_blocks = 256 * 32;
  if (blocks > max_blocks) blocks = max_blocks;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks), block(kThreads);
  if (parts_bf16 && y_bf16)
    hipLaunchKernelGGL((partial_sum_kernel<true, true>), grid, block, 0, stream, pp, nparts, Y, nvec, numel, bias, bias_kind, d);
  else if (parts_bf16)
    hipLaunchKernelGGL((partial_sum_kernel<true, false>), grid, block, 0, stream, pp, nparts, Y, nvec, numel, bias, bias_kind, d);
  else if (y_bf16)
    hipLaunchKernelGGL((partial_sum_kernel<false, true>), grid, block, 0, stream, pp, nparts, Y, nvec, numel, bias, bias_kind, d);
  else
    hipLaunchKernelGGL((partial_sum_kernel<false, false>), grid, block, 0, stream, pp, nparts, Y, nvec, numel, bias, bias_kind, d);
  return hipGetLastError();
}

}  // namespace tpmlp
