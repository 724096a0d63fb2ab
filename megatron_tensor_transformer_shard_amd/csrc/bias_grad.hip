// Gradient of a bias added to every row: db[c] = Σ_r G[r, c], for a bf16
// G [rows, cols] (row stride ld) and an fp32 db [cols].
//
// The column-parallel linear of the pages' code pattern adds its bias to
// every token's output ("Megatron-LM deep architecture", code-pattern
// section), and so does the row-parallel linear after its all-reduce; the
// gradient of such a bias is the column sum of the gradient of the layer's
// output: of dS (the gradient at GeLU's input) for the first layer's block
// b1_i, of dY for the second layer's b2.
//
// HBM-bound: 2 bytes read per element. Two passes and no atomics, so the
// result does not depend on timing:
//  1. A workgroup sums a block of kRows rows over 512 columns: each lane owns
//     8 adjacent columns (one 16-byte load per row), the 4 waves take every
//     4th row, and their sums are added in wave order through LDS into one
//     fp32 partial per column and row block.
//  2. One thread per column adds the row blocks' partials in block order,
//     loading kBatch of them at a time so that their latencies overlap (a
//     loop of dependent single loads left this pass latency-bound).
#include "common.hpp"
#include "kernels.hpp"

namespace tpmlp {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 128;              // rows per workgroup of pass 1
constexpr int kCols = 512;              // columns per workgroup of pass 1 (64 lanes x 8)
constexpr int kRowsPerWave = kRows / 4;
constexpr int kBatch = 16;              // partials loaded together in pass 2

__global__ __launch_bounds__(kThreads) void colsum_partial_kernel(const uint16_t* __restrict__ G,
                                                                  int64_t ld, int rows, int cols,
                                                                  float* __restrict__ partial) {
  __shared__ float red[4][kCols];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int c0 = blockIdx.x * kCols + lane * 8;
  const int r0 = blockIdx.y * kRows + wave;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (c0 < cols) {  // cols is a multiple of 8, so a lane's 8 columns are all inside or all out
    const uint16_t* p = G + (int64_t)r0 * ld + c0;
#pragma unroll 16
    for (int j = 0; j < kRowsPerWave; ++j) {
      if (r0 + 4 * j < rows) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(p + (int64_t)(4 * j) * ld);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += __uint_as_float(w[q] << 16);
          acc[2 * q + 1] += __uint_as_float(w[q] & 0xFFFF0000u);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[wave][lane * 8 + e] = acc[e];
  __syncthreads();
  // each thread finishes 2 of the 512 columns: waves 0..3 in order
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = 2 * t + h, c = blockIdx.x * kCols + k;
    if (c < cols)
      partial[(int64_t)blockIdx.y * cols + c] = ((red[0][k] + red[1][k]) + red[2][k]) + red[3][k];
  }
}

__global__ __launch_bounds__(kThreads) void colsum_finish_kernel(const float* __restrict__ partial,
                                                                 int blocks, int cols,
                                                                 float* __restrict__ out) {
  const int c = blockIdx.x * kThreads + threadIdx.x;
  if (c >= cols) return;
  float s = 0.0f;
  for (int b0 = 0; b0 < blocks; b0 += kBatch) {
    float v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      v[j] = b0 + j < blocks ? partial[(int64_t)(b0 + j) * cols + c] : 0.0f;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) s += v[j];  // block order; a missing block adds +0
  }
  out[c] = s;
}

}  // namespace

int64_t colsum_row_blocks(int64_t rows) { return (rows + kRows - 1) / kRows; }

hipError_t launch_colsum_bf16(const uint16_t* G, int64_t ld, int rows, int cols, float* out,
                              float* partial, hipStream_t stream) {
  if (cols <= 0) return hipSuccess;
  const int blocks = (int)colsum_row_blocks(rows);
  if (blocks > 0) {
    const dim3 grid((unsigned)((cols + kCols - 1) / kCols), (unsigned)blocks);
    hipLaunchKernelGGL(colsum_partial_kernel, grid, dim3(kThreads), 0, stream, G, ld, rows, cols,
                       partial);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(colsum_finish_kernel, dim3((unsigned)((cols + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, partial, blocks, cols, out);
  return hipGetLastError();
}

}  // namespace tpmlp
