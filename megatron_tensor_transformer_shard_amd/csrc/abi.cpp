// C ABI of the tensor-parallel MLP shard library (declared in include/tpmlp.h).
//
// Every entry point validates its arguments on the host before anything is
// enqueued (so an error status means no work was done), derives the rank's
// shard views, and enqueues the kernels on the caller's stream.
#include "../../include/tpmlp.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "kernels.hpp"

namespace {

using tpmlp::OutKind;

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
// Row strides (and so d, F, lda) are limited so that the kernels' per-lane
// byte offsets within a tile fit in 32 bits.
constexpr int64_t kMaxLd = int64_t(1) << 23;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
  uintptr_t lo, hi;  // byte range [lo, hi)
};

// Bytes touched by a rows x cols matrix with row stride ld (elements of `esize` bytes).
Span mat_span(const void* p, int64_t rows, int64_t cols, int64_t ld, int64_t esize) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  if (rows <= 0 || cols <= 0) return {lo, lo};
  return {lo, lo + (uintptr_t)(((rows - 1) * ld + cols) * esize)};
}

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.lo < a.hi && b.lo < b.hi; }

int status_of(hipError_t e) { return e == hipSuccess ? TPM_OK : TPM_ERR_HIP; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Shared size checks for a GEMM step with inputs [M, K] and [K, N].
int check_dims(int64_t M, int64_t K, int64_t N, int64_t mult) {
  if (M < 0 || K <= 0 || N <= 0) return TPM_ERR_SHAPE;
  if (M > kMaxDim || K > kMaxLd || N > kMaxLd) return TPM_ERR_SHAPE;
  if (K % mult != 0 || N % mult != 0) return TPM_ERR_SHAPE;
  if (M * K > (int64_t(1) << 46) || M * N > (int64_t(1) << 46) || K * N > (int64_t(1) << 46))
    return TPM_ERR_SHAPE;
  return TPM_OK;
}

size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

// The clock-stamped measurement calls: the stamps array must hold
// tp_clock_stamp_count(M, N) values (4 per workgroup of the largest grid any
// tile choice makes for an [M, N] output).
int check_stamps(const uint64_t* stamps, int64_t count, int64_t M, int64_t N) {
  if (stamps == nullptr) return TPM_ERR_NULL;
  if (!aligned16(stamps)) return TPM_ERR_ALIGN;
  if (M < 0 || N < 0 || M > kMaxDim || N > kMaxDim) return TPM_ERR_SHAPE;
  if (count < 4 * ((M + 127) / 128) * ((N + 127) / 128)) return TPM_ERR_WORKSPACE;
  return TPM_OK;
}

int col_gelu_stamped(const void* X, const void* A_i, int64_t lda, void* Z_i, int64_t M,
                     int64_t d, int64_t F, uint64_t* stamps, void* stream);
int row_partial_stamped(const void* Z_i, const void* B_i, void* Y_i, int y_dtype, int64_t M,
                        int64_t F, int64_t d, uint64_t* stamps, void* stream);
int row_partial_e4m3_stamped(const void* Zq, const float* sZ, const void* Bq_i, const float* sB,
                             void* Y_i, int64_t M, int64_t F, int64_t d, uint64_t* stamps,
                             void* stream);

}  // namespace

extern "C" {

int tp_abi_version(void) { return TPM_ABI_VERSION; }

const char* tp_status_string(int status) {
  switch (status) {
    case TPM_OK: return "TPM_OK: success";
    case TPM_ERR_NULL: return "TPM_ERR_NULL: a required pointer is NULL";
    case TPM_ERR_ARG: return "TPM_ERR_ARG: invalid N or rank";
    case TPM_ERR_SHAPE: return "TPM_ERR_SHAPE: invalid or inconsistent sizes";
    case TPM_ERR_DTYPE: return "TPM_ERR_DTYPE: unsupported element type";
    case TPM_ERR_ALIGN: return "TPM_ERR_ALIGN: pointer or row stride not 16-byte aligned";
    case TPM_ERR_WORKSPACE: return "TPM_ERR_WORKSPACE: workspace missing or too small";
    case TPM_ERR_ALIAS: return "TPM_ERR_ALIAS: an output overlaps an input";
    case TPM_ERR_HIP: return "TPM_ERR_HIP: a HIP launch failed";
    case TPM_ERR_SCRATCH:
      return "TPM_ERR_SCRATCH: Z_i would exceed the static scratch of tp_mlp_shard_noalloc "
             "(TPM_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown tpmlp status";
  }
}

int tp_mlp_col_gelu(const void* X, const void* A_i, int64_t lda, void* Z_i, int64_t M,
                    int64_t d, int64_t F, void* stream) {
  return col_gelu_stamped(X, A_i, lda, Z_i, M, d, F, nullptr, stream);
}

int tp_mlp_row_partial(const void* Z_i, const void* B_i, void* Y_i, int y_dtype, int64_t M,
                       int64_t F, int64_t d, void* stream) {
  return row_partial_stamped(Z_i, B_i, Y_i, y_dtype, M, F, d, nullptr, stream);
}

int64_t tp_clock_stamp_count(int64_t M, int64_t N) {
  if (M < 0 || N < 0 || M > kMaxDim || N > kMaxDim) return 0;
  return 4 * ((M + 127) / 128) * ((N + 127) / 128);
}

int tp_mlp_col_gelu_stamped(const void* X, const void* A_i, int64_t lda, void* Z_i, int64_t M,
                            int64_t d, int64_t F, uint64_t* stamps, int64_t stamp_count,
                            void* stream) {
  int st = check_stamps(stamps, stamp_count, M, F);
  if (st != TPM_OK) return st;
  return col_gelu_stamped(X, A_i, lda, Z_i, M, d, F, stamps, stream);
}

int tp_mlp_row_partial_stamped(const void* Z_i, const void* B_i, void* Y_i, int y_dtype,
                               int64_t M, int64_t F, int64_t d, uint64_t* stamps,
                               int64_t stamp_count, void* stream) {
  int st = check_stamps(stamps, stamp_count, M, d);
  if (st != TPM_OK) return st;
  return row_partial_stamped(Z_i, B_i, Y_i, y_dtype, M, F, d, stamps, stream);
}

int tp_mlp_row_partial_e4m3_stamped(const void* Zq, const float* sZ, const void* Bq_i,
                                    const float* sB, void* Y_i, int64_t M, int64_t F, int64_t d,
                                    uint64_t* stamps, int64_t stamp_count, void* stream) {
  int st = check_stamps(stamps, stamp_count, M, d);
  if (st != TPM_OK) return st;
  return row_partial_e4m3_stamped(Zq, sZ, Bq_i, sB, Y_i, M, F, d, stamps, stream);
}

}  // extern "C"

namespace {

int col_gelu_stamped(const void* X, const void* A_i, int64_t lda, void* Z_i, int64_t M,
                     int64_t d, int64_t F, uint64_t* stamps, void* stream) {
  int st = check_dims(M, d, F, 8);
  if (st != TPM_OK) return st;
  if (lda < F || lda > kMaxLd) return TPM_ERR_SHAPE;
  if (M == 0) return TPM_OK;
  if (!X || !A_i || !Z_i) return TPM_ERR_NULL;
  if (!aligned16(X) || !aligned16(A_i) || !aligned16(Z_i) || lda % 8 != 0) return TPM_ERR_ALIGN;
  const Span z = mat_span(Z_i, M, F, F, 2);
  if (overlap(z, mat_span(X, M, d, d, 2)) || overlap(z, mat_span(A_i, d, F, lda, 2)))
    return TPM_ERR_ALIAS;
  return status_of(tpmlp::launch_gemm_bf16(static_cast<const uint16_t*>(X), d,
                                           static_cast<const uint16_t*>(A_i), lda, Z_i, F,
                                           (int)M, (int)F, (int)d, OutKind::GeluBf16,
                                           as_stream(stream), stamps));
}

int row_partial_stamped(const void* Z_i, const void* B_i, void* Y_i, int y_dtype, int64_t M,
                        int64_t F, int64_t d, uint64_t* stamps, void* stream) {
  if (y_dtype != TPM_F32 && y_dtype != TPM_BF16) return TPM_ERR_DTYPE;
  int st = check_dims(M, F, d, 8);
  if (st != TPM_OK) return st;
  if (M == 0) return TPM_OK;
  if (!Z_i || !B_i || !Y_i) return TPM_ERR_NULL;
  if (!aligned16(Z_i) || !aligned16(B_i) || !aligned16(Y_i)) return TPM_ERR_ALIGN;
  const Span y = mat_span(Y_i, M, d, d, y_dtype == TPM_F32 ? 4 : 2);
  if (overlap(y, mat_span(Z_i, M, F, F, 2)) || overlap(y, mat_span(B_i, F, d, d, 2)))
    return TPM_ERR_ALIAS;
  return status_of(tpmlp::launch_gemm_bf16(
      static_cast<const uint16_t*>(Z_i), F, static_cast<const uint16_t*>(B_i), d, Y_i, d,
      (int)M, (int)d, (int)F, y_dtype == TPM_F32 ? OutKind::F32 : OutKind::Bf16,
      as_stream(stream), stamps));
}

}  // namespace

extern "C" {

size_t tp_mlp_shard_workspace_size(int64_t M, int64_t d, int64_t H, int N) {
  if (M < 0 || d <= 0 || H <= 0 || N < 1 || H % N != 0) return 0;
  if (M > kMaxDim || H > kMaxDim) return 0;
  const int64_t F = H / N;
  return round256((size_t)M * (size_t)F * 2);
}

int tp_mlp_shard(const void* X, const void* A, const void* B, void* Y_i, int y_dtype, int64_t M,
                 int64_t d, int64_t H, int N, int rank, void* workspace, size_t workspace_bytes,
                 void* stream) {
  if (y_dtype != TPM_F32 && y_dtype != TPM_BF16) return TPM_ERR_DTYPE;
  if (N < 1 || rank < 0 || rank >= N) return TPM_ERR_ARG;
  if (H <= 0 || H % N != 0) return TPM_ERR_SHAPE;
  const int64_t F = H / N;
  int st = check_dims(M, d, F, 8);
  if (st != TPM_OK) return st;
  if (H > kMaxLd || H * d > (int64_t(1) << 46)) return TPM_ERR_SHAPE;
  if (M == 0) return TPM_OK;
  if (!X || !A || !B || !Y_i) return TPM_ERR_NULL;
  if (!workspace || workspace_bytes < tp_mlp_shard_workspace_size(M, d, H, N))
    return TPM_ERR_WORKSPACE;
  if (!aligned16(X) || !aligned16(A) || !aligned16(B) || !aligned16(Y_i) || !aligned16(workspace))
    return TPM_ERR_ALIGN;
  const Span sx = mat_span(X, M, d, d, 2), sa = mat_span(A, d, H, H, 2);
  const Span sb = mat_span(B, H, d, d, 2);
  const Span sy = mat_span(Y_i, M, d, d, y_dtype == TPM_F32 ? 4 : 2);
  const Span sw = {reinterpret_cast<uintptr_t>(workspace),
                   reinterpret_cast<uintptr_t>(workspace) + (uintptr_t)(M * F * 2)};
  if (overlap(sy, sx) || overlap(sy, sa) || overlap(sy, sb) || overlap(sy, sw) ||
      overlap(sw, sx) || overlap(sw, sa) || overlap(sw, sb))
    return TPM_ERR_ALIAS;

  // Shard views ("Megatron architecture and 6D parallel guide", §3.1):
  // A_i = A[:, rank·F : (rank+1)·F] (row stride H), B_i = B[rank·F : (rank+1)·F, :].
  const uint16_t* A_i = static_cast<const uint16_t*>(A) + (int64_t)rank * F;
  const uint16_t* B_i = static_cast<const uint16_t*>(B) + (int64_t)rank * F * d;
  uint16_t* Z = static_cast<uint16_t*>(workspace);
  hipStream_t s = as_stream(stream);
  hipError_t e = tpmlp::launch_gemm_bf16(static_cast<const uint16_t*>(X), d, A_i, H, Z, F,
                                         (int)M, (int)F, (int)d, OutKind::GeluBf16, s);
  if (e != hipSuccess) return TPM_ERR_HIP;
  e = tpmlp::launch_gemm_bf16(Z, F, B_i, d, Y_i, d, (int)M, (int)d, (int)F,
                              y_dtype == TPM_F32 ? OutKind::F32 : OutKind::Bf16, s);
  return status_of(e);
}

// ------------------------------------------------ transposed weights --
// The weights stored as nn.Linear keeps them ([out, in]): the GEMMs read them
// K-contiguous (the engine's K-major Q operand) instead of N-contiguous.

int tp_mlp_col_gelu_wt(const void* X, const void* W1_i, int64_t ldw, void* Z_i, int64_t M,
                       int64_t d, int64_t F, void* stream) {
  int st = check_dims(M, d, F, 8);
  if (st != TPM_OK) return st;
  if (ldw < d || ldw > kMaxLd) return TPM_ERR_SHAPE;
  if (M == 0) return TPM_OK;
  if (!X || !W1_i || !Z_i) return TPM_ERR_NULL;
  if (!aligned16(X) || !aligned16(W1_i) || !aligned16(Z_i) || ldw % 8 != 0) return TPM_ERR_ALIGN;
  const Span z = mat_span(Z_i, M, F, F, 2);
  if (overlap(z, mat_span(X, M, d, d, 2)) || overlap(z, mat_span(W1_i, F, d, ldw, 2)))
    return TPM_ERR_ALIAS;
  return status_of(tpmlp::launch_gemm_bf16_ex(
      static_cast<const uint16_t*>(X), d, static_cast<const uint16_t*>(W1_i), ldw, Z_i, F,
      (int)M, (int)F, (int)d, OutKind::GeluBf16, tpmlp::Layout::QT, nullptr, 0, nullptr,
      as_stream(stream)));
}

// ------------------------------------------------ column-layer bias --

namespace {
// The biased column step in either weight layout: W is A_i [d, F] (row
// stride ldw >= F) or W1_i [F, d] (row stride ldw >= d).
int col_gelu_bias(const void* X, const void* W, int64_t ldw, bool transposed, const void* b_i,
                  void* Z_i, int64_t M, int64_t d, int64_t F, void* stream) {
  int st = check_dims(M, d, F, 8);
  if (st != TPM_OK) return st;
  if (ldw < (transposed ? d : F) || ldw > kMaxLd) return TPM_ERR_SHAPE;
  if (M == 0) return TPM_OK;
  if (!X || !W || !b_i || !Z_i) return TPM_ERR_NULL;
  if (!aligned16(X) || !aligned16(W) || !aligned16(b_i) || !aligned16(Z_i) || ldw % 8 != 0)
    return TPM_ERR_ALIGN;
  const Span z = mat_span(Z_i, M, F, F, 2);
  const Span w = transposed ? mat_span(W, F, d, ldw, 2) : mat_span(W, d, F, ldw, 2);
  if (overlap(z, mat_span(X, M, d, d, 2)) || overlap(z, w) || overlap(z, mat_span(b_i, 1, F, F, 2)))
    return TPM_ERR_ALIAS;
  return status_of(tpmlp::launch_gemm_bf16_bias(
      static_cast<const uint16_t*>(X), d, static_cast<const uint16_t*>(W), ldw,
      static_cast<const uint16_t*>(b_i), Z_i, F, (int)M, (int)F, (int)d, OutKind::GeluBiasBf16,
      transposed ? tpmlp::Layout::QT : tpmlp::Layout::NN, as_stream(stream)));
}
}  // namespace

int tp_mlp_col_gelu_bias(const void* X, const void* A_i, int64_t lda, const void* b_i, void* Z_i,
                         int64_t M, int64_t d, int64_t F, void* stream) {
  return col_gelu_bias(X, A_i, lda, false, b_i, Z_i, M, d, F, stream);
}

int tp_mlp_col_gelu_bias_wt(const void* X, const void* W1_i, int64_t ldw, const void* b_i,
                            void* Z_i, int64_t M, int64_t d, int64_t F, void* stream) {
  return col_gelu_bias(X, W1_i, ldw, true, b_i, Z_i, M, d, F, stream);
}

int tp_mlp_row_partial_wt(const void* Z_i, const void* W2_i, int64_t ldw, void* Y_i,
                          int y_dtype, int64_t M, int64_t F, int64_t d, void* stream) {
  if (y_dtype != TPM_F32 && y_dtype != TPM_BF16) return TPM_ERR_DTYPE;
  int st = check_dims(M, F, d, 8);
  if (st != TPM_OK) return st;
  if (ldw < F || ldw > kMaxLd) return TPM_ERR_SHAPE;
  if (M == 0) return TPM_OK;
  if (!Z_i || !W2_i || !Y_i) return TPM_ERR_NULL;
  if (!aligned16(Z_i) || !aligned16(W2_i) || !aligned16(Y_i) || ldw % 8 != 0) return TPM_ERR_ALIGN;
  const Span y = mat_span(Y_i, M, d, d, y_dtype == TPM_F32 ? 4 : 2);
  if (overlap(y, mat_span(Z_i, M, F, F, 2)) || overlap(y, mat_span(W2_i, d, F, ldw, 2)))
    return TPM_ERR_ALIAS;
  return status_of(tpmlp::launch_gemm_bf16_ex(
      static_cast<const uint16_t*>(Z_i), F, static_cast<const uint16_t*>(W2_i), ldw, Y_i, d,
      (int)M, (int)d, (int)F, y_dtype == TPM_F32 ? OutKind::F32 : OutKind::Bf16,
      tpmlp::Layout::QT, nullptr, 0, nullptr, as_stream(stream)));
}

int tp_mlp_shard_wt(const void* X, const void* W1, const void* W2, void* Y_i, int y_dtype,
                    int64_t M, int64_t d, int64_t H, int N, int rank, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (y_dtype != TPM_F32 && y_dtype != TPM_BF16) return TPM_ERR_DTYPE;
  if (N < 1 || rank < 0 || rank >= N) return TPM_ERR_ARG;
  if (H <= 0 || H % N != 0) return TPM_ERR_SHAPE;
  const int64_t F = H / N;
  int st = check_dims(M, d, F, 8);
  if (st != TPM_OK) return st;
  if (H > kMaxLd || d > kMaxLd || H * d > (int64_t(1) << 46)) return TPM_ERR_SHAPE;
  if (M == 0) return TPM_OK;
  if (!X || !W1 || !W2 || !Y_i) return TPM_ERR_NULL;
  if (!workspace || workspace_bytes < tp_mlp_shard_workspace_size(M, d, H, N))
    return TPM_ERR_WORKSPACE;
  if (!aligned16(X) || !aligned16(W1) || !aligned16(W2) || !aligned16(Y_i) ||
      !aligned16(workspace))
    return TPM_ERR_ALIGN;
  const Span sx = mat_span(X, M, d, d, 2), s1 = mat_span(W1, H, d, d, 2);
  const Span s2 = mat_span(W2, d, H, H, 2);
  const Span sy = mat_span(Y_i, M, d, d, y_dtype == TPM_F32 ? 4 : 2);
  const Span sw = {reinterpret_cast<uintptr_t>(workspace),
                   reinterpret_cast<uintptr_t>(workspace) + (uintptr_t)(M * F * 2)};
  if (overlap(sy, sx) || overlap(sy, s1) || overlap(sy, s2) || overlap(sy, sw) ||
      overlap(sw, sx) || overlap(sw, s1) || overlap(sw, s2))
    return TPM_ERR_ALIAS;

  // The shards of the transposed weights: W1_i = W1[rank·F : (rank+1)·F, :]
  // (dense rows), W2_i = W2[:, rank·F : (rank+1)·F] (row stride H).
  const uint16_t* W1_i = static_cast<const uint16_t*>(W1) + (int64_t)rank * F * d;
  const uint16_t* W2_i = static_cast<const uint16_t*>(W2) + (int64_t)rank * F;
  uint16_t* Z = static_cast<uint16_t*>(workspace);
  hipStream_t s = as_stream(stream);
  hipError_t e = tpmlp::launch_gemm_bf16_ex(static_cast<const uint16_t*>(X), d, W1_i, d, Z, F,
                                            (int)M, (int)F, (int)d, OutKind::GeluBf16,
                                            tpmlp::Layout::QT, nullptr, 0, nullptr, s);
  if (e != hipSuccess) return TPM_ERR_HIP;
  e = tpmlp::launch_gemm_bf16_ex(Z, F, W2_i, H, Y_i, d, (int)M, (int)d, (int)F,
                                 y_dtype == TPM_F32 ? OutKind::F32 : OutKind::Bf16,
                                 tpmlp::Layout::QT, nullptr, 0, nullptr, s);
  return status_of(e);
}

int tp_partial_sum(const void* const* parts, int N, int part_dtype, void* Y, int y_dtype,
                   int64_t numel, void* stream) {
  if ((part_dtype != TPM_F32 && part_dtype != TPM_BF16) ||
      (y_dtype != TPM_F32 && y_dtype != TPM_BF16))
    return TPM_ERR_DTYPE;
  if (N < 1 || N > TPM_MAX_PARTS) return TPM_ERR_ARG;
  if (numel < 0 || numel > (int64_t(1) << 40)) return TPM_ERR_SHAPE;
  if (numel == 0) return TPM_OK;
  if (!parts || !Y) return TPM_ERR_NULL;
  for (int i = 0; i < N; ++i)
    if (!parts[i]) return TPM_ERR_NULL;
  if (!aligned16(Y)) return TPM_ERR_ALIGN;
  for (int i = 0; i < N; ++i)
    if (!aligned16(parts[i])) return TPM_ERR_ALIGN;
  const int64_t pe = part_dtype == TPM_F32 ? 4 : 2, ye = y_dtype == TPM_F32 ? 4 : 2;
  const Span sy = mat_span(Y, 1, numel, numel, ye);
  for (int i = 0; i < N; ++i) {
    const Span sp = mat_span(parts[i], 1, numel, numel, pe);
    const bool in_place = (i == 0 && parts[0] == Y && pe == ye);
    if (!in_place && overlap(sy, sp)) return TPM_ERR_ALIAS;
  }
  return status_of(tpmlp::launch_partial_sum(parts, N, part_dtype == TPM_BF16, Y,
                                             y_dtype == TPM_BF16, numel, nullptr, 0, 1,
                                             as_stream(stream)));
}

int tp_partial_sum_rows(const void* const* parts, int N, int part_dtype, int64_t M, int64_t d,
                        int64_t row_begin, int64_t row_end, const void* bias, int bias_dtype,
                        void* Y, int y_dtype, void* stream) {
  if ((part_dtype != TPM_F32 && part_dtype != TPM_BF16) ||
      (y_dtype != TPM_F32 && y_dtype != TPM_BF16) ||
      (bias && bias_dtype != TPM_F32 && bias_dtype != TPM_BF16))
    return TPM_ERR_DTYPE;
  if (N < 1 || N > TPM_MAX_PARTS) return TPM_ERR_ARG;
  if (M < 0 || d <= 0 || d % 8 != 0 || d > kMaxLd || M > kMaxDim ||
      M * d > (int64_t(1) << 40))
    return TPM_ERR_SHAPE;
  if (row_begin < 0 || row_end < row_begin || row_end > M) return TPM_ERR_SHAPE;
  const int64_t rows = row_end - row_begin;
  if (rows == 0) return TPM_OK;
  if (!parts || !Y) return TPM_ERR_NULL;
  for (int i = 0; i < N; ++i)
    if (!parts[i]) return TPM_ERR_NULL;
  if (!aligned16(Y) || (bias && !aligned16(bias))) return TPM_ERR_ALIGN;
  for (int i = 0; i < N; ++i)
    if (!aligned16(parts[i])) return TPM_ERR_ALIGN;
  const int64_t pe = part_dtype == TPM_F32 ? 4 : 2, ye = y_dtype == TPM_F32 ? 4 : 2;
  const int64_t be = bias_dtype == TPM_F32 ? 4 : 2;
  const Span sy = mat_span(Y, rows, d, d, ye);
  const void* first[TPM_MAX_PARTS];
  for (int i = 0; i < N; ++i) {
    first[i] = static_cast<const uint8_t*>(parts[i]) + row_begin * d * pe;
    const Span sp = mat_span(parts[i], M, d, d, pe);
    // in place: Y is exactly the block's rows of parts[0], same dtype
    const bool in_place = (i == 0 && first[0] == Y && pe == ye);
    if (!in_place && overlap(sy, sp)) return TPM_ERR_ALIAS;
  }
  if (bias && overlap(sy, mat_span(bias, 1, d, d, be))) return TPM_ERR_ALIAS;
  return status_of(tpmlp::launch_partial_sum(
      first, N, part_dtype == TPM_BF16, Y, y_dtype == TPM_BF16, rows * d, bias,
      bias ? (bias_dtype == TPM_F32 ? 1 : 2) : 0, d, as_stream(stream)));
}

int tp_reduce_scatter_share(const void* const* parts, int N, int part_dtype, int64_t M,
                            int64_t d, int rank, const void* bias, int bias_dtype, void* Y,
                            int y_dtype, void* stream) {
  if (N < 1 || N > TPM_MAX_PARTS || rank < 0 || rank >= N) return TPM_ERR_ARG;
  if (M < 0 || M % N != 0) return TPM_ERR_SHAPE;
  // Rank j's share of the sequence-parallel reduce-scatter: with tokens stored
  // sequence-major, its 1/N of the sequence is the row block [j·M/N, (j+1)·M/N).
  const int64_t rows = M / N;
  return tp_partial_sum_rows(parts, N, part_dtype, M, d, rank * rows, (rank + 1) * rows, bias,
                             bias_dtype, Y, y_dtype, stream);
}

}  // extern "C"

// ------------------------------------------------- allocation-free shard --
// Z_i of tp_mlp_shard_noalloc lives in this file-scope device array instead of
// a caller's workspace. Each device holds its own copy (for the life of the
// process); its address on a device is looked up once, with that device
// current, and kept. Calls on one device share the array.
namespace {

static __device__ __align__(256) unsigned char scratch[TPM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, or NULL on a HIP error.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int tp_mlp_shard_noalloc(const void* X, const void* A, const void* B, void* Y_i, int y_dtype,
                         int64_t M, int64_t d, int64_t H, int N, int rank, void* stream) {
  // the same checks as tp_mlp_shard, before anything touches the device
  if (y_dtype != TPM_F32 && y_dtype != TPM_BF16) return TPM_ERR_DTYPE;
  if (N < 1 || rank < 0 || rank >= N) return TPM_ERR_ARG;
  if (H <= 0 || H % N != 0) return TPM_ERR_SHAPE;
  int st = check_dims(M, d, H / N, 8);
  if (st != TPM_OK) return st;
  if (H > kMaxLd || H * d > (int64_t(1) << 46)) return TPM_ERR_SHAPE;
  if (M == 0) return TPM_OK;
  if (!X || !A || !B || !Y_i) return TPM_ERR_NULL;
  const size_t need = tp_mlp_shard_workspace_size(M, d, H, N);
  if (need == 0 || need > (size_t)TPM_NOALLOC_SCRATCH_BYTES) return TPM_ERR_SCRATCH;
  void* z = scratch_on_current_device();
  if (z == nullptr) return TPM_ERR_HIP;
  return tp_mlp_shard(X, A, B, Y_i, y_dtype, M, d, H, N, rank, z,
                      (size_t)TPM_NOALLOC_SCRATCH_BYTES, stream);
}

// ------------------------------------------------------------------ fp8 --

int tp_amax_bf16(const void* T, int64_t numel, float* amax, void* stream) {
  if (numel < 0 || numel > (int64_t(1) << 40)) return TPM_ERR_SHAPE;
  if (!amax || (!T && numel > 0)) return TPM_ERR_NULL;
  if ((T && !aligned16(T)) || (reinterpret_cast<uintptr_t>(amax) & 3u)) return TPM_ERR_ALIGN;
  if (numel > 0 && overlap(mat_span(amax, 1, 1, 1, 4), mat_span(T, 1, numel, numel, 2)))
    return TPM_ERR_ALIAS;
  return status_of(tpmlp::launch_amax_bf16(static_cast<const uint16_t*>(T), numel, amax,
                                           as_stream(stream)));
}

int tp_quant_e4m3(const void* T, int64_t numel, const float* amax, void* Tq, float* scale,
                  void* stream) {
  if (numel < 0 || numel % 16 != 0 || numel > (int64_t(1) << 40)) return TPM_ERR_SHAPE;
  if (!amax || !scale || ((!T || !Tq) && numel > 0)) return TPM_ERR_NULL;
  if ((T && !aligned16(T)) || (Tq && !aligned16(Tq)) ||
      (reinterpret_cast<uintptr_t>(amax) & 3u) || (reinterpret_cast<uintptr_t>(scale) & 3u))
    return TPM_ERR_ALIGN;
  const Span st = mat_span(T, 1, numel, numel, 2), sq = mat_span(Tq, 1, numel, numel, 1);
  const Span ss = mat_span(scale, 1, 1, 1, 4), sa = mat_span(amax, 1, 1, 1, 4);
  if (overlap(sq, st) || overlap(sq, sa) || overlap(ss, st) || overlap(ss, sq) || overlap(ss, sa))
    return TPM_ERR_ALIAS;
  return status_of(tpmlp::launch_quant_e4m3(static_cast<const uint16_t*>(T), numel, amax,
                                            static_cast<uint8_t*>(Tq), scale, as_stream(stream)));
}

int tp_mlp_col_gelu_e4m3(const void* Xq, const float* sX, const void* Aq_i, int64_t lda,
                         const float* sA, void* Z_i, float* z_amax, int64_t M, int64_t d,
                         int64_t F, void* stream) {
  int st = check_dims(M, d, F, 16);
  if (st != TPM_OK) return st;
  if (lda < F || lda > kMaxLd) return TPM_ERR_SHAPE;
  if (M == 0) {
    if (z_amax) return status_of(tpmlp::launch_fill_f32(z_amax, 0.0f, as_stream(stream)));
    return TPM_OK;
  }
  if (!Xq || !sX || !Aq_i || !sA || !Z_i) return TPM_ERR_NULL;
  if (!aligned16(Xq) || !aligned16(Aq_i) || !aligned16(Z_i) || lda % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(z_amax) & 3u))
    return TPM_ERR_ALIGN;
  const Span z = mat_span(Z_i, M, F, F, 2);
  if (overlap(z, mat_span(Xq, M, d, d, 1)) || overlap(z, mat_span(Aq_i, d, F, lda, 1)) ||
      overlap(z, mat_span(sX, 1, 1, 1, 4)) || overlap(z, mat_span(sA, 1, 1, 1, 4)))
    return TPM_ERR_ALIAS;
  if (z_amax && (overlap(mat_span(z_amax, 1, 1, 1, 4), z) ||
                 overlap(mat_span(z_amax, 1, 1, 1, 4), mat_span(Xq, M, d, d, 1)) ||
                 overlap(mat_span(z_amax, 1, 1, 1, 4), mat_span(Aq_i, d, F, lda, 1))))
    return TPM_ERR_ALIAS;
  return status_of(tpmlp::launch_gemm_e4m3(
      static_cast<const uint8_t*>(Xq), d, sX, static_cast<const uint8_t*>(Aq_i), lda, sA,
      static_cast<uint16_t*>(Z_i), F, z_amax, nullptr, (int)M, (int)F, (int)d,
      OutKind::GeluBf16, as_stream(stream)));
}

int tp_mlp_row_partial_e4m3(const void* Zq, const float* sZ, const void* Bq_i, const float* sB,
                            void* Y_i, int64_t M, int64_t F, int64_t d, void* stream) {
  return row_partial_e4m3_stamped(Zq, sZ, Bq_i, sB, Y_i, M, F, d, nullptr, stream);
}

}  // extern "C"

namespace {

int row_partial_e4m3_stamped(const void* Zq, const float* sZ, const void* Bq_i, const float* sB,
                             void* Y_i, int64_t M, int64_t F, int64_t d, uint64_t* stamps,
                             void* stream) {
  int st = check_dims(M, F, d, 16);
  if (st != TPM_OK) return st;
  if (M == 0) return TPM_OK;
  if (!Zq || !sZ || !Bq_i || !sB || !Y_i) return TPM_ERR_NULL;
  if (!aligned16(Zq) || !aligned16(Bq_i) || !aligned16(Y_i)) return TPM_ERR_ALIGN;
  const Span y = mat_span(Y_i, M, d, d, 2);
  if (overlap(y, mat_span(Zq, M, F, F, 1)) || overlap(y, mat_span(Bq_i, F, d, d, 1)) ||
      overlap(y, mat_span(sZ, 1, 1, 1, 4)) || overlap(y, mat_span(sB, 1, 1, 1, 4)))
    return TPM_ERR_ALIAS;
  return status_of(tpmlp::launch_gemm_e4m3(
      static_cast<const uint8_t*>(Zq), F, sZ, static_cast<const uint8_t*>(Bq_i), d, sB,
      static_cast<uint16_t*>(Y_i), d, nullptr, nullptr, (int)M, (int)d, (int)F, OutKind::Bf16,
      as_stream(stream), stamps));
}

}  // namespace

extern "C" {

size_t tp_mlp_shard_e4m3_workspace_size(int64_t M, int64_t d, int64_t H, int N) {
  if (M < 0 || d <= 0 || H <= 0 || N < 1 || H % N != 0) return 0;
  if (M > kMaxDim || H > kMaxDim) return 0;
  const size_t MF = (size_t)M * (size_t)(H / N);
  return round256(MF * 2) + round256(MF) + 256;
}

int tp_mlp_shard_e4m3(const void* Xq, const float* sX, const void* Aq, const float* sA,
                      const void* Bq, const float* sB, void* Y_i, int64_t M, int64_t d, int64_t H,
                      int N, int rank, void* workspace, size_t workspace_bytes, void* stream) {
  if (N < 1 || rank < 0 || rank >= N) return TPM_ERR_ARG;
  if (H <= 0 || H % N != 0) return TPM_ERR_SHAPE;
  const int64_t F = H / N;
  int st = check_dims(M, d, F, 16);
  if (st != TPM_OK) return st;
  if (H > kMaxLd || H * d > (int64_t(1) << 46)) return TPM_ERR_SHAPE;
  if (M == 0) return TPM_OK;
  if (!Xq || !sX || !Aq || !sA || !Bq || !sB || !Y_i) return TPM_ERR_NULL;
  if (!workspace || workspace_bytes < tp_mlp_shard_e4m3_workspace_size(M, d, H, N))
    return TPM_ERR_WORKSPACE;
  if (!aligned16(Xq) || !aligned16(Aq) || !aligned16(Bq) || !aligned16(Y_i) ||
      !aligned16(workspace))
    return TPM_ERR_ALIGN;
  const size_t MF = (size_t)M * (size_t)F;
  const Span sx = mat_span(Xq, M, d, d, 1), sa = mat_span(Aq, d, H, H, 1);
  const Span sb = mat_span(Bq, H, d, d, 1), sy = mat_span(Y_i, M, d, d, 2);
  const Span sw = {reinterpret_cast<uintptr_t>(workspace),
                   reinterpret_cast<uintptr_t>(workspace) +
                       tp_mlp_shard_e4m3_workspace_size(M, d, H, N)};
  const Span ssx = mat_span(sX, 1, 1, 1, 4), ssa = mat_span(sA, 1, 1, 1, 4);
  const Span ssb = mat_span(sB, 1, 1, 1, 4);
  for (Span in : {sx, sa, sb, ssx, ssa, ssb})
    if (overlap(sy, in) || overlap(sw, in)) return TPM_ERR_ALIAS;
  if (overlap(sy, sw)) return TPM_ERR_ALIAS;

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint16_t* Z = reinterpret_cast<uint16_t*>(ws);
  uint8_t* Zq = ws + round256(MF * 2);
  float* z_amax = reinterpret_cast<float*>(Zq + round256(MF));
  float* sZ = z_amax + 1;
  const uint8_t* Aq_i = static_cast<const uint8_t*>(Aq) + (int64_t)rank * F;
  const uint8_t* Bq_i = static_cast<const uint8_t*>(Bq) + (int64_t)rank * F * d;
  hipStream_t s = as_stream(stream);
  hipError_t e = tpmlp::launch_gemm_e4m3(static_cast<const uint8_t*>(Xq), d, sX, Aq_i, H, sA, Z,
                                         F, z_amax, nullptr, (int)M, (int)F, (int)d,
                                         OutKind::GeluBf16, s);
  if (e != hipSuccess) return TPM_ERR_HIP;
  e = tpmlp::launch_quant_e4m3(Z, (int64_t)MF, z_amax, Zq, sZ, s);
  if (e != hipSuccess) return TPM_ERR_HIP;
  e = tpmlp::launch_gemm_e4m3(Zq, F, sZ, Bq_i, d, sB, static_cast<uint16_t*>(Y_i), d, nullptr,
                              nullptr, (int)M, (int)d, (int)F, OutKind::Bf16, s);
  return status_of(e);
}

// ------------------------------------------------- fp8 delayed scaling --

int tp_amax_history_push(float* history, uint32_t* count, int L, const float* amax,
                         float* next_scale, void* stream) {
  if (L < 1 || L > TPM_MAX_HISTORY) return TPM_ERR_ARG;
  if (!history || !count || !amax || !next_scale) return TPM_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(history) & 3u) || (reinterpret_cast<uintptr_t>(count) & 3u) ||
      (reinterpret_cast<uintptr_t>(amax) & 3u) || (reinterpret_cast<uintptr_t>(next_scale) & 3u))
    return TPM_ERR_ALIGN;
  const Span sh = mat_span(history, 1, L, L, 4), sc = mat_span(count, 1, 1, 1, 4);
  const Span sa = mat_span(amax, 1, 1, 1, 4), ss = mat_span(next_scale, 1, 1, 1, 4);
  if (overlap(sh, sc) || overlap(sh, sa) || overlap(sh, ss) || overlap(sc, sa) ||
      overlap(sc, ss) || overlap(sa, ss))
    return TPM_ERR_ALIAS;
  return status_of(
      tpmlp::launch_amax_history_push(history, count, L, amax, next_scale, as_stream(stream)));
}

int tp_mlp_col_gelu_e4m3_delayed(const void* Xq, const float* sX, const void* Aq_i, int64_t lda,
                                 const float* sA, const float* sZ, void* Zq_i, float* z_amax,
                                 int64_t M, int64_t d, int64_t F, void* stream) {
  int st = check_dims(M, d, F, 16);
  if (st != TPM_OK) return st;
  if (lda < F || lda > kMaxLd) return TPM_ERR_SHAPE;
  if (!z_amax) return TPM_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(z_amax) & 3u) return TPM_ERR_ALIGN;
  if (M == 0) return status_of(tpmlp::launch_fill_f32(z_amax, 0.0f, as_stream(stream)));
  if (!Xq || !sX || !Aq_i || !sA || !sZ || !Zq_i) return TPM_ERR_NULL;
  if (!aligned16(Xq) || !aligned16(Aq_i) || !aligned16(Zq_i) || lda % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(sZ) & 3u))
    return TPM_ERR_ALIGN;
  const Span z = mat_span(Zq_i, M, F, F, 1), za = mat_span(z_amax, 1, 1, 1, 4);
  for (Span in : {mat_span(Xq, M, d, d, 1), mat_span(Aq_i, d, F, lda, 1), mat_span(sX, 1, 1, 1, 4),
                  mat_span(sA, 1, 1, 1, 4), mat_span(sZ, 1, 1, 1, 4)})
    if (overlap(z, in) || overlap(za, in)) return TPM_ERR_ALIAS;
  if (overlap(z, za)) return TPM_ERR_ALIAS;
  return status_of(tpmlp::launch_gemm_e4m3(
      static_cast<const uint8_t*>(Xq), d, sX, static_cast<const uint8_t*>(Aq_i), lda, sA, Zq_i, F,
      z_amax, sZ, (int)M, (int)F, (int)d, OutKind::GeluE4m3, as_stream(stream)));
}

size_t tp_mlp_shard_e4m3_delayed_workspace_size(int64_t M, int64_t d, int64_t H, int N) {
  if (M < 0 || d <= 0 || H <= 0 || N < 1 || H % N != 0) return 0;
  if (M > kMaxDim || H > kMaxDim) return 0;
  return round256((size_t)M * (size_t)(H / N)) + 256;
}

int tp_mlp_shard_e4m3_delayed(const void* Xq, const float* sX, const void* Aq, const float* sA,
                              const void* Bq, const float* sB, const float* sZ, void* Y_i,
                              float* z_amax, int64_t M, int64_t d, int64_t H, int N, int rank,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (N < 1 || rank < 0 || rank >= N) return TPM_ERR_ARG;
  if (H <= 0 || H % N != 0) return TPM_ERR_SHAPE;
  const int64_t F = H / N;
  int st = check_dims(M, d, F, 16);
  if (st != TPM_OK) return st;
  if (H > kMaxLd || H * d > (int64_t(1) << 46)) return TPM_ERR_SHAPE;
  if (!z_amax) return TPM_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(z_amax) & 3u) return TPM_ERR_ALIGN;
  if (M == 0) return status_of(tpmlp::launch_fill_f32(z_amax, 0.0f, as_stream(stream)));
  if (!Xq || !sX || !Aq || !sA || !Bq || !sB || !sZ || !Y_i) return TPM_ERR_NULL;
  if (!workspace || workspace_bytes < tp_mlp_shard_e4m3_delayed_workspace_size(M, d, H, N))
    return TPM_ERR_WORKSPACE;
  if (!aligned16(Xq) || !aligned16(Aq) || !aligned16(Bq) || !aligned16(Y_i) ||
      !aligned16(workspace) || (reinterpret_cast<uintptr_t>(sZ) & 3u))
    return TPM_ERR_ALIGN;
  const Span sy = mat_span(Y_i, M, d, d, 2), sza = mat_span(z_amax, 1, 1, 1, 4);
  const Span sw = {reinterpret_cast<uintptr_t>(workspace),
                   reinterpret_cast<uintptr_t>(workspace) +
                       tp_mlp_shard_e4m3_delayed_workspace_size(M, d, H, N)};
  for (Span in : {mat_span(Xq, M, d, d, 1), mat_span(Aq, d, H, H, 1), mat_span(Bq, H, d, d, 1),
                  mat_span(sX, 1, 1, 1, 4), mat_span(sA, 1, 1, 1, 4), mat_span(sB, 1, 1, 1, 4),
                  mat_span(sZ, 1, 1, 1, 4)})
    if (overlap(sy, in) || overlap(sw, in) || overlap(sza, in)) return TPM_ERR_ALIAS;
  if (overlap(sy, sw) || overlap(sy, sza) || overlap(sw, sza)) return TPM_ERR_ALIAS;

  uint8_t* Zq = static_cast<uint8_t*>(workspace);
  const uint8_t* Aq_i = static_cast<const uint8_t*>(Aq) + (int64_t)rank * F;
  const uint8_t* Bq_i = static_cast<const uint8_t*>(Bq) + (int64_t)rank * F * d;
  hipStream_t s = as_stream(stream);
  hipError_t e = tpmlp::launch_gemm_e4m3(static_cast<const uint8_t*>(Xq), d, sX, Aq_i, H, sA, Zq,
                                         F, z_amax, sZ, (int)M, (int)F, (int)d,
                                         OutKind::GeluE4m3, s);
  if (e != hipSuccess) return TPM_ERR_HIP;
  e = tpmlp::launch_gemm_e4m3(Zq, F, sZ, Bq_i, d, sB, static_cast<uint16_t*>(Y_i), d, nullptr,
                              nullptr, (int)M, (int)d, (int)F, OutKind::Bf16, s);
  return status_of(e);
}

size_t tp_mlp_shard_backward_workspace_size(int64_t M, int64_t d, int64_t H, int N) {
  if (M < 0 || d <= 0 || H <= 0 || N < 1 || H % N != 0) return 0;
  if (M > kMaxDim || H > kMaxDim) return 0;
  const size_t mf = (size_t)M * (size_t)(H / N);
  return round256(mf * 4) + 2 * round256(mf * 2);
}

namespace {
// The bf16 backward of one rank's shard; with b1 (the column layer's whole
// bias [H]) S is recomputed with the rank's block b1_i and db1_i = Σ_m dS is
// written (bias-gradient scratch after the three workspace parts).
int shard_backward_bf16(const void* X, const void* A, const void* B, const void* dY,
                        const void* b1, float* dX_i, float* dA_i, float* dB_i, float* db1_i,
                        int64_t M, int64_t d, int64_t H, int N, int rank, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (N < 1 || rank < 0 || rank >= N) return TPM_ERR_ARG;
  if (H <= 0 || H % N != 0) return TPM_ERR_SHAPE;
  const int64_t F = H / N;
  int st = check_dims(M, d, F, 8);
  if (st != TPM_OK) return st;
  // M is the contraction length of the weight gradients.
  if (M % 8 != 0 || M > kMaxLd) return TPM_ERR_SHAPE;
  if (H > kMaxLd || H * d > (int64_t(1) << 46)) return TPM_ERR_SHAPE;
  const bool bias = b1 != nullptr || db1_i != nullptr;
  if (bias && (!b1 || !db1_i)) return TPM_ERR_NULL;
  if (M == 0) {  // no tokens: nothing to do, and a zero bias gradient
    if (!bias) return TPM_OK;
    if (!aligned16(db1_i)) return TPM_ERR_ALIGN;
    if (overlap(mat_span(db1_i, 1, F, F, 4), mat_span(b1, 1, H, H, 2))) return TPM_ERR_ALIAS;
    // the column sum of zero rows writes 0 to every column and reads no scratch
    return status_of(tpmlp::launch_colsum_bf16(nullptr, F, 0, (int)F, db1_i, nullptr,
                                               as_stream(stream)));
  }
  if (!X || !A || !B || !dY || !dX_i || !dA_i || !dB_i) return TPM_ERR_NULL;
  const size_t need = bias ? tp_mlp_shard_backward_bias_workspace_size(M, d, H, N)
                           : tp_mlp_shard_backward_workspace_size(M, d, H, N);
  if (!workspace || workspace_bytes < need) return TPM_ERR_WORKSPACE;
  if (!aligned16(X) || !aligned16(A) || !aligned16(B) || !aligned16(dY) || !aligned16(dX_i) ||
      !aligned16(dA_i) || !aligned16(dB_i) || !aligned16(workspace) ||
      (bias && (!aligned16(b1) || !aligned16(db1_i))))
    return TPM_ERR_ALIGN;
  const Span ins[5] = {mat_span(X, M, d, d, 2), mat_span(A, d, H, H, 2), mat_span(B, H, d, d, 2),
                       mat_span(dY, M, d, d, 2), mat_span(b1, bias ? 1 : 0, H, H, 2)};
  const Span outs[5] = {mat_span(dX_i, M, d, d, 4), mat_span(dA_i, d, F, F, 4),
                        mat_span(dB_i, F, d, d, 4), mat_span(db1_i, bias ? 1 : 0, F, F, 4),
                        {reinterpret_cast<uintptr_t>(workspace),
                         reinterpret_cast<uintptr_t>(workspace) + need}};
  for (int o = 0; o < 5; ++o) {
    for (int i = 0; i < 5; ++i)
      if (overlap(outs[o], ins[i])) return TPM_ERR_ALIAS;
    for (int p = o + 1; p < 5; ++p)
      if (overlap(outs[o], outs[p])) return TPM_ERR_ALIAS;
  }
  hipStream_t s = as_stream(stream);

  // Shard views as in the forward; A_i is [d, F] with row stride H, B_i [F, d] dense.
  const uint16_t* x = static_cast<const uint16_t*>(X);
  const uint16_t* dy = static_cast<const uint16_t*>(dY);
  const uint16_t* A_i = static_cast<const uint16_t*>(A) + (int64_t)rank * F;
  const uint16_t* B_i = static_cast<const uint16_t*>(B) + (int64_t)rank * F * d;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const size_t mf = (size_t)M * (size_t)F;
  float* S = reinterpret_cast<float*>(ws);
  uint16_t* dS = reinterpret_cast<uint16_t*>(ws + round256(mf * 4));
  uint16_t* Z = reinterpret_cast<uint16_t*>(ws + round256(mf * 4) + round256(mf * 2));
  using tpmlp::Layout;
  const int m = (int)M, dd = (int)d, f = (int)F;
  // S = X·A_i (+ b1_i), the forward's pre-activation, recomputed
  hipError_t e =
      bias ? tpmlp::launch_gemm_bf16_bias(x, d, A_i, H, static_cast<const uint16_t*>(b1) + rank * F,
                                          S, F, m, f, dd, OutKind::F32Bias, Layout::NN, s)
           : tpmlp::launch_gemm_bf16_ex(x, d, A_i, H, S, F, m, f, dd, OutKind::F32, Layout::NN,
                                        nullptr, 0, nullptr, s);
  // dS = bf16((dY·B_iᵀ) ⊙ GeLU'(S)), Z = bf16(GeLU(S)); B_iᵀ is B_i read K-contiguous
  if (e == hipSuccess)
    e = tpmlp::launch_gemm_bf16_ex(dy, d, B_i, d, dS, F, m, f, dd, OutKind::GeluGradBf16,
                                   Layout::QT, S, F, Z, s);
  // db1_i = Σ_m dS[m, :], the bias gradient, from the stored bf16 dS
  if (e == hipSuccess && bias)
    e = tpmlp::launch_colsum_bf16(dS, F, m, f, db1_i,
                                  reinterpret_cast<float*>(ws + round256(mf * 4) + 2 * round256(mf * 2)),
                                  s);
  // dX_i = dS·A_iᵀ
  if (e == hipSuccess)
    e = tpmlp::launch_gemm_bf16_ex(dS, F, A_i, H, dX_i, d, m, dd, f, OutKind::F32, Layout::QT,
                                   nullptr, 0, nullptr, s);
  // dB_i = Zᵀ·dY ([F, d]) and dA_i = Xᵀ·dS ([d, F]), contractions over the M
  // tokens, in one launch: each alone has too few output tiles to fill the chip
  if (e == hipSuccess)
    e = tpmlp::launch_gemm_bf16_pair({Z, F, dy, d, dB_i, d, f, dd, m},
                                     {x, d, dS, F, dA_i, F, dd, f, m}, OutKind::F32, Layout::PT, s);
  return status_of(e);
}
}  // namespace

size_t tp_mlp_shard_backward_bias_workspace_size(int64_t M, int64_t d, int64_t H, int N) {
  const size_t base = tp_mlp_shard_backward_workspace_size(M, d, H, N);
  if (base == 0) return 0;
  return base + round256((size_t)tpmlp::colsum_row_blocks(M) * (size_t)(H / N) * 4);
}

int tp_mlp_shard_backward(const void* X, const void* A, const void* B, const void* dY,
                          float* dX_i, float* dA_i, float* dB_i, int64_t M, int64_t d, int64_t H,
                          int N, int rank, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return shard_backward_bf16(X, A, B, dY, nullptr, dX_i, dA_i, dB_i, nullptr, M, d, H, N, rank,
                             workspace, workspace_bytes, stream);
}

int tp_mlp_shard_backward_bias(const void* X, const void* A, const void* b1, const void* B,
                               const void* dY, float* dX_i, float* dA_i, float* dB_i,
                               float* db1_i, int64_t M, int64_t d, int64_t H, int N, int rank,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return shard_backward_bf16(X, A, B, dY, b1, dX_i, dA_i, dB_i, db1_i, M, d, H, N, rank,
                             workspace, workspace_bytes, stream);
}

size_t tp_bias_grad_workspace_size(int64_t rows, int64_t cols) {
  if (rows < 0 || cols <= 0 || rows > kMaxDim || cols > kMaxLd) return 0;
  return round256((size_t)tpmlp::colsum_row_blocks(rows) * (size_t)cols * 4);
}

int tp_bias_grad_bf16(const void* G, int64_t ld, int64_t rows, int64_t cols, float* db,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 8 != 0 || cols > kMaxLd || rows > kMaxDim) return TPM_ERR_SHAPE;
  if (ld < cols || ld > kMaxLd) return TPM_ERR_SHAPE;
  // the partial pass has one 128-row block per grid row
  if (tpmlp::colsum_row_blocks(rows) > 65535) return TPM_ERR_SHAPE;
  if (!db || (rows > 0 && !G)) return TPM_ERR_NULL;
  const size_t need = tp_bias_grad_workspace_size(rows, cols);
  if (rows > 0 && (!workspace || workspace_bytes < need)) return TPM_ERR_WORKSPACE;
  if ((rows > 0 && (!aligned16(G) || !aligned16(workspace))) || !aligned16(db) || ld % 8 != 0)
    return TPM_ERR_ALIGN;
  const Span out = mat_span(db, 1, cols, cols, 4);
  if (rows > 0) {
    const Span ws{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need};
    if (overlap(out, mat_span(G, rows, cols, ld, 2)) || overlap(out, ws) ||
        overlap(ws, mat_span(G, rows, cols, ld, 2)))
      return TPM_ERR_ALIAS;
  }
  return status_of(tpmlp::launch_colsum_bf16(static_cast<const uint16_t*>(G), ld, (int)rows,
                                             (int)cols, db, static_cast<float*>(workspace),
                                             as_stream(stream)));
}

namespace {
// Byte offsets of the fp8 backward's workspace parts (each 256-byte aligned).
struct Fp8BwdLayout {
  size_t xq, xqt, aq, aqt, bqt, dyq, s, ds, z, dsq, zqt, total;
};
Fp8BwdLayout fp8_bwd_layout(int64_t M, int64_t d, int64_t F) {
  Fp8BwdLayout L{};
  size_t o = 256;  // amaxes and scales
  auto take = [&](size_t bytes) { const size_t at = o; o += round256(bytes); return at; };
  const size_t md = (size_t)M * d, df = (size_t)d * F, mf = (size_t)M * F;
  L.xq = take(md); L.xqt = take(md); L.aq = take(df); L.aqt = take(df); L.bqt = take(df);
  L.dyq = take(md); L.s = take(mf * 4); L.ds = take(mf * 2); L.z = take(mf * 2);
  L.dsq = take(mf); L.zqt = take(mf);
  L.total = o;
  return L;
}
}  // namespace

size_t tp_mlp_shard_backward_fp8_workspace_size(int64_t M, int64_t d, int64_t H, int N) {
  if (M < 0 || d <= 0 || H <= 0 || N < 1 || H % N != 0) return 0;
  if (M > kMaxDim || H > kMaxDim) return 0;
  return fp8_bwd_layout(M, d, H / N).total;
}

namespace {
// The fp8 backward of one rank's shard; with b1 (the column layer's whole
// bf16 bias [H]) the rank's block is added to the dequantised S, and
// db1_i = Σ_m dS (the bf16 dS) is written, with its scratch after the
// workspace's other parts.
int shard_backward_fp8(const void* X, const void* A, const void* B, const void* dY,
                       const void* b1, float* dX_i, float* dA_i, float* dB_i, float* db1_i,
                       int64_t M, int64_t d, int64_t H, int N, int rank, const float* w_amax,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (N < 1 || rank < 0 || rank >= N) return TPM_ERR_ARG;
  if (H <= 0 || H % N != 0) return TPM_ERR_SHAPE;
  const int64_t F = H / N;
  int st = check_dims(M, d, F, 16);
  if (st != TPM_OK) return st;
  // M is the row length of the transposed fp8 copies and the contraction
  // length of the weight gradients
  if (M % 16 != 0 || M > kMaxLd) return TPM_ERR_SHAPE;
  if (H > kMaxLd || H * d > (int64_t(1) << 46)) return TPM_ERR_SHAPE;
  // the quantise-and-transpose grid has one 64-row tile per y index
  constexpr int64_t kMaxTileRows = int64_t(65535) * 64;
  if (M > kMaxTileRows || d > kMaxTileRows || F > kMaxTileRows) return TPM_ERR_SHAPE;
  const bool bias = b1 != nullptr || db1_i != nullptr;
  if (bias && (!b1 || !db1_i)) return TPM_ERR_NULL;
  if (M == 0) {  // no tokens: nothing to do, and a zero bias gradient
    if (!bias) return TPM_OK;
    if (!aligned16(db1_i)) return TPM_ERR_ALIGN;
    if (overlap(mat_span(db1_i, 1, F, F, 4), mat_span(b1, 1, H, H, 2))) return TPM_ERR_ALIAS;
    return status_of(tpmlp::launch_colsum_bf16(nullptr, F, 0, (int)F, db1_i, nullptr,
                                               as_stream(stream)));
  }
  if (!X || !A || !B || !dY || !dX_i || !dA_i || !dB_i) return TPM_ERR_NULL;
  const Fp8BwdLayout L = fp8_bwd_layout(M, d, F);
  const size_t need = L.total + (bias ? round256((size_t)tpmlp::colsum_row_blocks(M) * F * 4) : 0);
  if (!workspace || workspace_bytes < need) return TPM_ERR_WORKSPACE;
  if (!aligned16(X) || !aligned16(A) || !aligned16(B) || !aligned16(dY) || !aligned16(dX_i) ||
      !aligned16(dA_i) || !aligned16(dB_i) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(w_amax) & 3u) || (bias && (!aligned16(b1) || !aligned16(db1_i))))
    return TPM_ERR_ALIGN;
  const Span ins[6] = {mat_span(X, M, d, d, 2), mat_span(A, d, H, H, 2), mat_span(B, H, d, d, 2),
                       mat_span(dY, M, d, d, 2), mat_span(w_amax, w_amax ? 1 : 0, 2, 2, 4),
                       mat_span(b1, bias ? 1 : 0, H, H, 2)};
  const Span outs[5] = {mat_span(dX_i, M, d, d, 4), mat_span(dA_i, d, F, F, 4),
                        mat_span(dB_i, F, d, d, 4), mat_span(db1_i, bias ? 1 : 0, F, F, 4),
                        {reinterpret_cast<uintptr_t>(workspace),
                         reinterpret_cast<uintptr_t>(workspace) + need}};
  for (int o = 0; o < 5; ++o) {
    for (int i = 0; i < 6; ++i)
      if (overlap(outs[o], ins[i])) return TPM_ERR_ALIAS;
    for (int p = o + 1; p < 5; ++p)
      if (overlap(outs[o], outs[p])) return TPM_ERR_ALIAS;
  }

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* am = reinterpret_cast<float*>(ws);       // amax: X, A, B, dY, dS, Z
  float* sc = am + 8;                             // scales in the same order
  uint8_t *Xq = ws + L.xq, *XqT = ws + L.xqt, *Aq = ws + L.aq, *AqT = ws + L.aqt;
  uint8_t *BqT = ws + L.bqt, *dYq = ws + L.dyq, *dSq = ws + L.dsq, *ZqT = ws + L.zqt;
  float* S = reinterpret_cast<float*>(ws + L.s);
  uint16_t* dS = reinterpret_cast<uint16_t*>(ws + L.ds);
  uint16_t* Z = reinterpret_cast<uint16_t*>(ws + L.z);
  const uint16_t* x = static_cast<const uint16_t*>(X);
  const uint16_t* dy = static_cast<const uint16_t*>(dY);
  const uint16_t* A_i = static_cast<const uint16_t*>(A) + (int64_t)rank * F;
  const uint16_t* B_i = static_cast<const uint16_t*>(B) + (int64_t)rank * F * d;
  hipStream_t s = as_stream(stream);
  const int m = (int)M, dd = (int)d, f = (int)F;
  using tpmlp::Fp8GemmArgs;
  constexpr int E4 = 0, E5 = 1;
  hipError_t e = hipSuccess;
  auto run = [&](hipError_t r) { if (e == hipSuccess) e = r; };
  // per-tensor amax scales: X, the whole of A and B (as in the fp8 forward;
  // given by the caller when w_amax is not NULL), dY; the six amax slots
  // (these four, then dS and Z) are cleared by one kernel
  const float* amA = w_amax ? w_amax : am + 1;
  const float* amB = w_amax ? w_amax + 1 : am + 2;
  run(tpmlp::launch_fill_f32(am, 0.0f, s, 6));
  {
    const uint16_t* ts[4] = {x, dy, static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B)};
    const int64_t ns[4] = {M * d, M * d, d * H, H * d};
    float* const outs4[4] = {am + 0, am + 3, am + 1, am + 2};
    run(tpmlp::launch_amax_bf16_multi(ts, ns, outs4, w_amax ? 2 : 4, s));
  }
  // quantised operands, in the orientation each GEMM reads them (X and A_i
  // in both, each from one read)
  run(tpmlp::launch_quant_fp8_tile(E4, x, d, m, dd, am + 0, Xq, d, XqT, M, sc + 0, s));
  run(tpmlp::launch_quant_fp8_tile(E4, A_i, H, dd, f, amA, Aq, F, AqT, d, sc + 1, s));
  run(tpmlp::launch_quant_fp8_tile(E4, B_i, d, f, dd, amB, nullptr, 0, BqT, F, sc + 2, s));
  run(tpmlp::launch_quant_fp8(E5, dy, M * d, am + 3, dYq, sc + 3, s));
  // S = (Xq·Aq_i)/(sX·sA) (+ b1_i)
  {
    Fp8GemmArgs a{Xq, d, sc + 0, Aq, F, sc + 1, S, F, nullptr, nullptr,
                  nullptr, 0, nullptr, nullptr, m, f, dd};
    if (bias) a.bias = static_cast<const uint16_t*>(b1) + (int64_t)rank * F;
    run(tpmlp::launch_gemm_fp8(a, bias ? OutKind::F32Bias : OutKind::F32, E4, E4, s));
  }
  // dS = bf16(((dYq·Bq_iᵀ)/(sdY·sB)) ⊙ GeLU'(S)), Z = bf16(GeLU(S)), their amaxes
  run(tpmlp::launch_gemm_fp8(Fp8GemmArgs{dYq, d, sc + 3, BqT, F, sc + 2, dS, F, am + 4, nullptr,
                                         S, F, Z, am + 5, m, f, dd},
                             OutKind::GeluGradBf16, E5, E4, s, false));
  // db1_i = Σ_m dS[m, :] from the bf16 dS, before its e5m2 quantisation
  if (bias)
    run(tpmlp::launch_colsum_bf16(dS, F, m, f, db1_i, reinterpret_cast<float*>(ws + L.total), s));
  run(tpmlp::launch_quant_fp8(E5, dS, M * F, am + 4, dSq, sc + 4, s));
  run(tpmlp::launch_quant_fp8_tile(E4, Z, F, m, f, am + 5, nullptr, 0, ZqT, M, sc + 5, s));
  // dX_i = (dSq·Aq_iᵀ)/(sdS·sA)
  run(tpmlp::launch_gemm_fp8(Fp8GemmArgs{dSq, F, sc + 4, AqT, d, sc + 1, dX_i, d, nullptr,
                                         nullptr, nullptr, 0, nullptr, nullptr, m, dd, f},
                             OutKind::F32, E5, E4, s));
  // dB_i = (Zqᵀ·dYq)/(sZ·sdY) and dA_i = (Xqᵀ·dSq)/(sX·sdS) in one launch: each
  // alone has too few output tiles to fill the chip
  run(tpmlp::launch_gemm_fp8_pair(
      Fp8GemmArgs{ZqT, M, sc + 5, dYq, d, sc + 3, dB_i, d, nullptr, nullptr, nullptr, 0, nullptr,
                  nullptr, f, dd, m},
      Fp8GemmArgs{XqT, M, sc + 0, dSq, F, sc + 4, dA_i, F, nullptr, nullptr, nullptr, 0, nullptr,
                  nullptr, dd, f, m},
      OutKind::F32, E4, E5, s));
  return status_of(e);
}
}  // namespace

int tp_mlp_shard_backward_fp8(const void* X, const void* A, const void* B, const void* dY,
                              float* dX_i, float* dA_i, float* dB_i, int64_t M, int64_t d,
                              int64_t H, int N, int rank, const float* w_amax, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return shard_backward_fp8(X, A, B, dY, nullptr, dX_i, dA_i, dB_i, nullptr, M, d, H, N, rank,
                            w_amax, workspace, workspace_bytes, stream);
}

size_t tp_mlp_shard_backward_fp8_bias_workspace_size(int64_t M, int64_t d, int64_t H, int N) {
  const size_t base = tp_mlp_shard_backward_fp8_workspace_size(M, d, H, N);
  if (base == 0) return 0;
  return base + round256((size_t)tpmlp::colsum_row_blocks(M) * (size_t)(H / N) * 4);
}

int tp_mlp_shard_backward_fp8_bias(const void* X, const void* A, const void* b1, const void* B,
                                   const void* dY, float* dX_i, float* dA_i, float* dB_i,
                                   float* db1_i, int64_t M, int64_t d, int64_t H, int N, int rank,
                                   const float* w_amax, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  return shard_backward_fp8(X, A, B, dY, b1, dX_i, dA_i, dB_i, db1_i, M, d, H, N, rank, w_amax,
                            workspace, workspace_bytes, stream);
}

int tp_attn_qkv(const void* X, const void* W_i, int64_t ldw, void* QKV_i, int64_t M, int64_t d,
                int64_t F3, void* stream) {
  int st = check_dims(M, d, F3, 8);
  if (st != TPM_OK) return st;
  if (ldw < F3 || ldw > kMaxLd) return TPM_ERR_SHAPE;
  if (M == 0) return TPM_OK;
  if (!X || !W_i || !QKV_i) return TPM_ERR_NULL;
  if (!aligned16(X) || !aligned16(W_i) || !aligned16(QKV_i) || ldw % 8 != 0) return TPM_ERR_ALIGN;
  const Span q = mat_span(QKV_i, M, F3, F3, 2);
  if (overlap(q, mat_span(X, M, d, d, 2)) || overlap(q, mat_span(W_i, d, F3, ldw, 2)))
    return TPM_ERR_ALIAS;
  return status_of(tpmlp::launch_gemm_bf16(static_cast<const uint16_t*>(X), d,
                                           static_cast<const uint16_t*>(W_i), ldw, QKV_i, F3,
                                           (int)M, (int)F3, (int)d, OutKind::Bf16,
                                           as_stream(stream)));
}

int tp_attn_heads(const void* QKV, int64_t ld, void* O, int64_t ldo, int64_t B, int64_t S,
                  int64_t heads, int causal, void* stream) {
  if (B < 0 || S < 0 || heads < 1 || heads > 65536) return TPM_ERR_SHAPE;
  if (ld < 3 * heads * TPM_ATTN_HEAD_DIM || ldo < heads * TPM_ATTN_HEAD_DIM) return TPM_ERR_SHAPE;
  if (ld > kMaxLd || ldo > kMaxLd) return TPM_ERR_SHAPE;
  // per-sequence byte offsets of the key/value loads are 32-bit
  if (S > 0 && ((S - 1) * ld + ld) * 2 >= (int64_t(1) << 32)) return TPM_ERR_SHAPE;
  const int64_t M = B * S;
  if (M > kMaxDim || (M > 0 && ((M + 127) / 128) * heads > kMaxDim)) return TPM_ERR_SHAPE;
  if (M == 0) return TPM_OK;
  if (!QKV || !O) return TPM_ERR_NULL;
  if (!aligned16(QKV) || !aligned16(O) || ld % 8 != 0 || ldo % 8 != 0) return TPM_ERR_ALIGN;
  if (overlap(mat_span(O, M, heads * TPM_ATTN_HEAD_DIM, ldo, 2),
              mat_span(QKV, M, 3 * heads * TPM_ATTN_HEAD_DIM, ld, 2)))
    return TPM_ERR_ALIAS;
  return status_of(tpmlp::launch_attention(static_cast<const uint16_t*>(QKV), ld,
                                           static_cast<uint16_t*>(O), ldo, (int)B, (int)S,
                                           (int)heads, causal != 0, as_stream(stream)));
}

size_t tp_attn_shard_workspace_size(int64_t M, int64_t d, int N) {
  if (M < 0 || d <= 0 || N < 1 || d % N != 0 || M > kMaxDim) return 0;
  const size_t mf = (size_t)M * (size_t)(d / N);
  return round256(mf * 6) + round256(mf * 2);
}

int tp_attn_shard(const void* X, const void* Wqkv, const void* Wo, void* Y_i, int y_dtype,
                  int64_t B, int64_t S, int64_t d, int64_t heads, int N, int rank, int causal,
                  void* workspace, size_t workspace_bytes, void* stream) {
  if (y_dtype != TPM_F32 && y_dtype != TPM_BF16) return TPM_ERR_DTYPE;
  if (N < 1 || rank < 0 || rank >= N) return TPM_ERR_ARG;
  if (B < 0 || S < 0 || d <= 0 || heads < 1) return TPM_ERR_SHAPE;
  if (d % heads != 0 || d / heads != TPM_ATTN_HEAD_DIM || heads % N != 0) return TPM_ERR_SHAPE;
  const int64_t F = d / N, hr = heads / N, M = B * S;
  int st = check_dims(M, d, 3 * F, 8);
  if (st != TPM_OK) return st;
  if (3 * d > kMaxLd || 3 * d * d > (int64_t(1) << 46)) return TPM_ERR_SHAPE;
  if (S > 0 && S * 3 * F * 2 >= (int64_t(1) << 32)) return TPM_ERR_SHAPE;
  if (M == 0) return TPM_OK;
  if (!X || !Wqkv || !Wo || !Y_i) return TPM_ERR_NULL;
  const size_t need = tp_attn_shard_workspace_size(M, d, N);
  if (!workspace || workspace_bytes < need) return TPM_ERR_WORKSPACE;
  if (!aligned16(X) || !aligned16(Wqkv) || !aligned16(Wo) || !aligned16(Y_i) ||
      !aligned16(workspace))
    return TPM_ERR_ALIGN;
  const Span sy = mat_span(Y_i, M, d, d, y_dtype == TPM_F32 ? 4 : 2);
  const Span sw = {reinterpret_cast<uintptr_t>(workspace),
                   reinterpret_cast<uintptr_t>(workspace) + need};
  const Span ins[3] = {mat_span(X, M, d, d, 2), mat_span(Wqkv, d, 3 * d, 3 * d, 2),
                       mat_span(Wo, d, d, d, 2)};
  for (const Span& in : ins)
    if (overlap(sy, in) || overlap(sw, in)) return TPM_ERR_ALIAS;
  if (overlap(sy, sw)) return TPM_ERR_ALIAS;

  // Rank i's heads [i·hr, (i+1)·hr): columns [i·3F, (i+1)·3F) of the
  // head-major W_qkv and rows [i·F, (i+1)·F) of W_o.
  const uint16_t* W_i = static_cast<const uint16_t*>(Wqkv) + (int64_t)rank * 3 * F;
  const uint16_t* Wo_i = static_cast<const uint16_t*>(Wo) + (int64_t)rank * F * d;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint16_t* QKV = reinterpret_cast<uint16_t*>(ws);
  uint16_t* O = reinterpret_cast<uint16_t*>(ws + round256((size_t)M * F * 6));
  hipStream_t s = as_stream(stream);
  hipError_t e = tpmlp::launch_gemm_bf16(static_cast<const uint16_t*>(X), d, W_i, 3 * d, QKV,
                                         3 * F, (int)M, (int)(3 * F), (int)d, OutKind::Bf16, s);
  if (e == hipSuccess)
    e = tpmlp::launch_attention(QKV, 3 * F, O, F, (int)B, (int)S, (int)hr, causal != 0, s);
  if (e == hipSuccess)
    e = tpmlp::launch_gemm_bf16(O, F, Wo_i, d, Y_i, d, (int)M, (int)d, (int)F,
                                y_dtype == TPM_F32 ? OutKind::F32 : OutKind::Bf16, s);
  return status_of(e);
}

}  // extern "C"
