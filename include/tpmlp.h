/*
 * tpmlp.h - one tensor-parallel rank's share of the Megatron MLP block on an
 * AMD Instinct MI355X (gfx950), as a C ABI.
 *
 * The block is Y = GeLU(X·A)·B with A [d, 4d] and B [4d, d]. With N-way tensor
 * parallelism the first weight is split by columns and the second by rows;
 * rank i holds A_i = A[:, i·F:(i+1)·F] and B_i = B[i·F:(i+1)·F, :], F = 4d/N
 * ("Megatron architecture and 6D parallel guide", §3.1 tensor-parallel
 * principle, TP=2 example). Each rank computes Z_i = GeLU(X·A_i) with no
 * exchange, because GeLU is elementwise, and its partial output
 * Y_i = Z_i·B_i; the block's output is the sum of the partials,
 * Y = Σ_i Y_i ("Megatron-LM deep architecture", column/row-parallel section,
 * eq. for Output). On the pages that sum is one AllReduce(sum); here it is a
 * plain on-device sum of partials computed one after another on one GPU.
 *
 * Conventions shared by every call:
 *  - Matrices are row-major. X is [M, d], Z_i is [M, F], Y_i and Y are [M, d];
 *    these are dense (row stride = column count). Weights use the math layout
 *    of the pages' formula (A: [d, H], B: [H, d]), not nn.Linear's [out, in].
 *  - Pointers named as device pointers must be device memory of the current
 *    HIP device; host pointers are named as such. All data pointers must be
 *    16-byte aligned and every row stride in bytes a multiple of 16, so d and
 *    F must be multiples of 8 for bf16 and of 16 for e4m3. Row strides (d, F,
 *    H, lda) are at most 2^23 elements. M is any value >= 1 (partial tiles
 *    are handled); M = 0 is a no-op that returns TPM_OK.
 *  - The caller owns every buffer and keeps it alive until the work on
 *    `stream` has finished. The library allocates nothing, keeps no pointers
 *    and has no global mutable state, with one stated exception:
 *    tp_mlp_shard_noalloc uses a static device array (and keeps its address
 *    per device). Outputs are overwritten, never accumulated, and must not
 *    overlap any input (TPM_ERR_ALIAS).
 *  - `stream` is a hipStream_t passed as void*; NULL means the default
 *    stream. Every call only enqueues work and returns; device faults surface
 *    at the caller's next synchronisation.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    non-zero status means no work was enqueued, except TPM_ERR_HIP, which
 *    reports a failed launch (work of earlier launches of the same call may
 *    have been enqueued).
 *  - bfloat16 rounding is round-to-nearest-even. GeLU is the exact form
 *    x·Φ(x) = ½·x·(1 + erf(x/√2)) (the pages name GeLU without defining it).
 */
#ifndef TPMLP_H
#define TPMLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TPM_ABI_VERSION 7

/* Element types. */
typedef enum {
  TPM_BF16 = 0, /* bfloat16 */
  TPM_F32 = 1,  /* IEEE binary32 */
  TPM_E4M3 = 2  /* OCP 8-bit float E4M3 ("E4M3FN": max 448, no inf) */
} tpm_dtype;

/* Status codes (all calls return int). */
typedef enum {
  TPM_OK = 0,
  TPM_ERR_NULL = -1,      /* a required pointer is NULL */
  TPM_ERR_ARG = -2,       /* N < 1, N > TPM_MAX_PARTS, rank not in [0, N) */
  TPM_ERR_SHAPE = -3,     /* negative or inconsistent sizes, H not divisible by N,
                             a width that is not a multiple of 8 (16 for e4m3) */
  TPM_ERR_DTYPE = -4,     /* unsupported element type for this call */
  TPM_ERR_ALIGN = -5,     /* pointer not 16-byte aligned, row stride not 16-byte multiple */
  TPM_ERR_WORKSPACE = -6, /* workspace NULL or smaller than the size query returns */
  TPM_ERR_ALIAS = -7,     /* an output overlaps an input */
  TPM_ERR_HIP = -8,       /* a HIP launch failed */
  TPM_ERR_SCRATCH = -9    /* tp_mlp_shard_noalloc: Z_i larger than its static scratch */
} tpm_status;

/* Largest number of partials tp_partial_sum accepts in one call. */
#define TPM_MAX_PARTS 64

int tp_abi_version(void);
/* Static string naming a status code; never NULL. */
const char* tp_status_string(int status);

/*
 * Column-parallel step ("Megatron-LM deep architecture", column-parallel
 * linear: every rank takes the same X and computes GeLU(X·W_1,i) locally).
 *   Z_i = bf16(GeLU(X · A_i)), accumulated in fp32, GeLU in fp32, one
 *   rounding to bf16 per element.
 * X   : device, bf16 [M, d], dense.
 * A_i : device, bf16 [d, F] with row stride lda >= F elements (lda = H when
 *       A_i is a column block of a full A [d, H]).
 * Z_i : device, bf16 [M, F], dense; written.
 */
int tp_mlp_col_gelu(const void* X, const void* A_i, int64_t lda, void* Z_i,
                    int64_t M, int64_t d, int64_t F, void* stream);

/*
 * Row-parallel step ("Megatron-LM deep architecture", row-parallel linear:
 * the local activation times the local row block of W_2 gives the partial).
 *   Y_i = Z_i · B_i, accumulated in fp32.
 * Z_i : device, bf16 [M, F], dense.
 * B_i : device, bf16 [F, d], dense (a row block of a full B is dense).
 * Y_i : device, [M, d], dense, y_dtype TPM_F32 (default) or TPM_BF16.
 */
int tp_mlp_row_partial(const void* Z_i, const void* B_i, void* Y_i, int y_dtype,
                       int64_t M, int64_t F, int64_t d, void* stream);

/*
 * Bytes of device workspace tp_mlp_shard needs (Z_i, bf16 [M, F], 256-byte
 * aligned). Returns 0 for invalid sizes.
 */
size_t tp_mlp_shard_workspace_size(int64_t M, int64_t d, int64_t H, int N);

/*
 * One rank's partial output of the N-way split MLP
 * ("Megatron architecture and 6D parallel guide", §3.1 forward pass:
 * Y_i = GeLU(X·A_i)·B_i on each GPU):
 *   F = H / N, A_i = A[:, rank·F : (rank+1)·F], B_i = B[rank·F : (rank+1)·F, :],
 *   Z_i = bf16(GeLU(X·A_i)) into the workspace, then Y_i = Z_i·B_i.
 * X : device, bf16 [M, d]. A : device, bf16 [d, H]. B : device, bf16 [H, d].
 * Pass N = 1, rank = 0 with A = A_i [d, F] and B = B_i [F, d] to run a shard
 * that is stored on its own.
 * Y_i : device, [M, d], y_dtype TPM_F32 or TPM_BF16.
 * workspace : device, at least tp_mlp_shard_workspace_size(M, d, H, N) bytes,
 *   16-byte aligned; its contents on return are Z_i.
 */
int tp_mlp_shard(const void* X, const void* A, const void* B, void* Y_i, int y_dtype,
                 int64_t M, int64_t d, int64_t H, int N, int rank,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free form of tp_mlp_shard, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments without the workspace, the same
 * kernels and the same results, bit for bit. Z_i is kept in a static device
 * array of TPM_NOALLOC_SCRATCH_BYTES that the library holds on each device it
 * runs on until the process ends (its address is looked up on the first call
 * on a device). The call allocates nothing. Z_i must fit:
 * tp_mlp_shard_workspace_size(M, d, H, N) <= TPM_NOALLOC_SCRATCH_BYTES, else
 * TPM_ERR_SCRATCH (checked on the host, nothing enqueued). Every call on one
 * device shares that array: calls that overlap in time on one device (on
 * different streams, or from several host threads without ordering) race on
 * it and must not be issued. The array keeps the last call's Z_i.
 */
#define TPM_NOALLOC_SCRATCH_BYTES (64 * 1024 * 1024)
int tp_mlp_shard_noalloc(const void* X, const void* A, const void* B, void* Y_i, int y_dtype,
                         int64_t M, int64_t d, int64_t H, int N, int rank, void* stream);

/*
 * ---------------------------------------------------------------------------
 * Measurement calls: the forward's GEMM steps with per-workgroup clock stamps,
 * so the shader clock the kernel actually ran at can be reported beside its
 * throughput (the MFMA peak scales with that clock). Each is the production
 * kernel of tp_mlp_col_gelu / tp_mlp_row_partial / tp_mlp_row_partial_e4m3
 * (same tile choice, same results), given a stamps array: workgroup w writes
 * stamps[4w .. 4w+3] = {shader-clock counter at its start, constant 100 MHz
 * counter at its start, shader-clock counter once its stores have completed,
 * 100 MHz counter then}. Entries of workgroups the launch does not have are
 * left as they were (zero them first to count the workgroups).
 * stamps : device, 16-byte aligned, stamp_count >= tp_clock_stamp_count(M, N)
 *   values (M, N: rows and columns of the step's output), else
 *   TPM_ERR_WORKSPACE; it must not overlap any other argument.
 * ---------------------------------------------------------------------------
 */
int64_t tp_clock_stamp_count(int64_t M, int64_t N);
int tp_mlp_col_gelu_stamped(const void* X, const void* A_i, int64_t lda, void* Z_i,
                            int64_t M, int64_t d, int64_t F, uint64_t* stamps,
                            int64_t stamp_count, void* stream);
int tp_mlp_row_partial_stamped(const void* Z_i, const void* B_i, void* Y_i, int y_dtype,
                               int64_t M, int64_t F, int64_t d, uint64_t* stamps,
                               int64_t stamp_count, void* stream);
int tp_mlp_row_partial_e4m3_stamped(const void* Zq, const float* sZ, const void* Bq_i,
                                    const float* sB, void* Y_i, int64_t M, int64_t F,
                                    int64_t d, uint64_t* stamps, int64_t stamp_count,
                                    void* stream);

/*
 * ---------------------------------------------------------------------------
 * The same forward with the weights stored as their transposes, the
 * [out_features, in_features] layout of the linear layers in the pages'
 * column- and row-parallel code pattern ("Megatron-LM deep architecture",
 * code-pattern section): W1 = Aᵀ [H, d] and W2 = Bᵀ [d, H]. Rank i's
 * shards are W1_i = W1[i·F : (i+1)·F, :] (a block of rows) and
 * W2_i = W2[:, i·F : (i+1)·F] (a block of columns); the products and the
 * outputs are those of the math-layout calls above, to the bit.
 * ---------------------------------------------------------------------------
 */

/*
 * Z_i = bf16(GeLU(X · W1_iᵀ)). X : device, bf16 [M, d], dense.
 * W1_i : device, bf16 [F, d], row stride ldw >= d (a row block of W1).
 * Z_i : device, bf16 [M, F], dense. Errors as for tp_mlp_col_gelu.
 */
int tp_mlp_col_gelu_wt(const void* X, const void* W1_i, int64_t ldw, void* Z_i, int64_t M,
                       int64_t d, int64_t F, void* stream);

/*
 * Y_i = Z_i · W2_iᵀ, accumulated in fp32. Z_i : device, bf16 [M, F], dense.
 * W2_i : device, bf16 [d, F], row stride ldw >= F (a column block of W2 has
 * ldw = H). Y_i : device, [M, d], dense, y_dtype TPM_F32 or TPM_BF16.
 */
int tp_mlp_row_partial_wt(const void* Z_i, const void* W2_i, int64_t ldw, void* Y_i,
                          int y_dtype, int64_t M, int64_t F, int64_t d, void* stream);

/*
 * tp_mlp_shard with W1 = Aᵀ : device, bf16 [H, d] and W2 = Bᵀ : device,
 * bf16 [d, H], both dense; the workspace is sized by
 * tp_mlp_shard_workspace_size and holds Z_i on return.
 */
int tp_mlp_shard_wt(const void* X, const void* W1, const void* W2, void* Y_i, int y_dtype,
                    int64_t M, int64_t d, int64_t H, int N, int rank, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * ---------------------------------------------------------------------------
 * The column-parallel linear with its bias ("Megatron-LM deep architecture",
 * code-pattern section: the column-parallel layer holds a bias of its own
 * output width, H/N values per rank, and adds it inside the linear, so
 * before the GeLU that the column/row-parallel section applies to its
 * output):
 *   Z_i = bf16(GeLU(X·A_i + b1_i)), b1_i = b1[i·F : (i+1)·F].
 * The sum is taken in fp32 (the fp32 accumulator plus the bias, one
 * rounding), then GeLU, then one RNE rounding to bf16. The second layer's
 * bias is added once, after the sum of the partials (tp_partial_sum_rows).
 * ---------------------------------------------------------------------------
 */

/*
 * X : device, bf16 [M, d], dense. A_i : device, bf16 [d, F], row stride
 * lda >= F (the math layout, as tp_mlp_col_gelu). b_i : device, bf16 [F],
 * 16-byte aligned (a block of b1 at an offset of i·F elements, F a multiple
 * of 8). Z_i : device, bf16 [M, F], dense; must not overlap X, A_i or b_i.
 * Errors as for tp_mlp_col_gelu, and TPM_ERR_NULL when b_i is NULL.
 */
int tp_mlp_col_gelu_bias(const void* X, const void* A_i, int64_t lda, const void* b_i, void* Z_i,
                         int64_t M, int64_t d, int64_t F, void* stream);

/*
 * The same with W1_i : device, bf16 [F, d], row stride ldw >= d (the
 * [out, in] layout of tp_mlp_col_gelu_wt).
 */
int tp_mlp_col_gelu_bias_wt(const void* X, const void* W1_i, int64_t ldw, const void* b_i,
                            void* Z_i, int64_t M, int64_t d, int64_t F, void* stream);

/*
 * Backward of one rank's shard when the forward had the column layer's bias
 * (tp_mlp_col_gelu_bias): as tp_mlp_shard_backward, with S = X·A_i + b1_i
 * recomputed, and also
 *   db1_i = Σ_m dS[m, :]   (the gradient of this rank's block of b1)
 * ("Megatron-LM deep architecture", code pattern: the column layer's bias
 * is added to every token's output, so its gradient sums the gradient at
 * that output over the tokens; dS is the gradient at GeLU's input, summed
 * as the bf16 values the other gradients use, in fp32).
 * b1 : device, bf16 [H], the whole first bias (the rank's block is taken at
 *   rank·F). db1_i : device, fp32 [F], written. The second layer's bias
 *   gradient, the same on every rank, is tp_bias_grad_bf16 of dY.
 * workspace : tp_mlp_shard_backward_bias_workspace_size bytes. M = 0 writes
 * db1_i = 0 and nothing else. Errors as tp_mlp_shard_backward, and
 * TPM_ERR_NULL when b1 or db1_i is NULL.
 */
size_t tp_mlp_shard_backward_bias_workspace_size(int64_t M, int64_t d, int64_t H, int N);
int tp_mlp_shard_backward_bias(const void* X, const void* A, const void* b1, const void* B,
                               const void* dY, float* dX_i, float* dA_i, float* dB_i,
                               float* db1_i, int64_t M, int64_t d, int64_t H, int N, int rank,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * The fp8 backward (tp_mlp_shard_backward_fp8) when the forward had the
 * column layer's bias: the rank's block of b1 (bf16, not quantised) is added
 * to the dequantised S, and db1_i = Σ_m dS[m, :] is taken over the bf16 dS
 * before its e5m2 quantisation (the higher-precision gradient), in fp32.
 * Arguments as tp_mlp_shard_backward_fp8 plus b1 (device, bf16 [H]) and
 * db1_i (device, fp32 [F], written); workspace:
 * tp_mlp_shard_backward_fp8_bias_workspace_size bytes, laid out as the fp8
 * backward's with the bias-gradient scratch after it. M = 0 writes
 * db1_i = 0 and nothing else.
 */
size_t tp_mlp_shard_backward_fp8_bias_workspace_size(int64_t M, int64_t d, int64_t H, int N);
int tp_mlp_shard_backward_fp8_bias(const void* X, const void* A, const void* b1, const void* B,
                                   const void* dY, float* dX_i, float* dA_i, float* dB_i,
                                   float* db1_i, int64_t M, int64_t d, int64_t H, int N, int rank,
                                   const float* w_amax, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * Gradient of a bias added to every row of a layer's output:
 *   db[c] = Σ_r G[r, c], summed in fp32 (two passes, no atomics: the result
 *   does not depend on timing).
 * G : device, bf16 [rows, cols], row stride ld >= cols (a multiple of 8);
 *   cols a multiple of 8. db : device, fp32 [cols], written (0 when rows is
 *   0). workspace : tp_bias_grad_workspace_size(rows, cols) bytes of
 *   scratch (none needed when rows is 0); must not overlap G or db.
 * Used for the row layer's bias with G = dY. Errors: TPM_ERR_SHAPE,
 * TPM_ERR_NULL, TPM_ERR_WORKSPACE, TPM_ERR_ALIGN (16-byte pointers),
 * TPM_ERR_ALIAS.
 */
size_t tp_bias_grad_workspace_size(int64_t rows, int64_t cols);
int tp_bias_grad_bf16(const void* G, int64_t ld, int64_t rows, int64_t cols, float* db,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sum of the partial outputs, the arithmetic of the AllReduce(sum) that ends
 * the block ("Megatron-LM deep architecture", eq. for Output:
 * Output = Σ_i Y_i):
 *   Y = Σ_{i=0}^{N-1} parts[i], added in rank order in fp32.
 * parts : HOST array of N device pointers, each [numel] of part_dtype
 *   (TPM_F32 or TPM_BF16). 1 <= N <= TPM_MAX_PARTS.
 * Y : device, [numel] of y_dtype (TPM_F32 or TPM_BF16). Y may be exactly
 *   parts[0] (in-place) when the dtypes match; any other overlap is an error.
 */
int tp_partial_sum(const void* const* parts, int N, int part_dtype, void* Y, int y_dtype,
                   int64_t numel, void* stream);

/*
 * A block of rows of the sum of the partial outputs, plus an optional bias
 * added once, after the sum:
 *   Y[r - row_begin, c] = (Σ_{i=0}^{N-1} parts[i][r, c]) + bias[c],
 *   r in [row_begin, row_end), added in rank order in fp32, bias last.
 * Under sequence parallelism the AllReduce that ends the block becomes a
 * ReduceScatter that leaves each GPU the sum over its own slice of the
 * sequence ("Megatron-LM deep architecture", sequence-parallel section:
 * AllReduce = AllGather(ReduceScatter)); with tokens stored sequence-major
 * ([S, B, H]), rank j's share is rows [j·M/N, (j+1)·M/N). The bias of the
 * row-parallel linear is added once, after the reduction (same page, code
 * pattern of the row-parallel linear), never per partial. row_begin = 0,
 * row_end = M with a bias is the all-reduce form.
 * parts : HOST array of N device pointers, each [M, d] dense of part_dtype
 *   (TPM_F32 or TPM_BF16); 1 <= N <= TPM_MAX_PARTS. d is a multiple of 8.
 * bias : device [d] of bias_dtype (TPM_F32 or TPM_BF16), or NULL (then
 *   bias_dtype is ignored).
 * Y : device [row_end - row_begin, d] dense of y_dtype (TPM_F32 or
 *   TPM_BF16). Y may be exactly the first row of the block in parts[0]
 *   (in place) when the dtypes match; any other overlap is an error.
 * 0 <= row_begin <= row_end <= M; an empty range is a no-op.
 */
int tp_partial_sum_rows(const void* const* parts, int N, int part_dtype, int64_t M, int64_t d,
                        int64_t row_begin, int64_t row_end, const void* bias, int bias_dtype,
                        void* Y, int y_dtype, void* stream);

/*
 * Rank `rank`'s share of the sequence-parallel reduce-scatter of the N
 * partial outputs ("Megatron-LM deep architecture", sequence-parallel
 * section: the AllReduce ending the block becomes a ReduceScatter, and each
 * GPU keeps the sum over its 1/N of the sequence): tp_partial_sum_rows over
 * rows [rank·M/N, (rank+1)·M/N), bias added once. Tokens are stored
 * sequence-major ([S, B, H]), so that share is one contiguous row block.
 * Arguments as tp_partial_sum_rows; Y is [M/N, d]. rank not in [0, N):
 * TPM_ERR_ARG; M not divisible by N: TPM_ERR_SHAPE.
 */
int tp_reduce_scatter_share(const void* const* parts, int N, int part_dtype, int64_t M,
                            int64_t d, int rank, const void* bias, int bias_dtype, void* Y,
                            int y_dtype, void* stream);

/* ------------------------------------------------------------------------
 * fp8 e4m3 variant ("Megatron-LM deep architecture", FP8 hybrid precision:
 * E4M3 for forward activation×weight GEMMs, each tensor scaled by a factor
 * derived from its amax). Current scaling: a tensor's scale is
 * s = 448 / amax(tensor), an fp32 division (s = 1 when amax = 0); a value t is
 * stored as e4m3(clamp(fp32(t·s), ±448)), rounded to nearest even; a GEMM of
 * two quantised operands is divided by the product of their scales.
 * Scales live in device memory as fp32 s (not 1/s).
 * ------------------------------------------------------------------------ */

/*
 * amax[0] = max |T| over numel bf16 values (device T, device amax).
 * amax is overwritten (the call clears it itself on the stream).
 */
int tp_amax_bf16(const void* T, int64_t numel, float* amax, void* stream);

/*
 * Quantise a bf16 tensor with the scale derived from a device amax:
 * scale[0] = s = 448/amax[0] (1 if amax[0] == 0); Tq[j] = e4m3(T[j]·s).
 * T : device bf16 [numel]; amax : device fp32 [1]; Tq : device e4m3 [numel];
 * scale : device fp32 [1], written. numel must be a multiple of 16.
 */
int tp_quant_e4m3(const void* T, int64_t numel, const float* amax, void* Tq, float* scale,
                  void* stream);

/*
 * fp8 column-parallel step: Z_i = bf16(GeLU((Xq·Aq_i) / (sX·sA))) and, when
 * z_amax is not NULL, z_amax[0] = max |Z_i| (the call clears it first).
 * Xq : device e4m3 [M, d]; Aq_i : device e4m3 [d, F], row stride lda;
 * sX, sA : device fp32 [1] scales; Z_i : device bf16 [M, F].
 */
int tp_mlp_col_gelu_e4m3(const void* Xq, const float* sX, const void* Aq_i, int64_t lda,
                         const float* sA, void* Z_i, float* z_amax,
                         int64_t M, int64_t d, int64_t F, void* stream);

/*
 * fp8 row-parallel step: Y_i = bf16((Zq·Bq_i) / (sZ·sB)).
 * Zq : device e4m3 [M, F]; Bq_i : device e4m3 [F, d]; sZ, sB : device fp32 [1];
 * Y_i : device bf16 [M, d].
 */
int tp_mlp_row_partial_e4m3(const void* Zq, const float* sZ, const void* Bq_i,
                            const float* sB, void* Y_i, int64_t M, int64_t F, int64_t d,
                            void* stream);

/* Bytes of workspace tp_mlp_shard_e4m3 needs: Z (bf16), Zq (e4m3), amax and
 * scale of Z. Returns 0 for invalid sizes. */
size_t tp_mlp_shard_e4m3_workspace_size(int64_t M, int64_t d, int64_t H, int N);

/*
 * fp8 partial output of one rank: with F = H/N and the rank's blocks of the
 * quantised A [d, H] and B [H, d] (one scale per whole tensor):
 *   Z = bf16(GeLU((Xq·Aq_i)/(sX·sA))), amax_Z = max|Z|, sZ = 448/amax_Z,
 *   Zq = e4m3(Z·sZ), Y_i = bf16((Zq·Bq_i)/(sZ·sB)).
 * Y_i : device bf16 [M, d]. Workspace as for tp_mlp_shard, sized by
 * tp_mlp_shard_e4m3_workspace_size; on return it holds Z, Zq, amax_Z, sZ.
 */
int tp_mlp_shard_e4m3(const void* Xq, const float* sX, const void* Aq, const float* sA,
                      const void* Bq, const float* sB, void* Y_i,
                      int64_t M, int64_t d, int64_t H, int N, int rank,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * fp8 delayed scaling ("Megatron-LM deep architecture", FP8 hybrid precision
 * and delayed scaling: the scale a step applies is predicted from the moving
 * average of the amaxes measured in earlier steps instead of the tensor's own
 * amax, so it is known before the tensor is produced). Here it is applied to
 * Z, the one tensor quantised inside the path: the column-parallel GEMM
 * quantises Z in its epilogue with the predicted scale and records the step's
 * amax, which tp_amax_history_push adds to the history.
 * Z is still rounded to bf16 after GeLU and before the scale is applied, so
 * with the same scale the codes equal those of the current-scaling path.
 * ------------------------------------------------------------------------ */

/* Longest amax history a tensor may keep. */
#define TPM_MAX_HISTORY 65536

/*
 * Record one step's amax and derive the next step's scale.
 * history : device fp32 [L], a ring of the recorded amaxes (zero it, with
 *   count, before the first step).
 * count : device uint32 [1], the number of steps recorded so far.
 * The call writes amax[0] into history[count % L], increments count, and sets
 * next_scale[0] = 448 / mean of the last min(count, L) recorded amaxes (the
 * mean in fp32; 1 when it is 0). amax, next_scale: device fp32 [1].
 * 1 <= L <= TPM_MAX_HISTORY. Calls on one history must be ordered on a
 * stream (each reads what the previous wrote).
 */
int tp_amax_history_push(float* history, uint32_t* count, int L, const float* amax,
                         float* next_scale, void* stream);

/*
 * fp8 column-parallel step with a given scale for Z:
 *   Z = bf16(GeLU((Xq·Aq_i)/(sX·sA))), Zq_i = e4m3(clamp(fp32(Z·sZ), ±448)),
 *   z_amax[0] = max|Z| (the call clears it first; never NULL here).
 * Xq : device e4m3 [M, d]; Aq_i : device e4m3 [d, F], row stride lda;
 * sX, sA, sZ : device fp32 [1]; Zq_i : device e4m3 [M, F], dense.
 */
int tp_mlp_col_gelu_e4m3_delayed(const void* Xq, const float* sX, const void* Aq_i, int64_t lda,
                                 const float* sA, const float* sZ, void* Zq_i, float* z_amax,
                                 int64_t M, int64_t d, int64_t F, void* stream);

/* Bytes of workspace tp_mlp_shard_e4m3_delayed needs (Zq, e4m3 [M, F]).
 * Returns 0 for invalid sizes. */
size_t tp_mlp_shard_e4m3_delayed_workspace_size(int64_t M, int64_t d, int64_t H, int N);

/*
 * fp8 partial output of one rank with Z quantised by the given scale sZ:
 *   Zq = e4m3(bf16(GeLU((Xq·Aq_i)/(sX·sA)))·sZ), Y_i = bf16((Zq·Bq_i)/(sZ·sB)),
 *   z_amax[0] = max|Z| (to be recorded with tp_amax_history_push).
 * Shapes and the shard map as for tp_mlp_shard_e4m3. The workspace holds Zq
 * on return.
 */
int tp_mlp_shard_e4m3_delayed(const void* Xq, const float* sX, const void* Aq, const float* sA,
                              const void* Bq, const float* sB, const float* sZ, void* Y_i,
                              float* z_amax, int64_t M, int64_t d, int64_t H, int N, int rank,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace tp_mlp_shard_backward needs: S (fp32 [M, F]),
 * dS and Z (bf16 [M, F] each), each 256-byte aligned. 0 for invalid sizes.
 */
size_t tp_mlp_shard_backward_workspace_size(int64_t M, int64_t d, int64_t H, int N);

/*
 * Backward of one rank's shard: the chain rule through Y_i = GeLU(X·A_i)·B_i
 * for the output gradient dY. The pages give the backward's communication
 * only ("Megatron-LM" glossary and "Megatron architecture and 6D parallel
 * guide", tensor-parallel communication: AllReduces in the backward pass):
 * every rank receives the same dY because the forward ends in a sum, and the
 * ranks' input gradients dX_i are summed because X is replicated. The
 * arithmetic is the chain rule through the forward as computed. With
 * F = H / N and the shard views of tp_mlp_shard:
 *   S    = X·A_i                     recomputed in fp32 (the forward keeps only Z)
 *   dS   = bf16((dY·B_iᵀ) ⊙ GeLU'(S)), GeLU'(x) = Φ(x) + x·φ(x)
 *   Z    = bf16(GeLU(S))             (bit-identical to the forward's Z_i)
 *   dX_i = dS·A_iᵀ                   this rank's part of the input gradient
 *   dA_i = Xᵀ·dS                     gradient of the column block A_i
 *   dB_i = Z ᵀ·dY                    gradient of the row block B_i
 * all accumulated in fp32. The input gradient is Σ_i dX_i (tp_partial_sum).
 * X, dY : device, bf16 [M, d]. A : device, bf16 [d, H]. B : device, bf16 [H, d].
 * dX_i : device, fp32 [M, d]. dA_i : device, fp32 [d, F]. dB_i : device, fp32 [F, d].
 *   All dense; overwritten; no output may overlap an input, another output
 *   or the workspace.
 * M must be a multiple of 8 (it is the contraction length of dA_i and dB_i).
 * workspace : device, at least tp_mlp_shard_backward_workspace_size(M, d, H, N)
 *   bytes, 16-byte aligned; on return it holds S, dS, Z in that order, each
 *   at a 256-byte-rounded offset.
 */
int tp_mlp_shard_backward(const void* X, const void* A, const void* B, const void* dY,
                          float* dX_i, float* dA_i, float* dB_i, int64_t M, int64_t d,
                          int64_t H, int N, int rank, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * Bytes of device workspace tp_mlp_shard_backward_fp8 needs; 0 for invalid sizes.
 */
size_t tp_mlp_shard_backward_fp8_workspace_size(int64_t M, int64_t d, int64_t H, int N);

/*
 * The backward of tp_mlp_shard_backward with fp8 GEMMs in the hybrid formats
 * ("Megatron-LM deep architecture", FP8 hybrid precision section: E4M3 for
 * activations and weights, E5M2, with its wider range, for the backward's
 * gradients). Each tensor is quantised with its own current amax scale,
 * s = 448/amax (e4m3) or 57344/amax (e5m2), values clamped to the format's
 * range, RNE: X, the whole of A and B (as in the fp8 forward) and Z in e4m3;
 * dY and dS in e5m2. With q(T) the codes and s_T the scale:
 *   S    = (q(X)·q(A)_i) / (s_X·s_A)                   (fp32)
 *   dS   = bf16(((q(dY)·q(B)_iᵀ) / (s_dY·s_B)) ⊙ GeLU'(S)),  Z = bf16(GeLU(S))
 *   dX_i = (q(dS)·q(A)_iᵀ) / (s_dS·s_A)
 *   dA_i = (q(X)ᵀ·q(dS)) / (s_X·s_dS),  dB_i = (q(Z)ᵀ·q(dY)) / (s_Z·s_dY)
 * all accumulated in fp32; the transposed operands are quantised straight
 * into their transposed layout. Arguments, layouts and outputs as for
 * tp_mlp_shard_backward; M, d and F = H/N must be multiples of 16.
 * w_amax : NULL, or device fp32 [2] = {max|A|, max|B|} over the whole weights
 *   (e.g. from tp_amax_bf16): the weights' amaxes do not change between the
 *   forward and the backward of a step, so a caller that already has them (or
 *   runs every rank's backward against the same weights) passes them instead
 *   of having every call read all of A and B again. NULL: computed here.
 * workspace : device, at least tp_mlp_shard_backward_fp8_workspace_size(M, d, H, N)
 *   bytes, 16-byte aligned; the first 64 bytes hold the amaxes of X, A, B, dY,
 *   dS, Z (floats 0-5; those of A and B only when computed here) and the
 *   scales of the six (floats 8-13).
 */
int tp_mlp_shard_backward_fp8(const void* X, const void* A, const void* B, const void* dY,
                              float* dX_i, float* dA_i, float* dB_i, int64_t M, int64_t d,
                              int64_t H, int N, int rank, const float* w_amax, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * ---------------------------------------------------------------------------
 * Attention shard. With h heads of width dh = d/h and N ranks, rank i owns
 * heads [i·h/N, (i+1)·h/N) and computes their attention with no exchange
 * ("Megatron-LM" glossary, tensor-parallel section: QKV projection column
 * parallel, attention head parallel, output projection row parallel with an
 * AllReduce; "Megatron architecture and 6D parallel guide", §3.2: 32 heads
 * at TP=8 give 4 per GPU). The fused projection weight W_qkv [d, 3d] is
 * stored head-major: columns [h·3dh, (h+1)·3dh) are head h's query, key and
 * value columns, so a rank's heads are one contiguous column block
 * [i·3F, (i+1)·3F), F = d/N. W_o [d, d]: rank i holds rows [i·F, (i+1)·F).
 * Tokens are batch-major: row b·S + t is token t of sequence b. The
 * attention kernels take dh = TPM_ATTN_HEAD_DIM only.
 * ---------------------------------------------------------------------------
 */
#define TPM_ATTN_HEAD_DIM 128

/*
 * Column-parallel QKV projection of one rank: QKV_i = bf16(X · W_i), fp32
 * accumulation, one rounding.
 * X : device, bf16 [M, d], dense. W_i : device, bf16 [d, F3] with row stride
 * ldw >= F3 (ldw = 3d for a column block of W_qkv). QKV_i : device, bf16
 * [M, F3], dense; written.
 */
int tp_attn_qkv(const void* X, const void* W_i, int64_t ldw, void* QKV_i, int64_t M,
                int64_t d, int64_t F3, void* stream);

/*
 * Attention of `heads` heads (dh = TPM_ATTN_HEAD_DIM) over B sequences of S
 * tokens: for sequence b and head j,
 *   O_bj = softmax(Q_bj·K_bjᵀ / √dh + mask)·V_bj,
 * mask = −inf where key > query when `causal` is non-zero, else none. Scores
 * and the softmax are fp32 (exp2 of scaled scores); the probabilities are
 * rounded to bf16 for the P·V product, whose fp32 sum is divided by the
 * fp32 sum of the unrounded probabilities; O is rounded to bf16 once.
 * QKV : device, bf16 [B·S, ld], head j's Q, K, V at columns 3j·dh, 3j·dh + dh,
 *   3j·dh + 2dh (ld >= 3·heads·dh, a multiple of 8; (S·ld·2) < 2^32).
 * O : device, bf16 [B·S, ldo], head j at columns [j·dh, (j+1)·dh) (ldo >=
 *   heads·dh, a multiple of 8); written; must not overlap QKV.
 */
int tp_attn_heads(const void* QKV, int64_t ld, void* O, int64_t ldo, int64_t B, int64_t S,
                  int64_t heads, int causal, void* stream);

/*
 * Bytes of device workspace tp_attn_shard needs (QKV_i, bf16 [M, 3F], then
 * O_i, bf16 [M, F], each 256-byte aligned). 0 for invalid sizes.
 */
size_t tp_attn_shard_workspace_size(int64_t M, int64_t d, int N);

/*
 * One rank's partial output of the N-way split attention block:
 *   QKV_i = bf16(X·W_qkv[:, i·3F:(i+1)·3F]), O_i = attention of its h/N heads,
 *   Y_i = O_i·W_o[i·F:(i+1)·F, :] (fp32 accumulation);
 * the block's output is Σ_i Y_i (tp_partial_sum), the AllReduce's sum.
 * X : device, bf16 [B·S, d]. W_qkv : device, bf16 [d, 3d] (head-major).
 * W_o : device, bf16 [d, d]. Y_i : device, [B·S, d], y_dtype TPM_F32 or TPM_BF16.
 * d / heads must equal TPM_ATTN_HEAD_DIM and N must divide heads.
 * workspace : device, at least tp_attn_shard_workspace_size(B·S, d, N) bytes,
 *   16-byte aligned; on return it holds QKV_i and O_i.
 */
int tp_attn_shard(const void* X, const void* Wqkv, const void* Wo, void* Y_i, int y_dtype,
                  int64_t B, int64_t S, int64_t d, int64_t heads, int N, int rank, int causal,
                  void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TPMLP_H */
