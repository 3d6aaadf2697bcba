/*
 * sgemm.h - single-precision general matrix multiply for AMD Instinct MI355X (gfx950).
 *
 * Computes C <- alpha * A * B + beta * C on row-major fp32 matrices:
 *
 *     A(i,k) = A[i*lda + k]    0 <= i < M, 0 <= k < K
 *     B(k,j) = B[k*ldb + j]    0 <= k < K, 0 <= j < N
 *     C(i,j) = C[i*ldc + j]    0 <= i < M, 0 <= j < N
 *
 * The operation is the BLAS-style form of the tiled kernels on the pages: the
 * product accumulated in a register tile, then alpha times it plus beta times the
 * old C, with C not read when beta is zero ("Micro_gemm_4x4 - cuBLAS micro GEMM
 * skeleton", sections "Kernel signature" and "Final C write (alpha, beta)").
 * Leading dimensions generalise the pages' packed A[row*K + k] indexing the way
 * the GPT-2 post's kernel takes strided views ("GPU Target - GPT-2 on the GPU",
 * section "Tiled matrix multiplication").
 *
 * Conventions shared by every entry point:
 *  - Pointers are device pointers (hipMalloc or torch CUDA tensors). The library
 *    never allocates, copies, frees or keeps them; the caller keeps every buffer
 *    alive until the work queued on `stream` has finished.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *    Calls are asynchronous: they queue one kernel (or none) and return.
 *  - Only the M x N window of C is written. Entries of C with column >= N in the
 *    ldc gap, and A and B, are never written.
 *  - When beta == 0, C is write-only: NaN or Inf already in C does not propagate.
 *    When alpha == 0 or K == 0, A and B are not read and C <- beta * C.
 *  - C must not overlap A or B.
 *  - Any alignment of at least 4 bytes is accepted. When A, B and C are 16-byte
 *    aligned, lda, ldb, ldc are multiples of 4 and so are N and K, the kernels use
 *    128-bit loads and stores; otherwise they use 32-bit ones. This is never an error.
 *  - Results match the exact product within 4*max(K,1)*2^-24*(|alpha|*sum_k|a_ik*b_kj|
 *    + |beta*c_ij|) per entry. For one configuration, sizes and alignment, results
 *    are bitwise reproducible from run to run.
 *
 * Return values: 0 on success; -i when argument i (1-based, in declaration order;
 * the first invalid one) is invalid; SGEMM_ERROR_TOO_LARGE, SGEMM_ERROR_BAD_CONFIG or
 * SGEMM_ERROR_WORKSPACE for the cases named below; a positive hipError_t when the kernel launch fails. Errors raised while
 * the kernel runs surface at the caller's next synchronisation. Nothing throws.
 */
#ifndef TILED_FP32_GEMM_SGEMM_H
#define TILED_FP32_GEMM_SGEMM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SGEMM_SUCCESS 0
/* The problem does not fit one launch: the tile count times the configuration's threads
 * per tile passes 2^32 - 1, or, for a stream-K configuration, the product has more than
 * 16384 tiles or (compute units + 1) x tiles x K-tiles reaches 2^31. */
#define SGEMM_ERROR_TOO_LARGE (-100)
/* sgemm_ex / sgemm_general: the configuration id is not in [-1, sgemm_config_count()). */
#define SGEMM_ERROR_BAD_CONFIG (-101)
/* A stream-K configuration was requested without a workspace of sgemm_workspace_size()
 * bytes (or for a strided-batched call, which stream-K does not serve). */
#define SGEMM_ERROR_WORKSPACE (-102)

/* Operand forms: read the matrix as stored, or its transpose. */
#define SGEMM_OP_N 0
#define SGEMM_OP_T 1

/* Activations applied after the bias (sgemm_bias_act, sgemm_general). */
#define SGEMM_ACT_NONE 0
/* tanh-form GELU: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))). */
#define SGEMM_ACT_GELU_TANH 1

/*
 * C <- alpha * A * B + beta * C (row-major fp32), on `stream`.
 *
 * Arguments, by 1-based position (the number returned as -i when invalid):
 *   1 M, 2 N, 3 K  >= 0. M == 0 or N == 0 returns 0 without touching any pointer.
 *   4 alpha        any float.
 *   5 A            device pointer; may be NULL only if A is not read (M == 0, N == 0,
 *                  K == 0 or alpha == 0).
 *   6 lda          >= max(1, K).
 *   7 B            device pointer; NULL allowed under the same condition as A.
 *   8 ldb          >= max(1, N).
 *   9 beta         any float.
 *  10 C            device pointer; NULL allowed only if M == 0 or N == 0.
 *  11 ldc          >= max(1, N).
 *  12 stream       hipStream_t or NULL.
 */
int sgemm(int M, int N, int K, float alpha,
          const float *A, int lda,
          const float *B, int ldb,
          float beta, float *C, int ldc,
          void *stream);

/*
 * Same as sgemm, with the kernel configuration chosen by the caller: `config` in
 * [0, sgemm_config_count()) forces that configuration, -1 picks it as sgemm does.
 * Argument positions in error codes are those of sgemm (config is not counted).
 * Used by tests and tuning sweeps.
 */
int sgemm_ex(int config, int M, int N, int K, float alpha,
             const float *A, int lda,
             const float *B, int ldb,
             float beta, float *C, int ldc,
             void *stream);

/*
 * C <- alpha * op(A) * op(B) + beta * C, with op(A) M x K and op(B) K x N, where
 *   opA == SGEMM_OP_N: op(A)(i,k) = A[i*lda + k]  (A stored M x K, lda >= max(1, K))
 *   opA == SGEMM_OP_T: op(A)(i,k) = A[k*lda + i]  (A stored K x M, lda >= max(1, M))
 *   opB == SGEMM_OP_N: op(B)(k,j) = B[k*ldb + j]  (B stored K x N, ldb >= max(1, N))
 *   opB == SGEMM_OP_T: op(B)(k,j) = B[j*ldb + k]  (B stored N x K, ldb >= max(1, K))
 * Transposed operands are read in place: the GPT-2 post's kernel takes transposed
 * views without copies ("GPU Target - GPT-2 on the GPU", section "Tiled matrix
 * multiplication"). The 128-bit path needs the stored rows' contiguous extent (K or M
 * for A, N or K for B) to be a multiple of 4; otherwise as for sgemm.
 *
 * Arguments by position: 1 opA, 2 opB, 3 M, 4 N, 5 K, 6 alpha, 7 A, 8 lda, 9 B, 10 ldb,
 * 11 beta, 12 C, 13 ldc, 14 stream. opA and opB must be SGEMM_OP_N or SGEMM_OP_T.
 */
int sgemm_op(int opA, int opB, int M, int N, int K, float alpha,
             const float *A, int lda,
             const float *B, int ldb,
             float beta, float *C, int ldc,
             void *stream);

/*
 * C <- act(alpha * op(A) * op(B) + beta * C + bias), with bias[j] added to column j
 * (bias has N entries, or is NULL for none) and act SGEMM_ACT_NONE or
 * SGEMM_ACT_GELU_TANH applied last. This is a GPT-2 linear layer, x @ W + b, optionally
 * followed by its GELU ("GPU Target - GPT-2 on the GPU", sections "The whole model as
 * one kernel" and "From loops to kernels"), fused into the product's final write.
 * With alpha == 0 or K == 0 the result is act(beta * C + bias).
 * Results match the oracle within 4*(max(K,1)+1)*2^-24*(|alpha|*sum|a*b| + |beta*c| +
 * |bias_j|), carried through GELU with a factor 1.13 plus 8*2^-24*(|t| + |gelu(t)|).
 *
 * Arguments by position: 1 opA, 2 opB, 3 M, 4 N, 5 K, 6 alpha, 7 A, 8 lda, 9 B, 10 ldb,
 * 11 beta, 12 C, 13 ldc, 14 bias, 15 act, 16 stream.
 */
int sgemm_bias_act(int opA, int opB, int M, int N, int K, float alpha,
                   const float *A, int lda,
                   const float *B, int ldb,
                   float beta, float *C, int ldc,
                   const float *bias, int act,
                   void *stream);

/*
 * sgemm_bias_act with the kernel configuration chosen by the caller (config as for
 * sgemm_ex; it is not counted in argument positions). Used by tests and sweeps.
 */
int sgemm_general(int config, int opA, int opB, int M, int N, int K, float alpha,
                  const float *A, int lda,
                  const float *B, int ldb,
                  float beta, float *C, int ldc,
                  const float *bias, int act,
                  void *stream);

/*
 * General-stride form: C <- act(alpha * A * B + beta * C + bias) on operands given by a row
 * and a column stride each (in floats):
 *   A(i,k) = A[i*rsA + k*csA], B(k,j) = B[k*rsB + j*csB], C(i,j) = C[i*rsC + j*csC].
 * The GPT-2 post's kernel takes operands with dynamic sizes, strides and offsets, so that
 * sliced and transposed views run without copies ("GPU Target - GPT-2 on the GPU",
 * section "Tiled matrix multiplication"); this is that form. Strides of A and B may be any
 * value >= 0 (0 repeats a row or column); C's must give distinct entries distinct
 * addresses (csC >= 1 and rsC >= (N-1)*csC + 1, or rsC >= 1 and csC >= (M-1)*rsC + 1).
 * Each operand's largest offset, (rows-1)*rs + (cols-1)*cs, must be below 2^60 floats
 * (else the row stride's position is returned).
 * Layouts with a unit stride in one dimension (the other at least the extent it spans)
 * run the stored-matrix kernels with the automatic choice, as sgemm_bias_act would; a
 * column-major C with no bias runs as the transposed product; every other layout runs a
 * register-staged tile kernel that reads and writes float by float. C must not overlap A
 * or B. No stream-K; nothing is allocated; results within the same bound as
 * sgemm_bias_act.
 *
 * Arguments by position: 1 M, 2 N, 3 K, 4 alpha, 5 A, 6 rsA, 7 csA, 8 B, 9 rsB, 10 csB,
 * 11 beta, 12 C, 13 rsC, 14 csC, 15 bias, 16 act, 17 stream. Returns -i for invalid
 * argument i (a C window whose entries would share addresses is reported as 13), 0 on
 * success, SGEMM_ERROR_TOO_LARGE past the launch limits, or a positive hipError_t.
 */
int sgemm_strided(int M, int N, int K, float alpha,
                  const float *A, long long rsA, long long csA,
                  const float *B, long long rsB, long long csB,
                  float beta, float *C, long long rsC, long long csC,
                  const float *bias, int act,
                  void *stream);

/*
 * Strided-batched form: for b in [0, batch), C_b <- alpha * A_b * B_b + beta * C_b with
 * A_b = A + b*strideA, B_b = B + b*strideB, C_b = C + b*strideC (strides in floats).
 * All batches share M, N, K, the leading dimensions and the scalars. The batched
 * product of the GPT-2 post's attention heads, which adds a third grid dimension
 * indexed by batch ("GPU Target - GPT-2 on the GPU", section "Tiled matrix
 * multiplication").
 *
 * Arguments by position: 1 M, 2 N, 3 K, 4 alpha, 5 A, 6 lda, 7 strideA, 8 B, 9 ldb,
 * 10 strideB, 11 beta, 12 C, 13 ldc, 14 strideC, 15 batch, 16 stream.
 * batch >= 0 and at most 65535; batch == 0 returns 0. strideA, strideB >= 0 (0 reuses
 * one matrix for all batches), and (batch-1) times each stride at most 2^60 floats. The C
 * windows must not overlap, unless batch == 1:
 * strideC >= (M-1)*ldc + N (stacked), or N <= strideC and (batch-1)*strideC + N <= ldc
 * (side by side within each row). Other rules as for sgemm.
 */
int sgemm_strided_batched(int M, int N, int K, float alpha,
                          const float *A, int lda, long long strideA,
                          const float *B, int ldb, long long strideB,
                          float beta, float *C, int ldc, long long strideC,
                          int batch, void *stream);

/*
 * Strided-batched form with operand forms: for b in [0, batch),
 *   C_b <- alpha * op(A_b) * op(B_b) + beta * C_b,
 * A_b = A + b*strideA, B_b = B + b*strideB, C_b = C + b*strideC (strides in floats), op
 * as for sgemm_op (a transposed operand is read in place). This is the per-head product of
 * attention in the GPT-2 post: its batched kernel adds a grid dimension indexed by batch,
 * and takes strided and transposed views without copies ("GPU Target - GPT-2 on the GPU",
 * section "Tiled matrix multiplication"). With Q, K and V the three 768-column blocks of a
 * 1024 x 2304 row-major QKV matrix (12 heads of 64 columns):
 *   scores_h = Q_h K_h^T / 8:  opA = N, opB = T, M = N = 1024, K = 64, alpha = 0.125,
 *       A = QKV, lda = 2304, strideA = 64; B = QKV + 768, ldb = 2304, strideB = 64;
 *       C = S (12 x 1024 x 1024), ldc = 1024, strideC = 1024 * 1024;
 *   out_h = P_h V_h:           opA = opB = N, M = 1024, N = 64, K = 1024,
 *       A = P, lda = 1024, strideA = 1024 * 1024; B = QKV + 1536, ldb = 2304, strideB = 64;
 *       C = O (1024 x 768), ldc = 768, strideC = 64 (heads side by side in each row).
 *
 * Arguments by position: 1 opA, 2 opB, 3 M, 4 N, 5 K, 6 alpha, 7 A, 8 lda, 9 strideA, 10 B,
 * 11 ldb, 12 strideB, 13 beta, 14 C, 15 ldc, 16 strideC, 17 batch, 18 stream.
 *  - strideA, strideB >= 0 (0 reuses one matrix for every batch); lda and ldb follow op.
 *  - batch in [0, 65535]; batch == 0 returns 0.
 *  - The C windows must not overlap (unless batch == 1): either stacked,
 *    strideC >= (M-1)*ldc + N, or side by side within each row, N <= strideC and
 *    (batch-1)*strideC + N <= ldc. Otherwise -16.
 *  - The 128-bit path needs the strides to be multiples of 4, besides the rules of sgemm_op.
 * The library never picks a stream-K configuration for a batched call.
 */
int sgemm_strided_batched_op(int opA, int opB, int M, int N, int K, float alpha,
                             const float *A, int lda, long long strideA,
                             const float *B, int ldb, long long strideB,
                             float beta, float *C, int ldc, long long strideC,
                             int batch, void *stream);

/*
 * sgemm_strided_batched_op with a forced configuration (config as for sgemm_ex, not
 * counted in argument positions; a stream-K configuration returns SGEMM_ERROR_WORKSPACE),
 * a bias and an activation applied to every batch as in sgemm_bias_act (bias has N
 * entries, shared by all batches, or is NULL):
 *   C_b <- act(alpha * op(A_b) * op(B_b) + beta * C_b + bias).
 * Used by tests and sweeps, and by batched linear layers.
 *
 * Arguments by position: 1 opA, 2 opB, 3 M, 4 N, 5 K, 6 alpha, 7 A, 8 lda, 9 strideA, 10 B,
 * 11 ldb, 12 strideB, 13 beta, 14 C, 15 ldc, 16 strideC, 17 bias, 18 act, 19 batch, 20 stream.
 */
int sgemm_strided_batched_general(int config, int opA, int opB, int M, int N, int K, float alpha,
                                  const float *A, int lda, long long strideA,
                                  const float *B, int ldb, long long strideB,
                                  float beta, float *C, int ldc, long long strideC,
                                  const float *bias, int act,
                                  int batch, void *stream);

/*
 * sgemm_general with a workspace, which lets the library use stream-K configurations
 * (names starting "sk_" or "sk16_"). Those split the product's tiles x K-tiles work into
 * one equal contiguous share per compute unit, so the chip stays full when the tile count
 * does not divide evenly over the compute units (for example the GPT-2 QKV layer, 1536^3
 * and 2560^3). The direct-copy ones (names ending "d") first run every whole round of
 * tiles but the last one tile per workgroup and split only the last round's tiles; the
 * register-staged ones split all of them.
 * A tile shared by several workgroups is finished by the one that arrives last, which
 * adds the partial sums in a fixed order: results stay bitwise reproducible from run
 * to run, and within the same error bound as every other configuration. On operands only
 * 4-byte aligned, a direct-copy stream-K configuration runs with the unaligned copy form
 * (sgemm_config_describe) and a register-staged one runs the data-parallel kernel of its
 * tile instead.
 *
 *  workspace        device memory of workspace_bytes, 16-byte aligned, owned by the
 *                   caller. Zero-fill it once before its first use: its first 64 KiB
 *                   hold per-tile counters, which every call leaves at zero again; the
 *                   rest holds partial tiles while a call runs. Calls that may run at
 *                   the same time (on different streams) need separate workspaces.
 *                   NULL with workspace_bytes == 0 is allowed.
 *  workspace_bytes  its size. With config == -1 the library considers the stream-K
 *                   configurations whose sgemm_workspace_size() fits, and otherwise
 *                   behaves as sgemm_general; a forced stream-K configuration whose
 *                   workspace does not fit returns SGEMM_ERROR_WORKSPACE.
 *
 * Arguments by position: 1 opA, 2 opB, 3 M, 4 N, 5 K, 6 alpha, 7 A, 8 lda, 9 B, 10 ldb,
 * 11 beta, 12 C, 13 ldc, 14 bias, 15 act, 16 workspace, 17 workspace_bytes, 18 stream
 * (config is not counted). -16 when workspace is misaligned, or NULL with a nonzero size.
 */
int sgemm_general_ws(int config, int opA, int opB, int M, int N, int K, float alpha,
                     const float *A, int lda,
                     const float *B, int ldb,
                     float beta, float *C, int ldc,
                     const float *bias, int act,
                     void *workspace, size_t workspace_bytes,
                     void *stream);

/* Bytes of the scratch array that sgemm_general_noalloc uses on each GPU: 64 KiB of tile
 * counters plus two 128 x 128 fp32 partial tiles for each of 256 compute units. */
#define SGEMM_NOALLOC_SCRATCH_BYTES (65536ull + 2ull * 256ull * 128ull * 128ull * 4ull)

/*
 * sgemm_general_ws for callers that cannot allocate device memory or pass a workspace:
 * code under HIP graph capture, tight serving loops, and harnesses that forbid hipMalloc.
 * It calls no hipMalloc, hipFree or allocating routine. The stream-K configurations use a
 * scratch array of SGEMM_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs
 * on, from the first call on that GPU until the process ends; everything else is as for
 * sgemm_general_ws with that array as the workspace.
 *  - Every call on a GPU shares that GPU's array. Calls that may overlap on one GPU (on
 *    different streams, or from several threads) race on it and must not be issued; calls
 *    queued in order on one stream are fine.
 *  - The first call on a GPU looks up the array's address and queues a small kernel on
 *    `stream` that zeroes its tile counters; every later call leaves them at zero again.
 *  - A forced stream-K configuration whose workspace (sgemm_workspace_size) exceeds the
 *    array returns SGEMM_ERROR_WORKSPACE; with config == -1 only stream-K configurations
 *    that fit are considered.
 *  - A failure to look up the array returns a positive hipError_t.
 *
 * Arguments by position, as sgemm_general: 1 opA, 2 opB, 3 M, 4 N, 5 K, 6 alpha, 7 A, 8 lda,
 * 9 B, 10 ldb, 11 beta, 12 C, 13 ldc, 14 bias, 15 act, 16 stream (config is not counted).
 */
int sgemm_general_noalloc(int config, int opA, int opB, int M, int N, int K, float alpha,
                          const float *A, int lda,
                          const float *B, int ldb,
                          float beta, float *C, int ldc,
                          const float *bias, int act,
                          void *stream);

/*
 * Workspace bytes that stream-K configuration `config` needs on the current device
 * (64 KiB of counters plus two partial tiles per compute unit: one sharing workgroup per
 * compute unit at most), or with config == -1
 * the most any of them needs. 0 for other configurations, or when the device cannot be
 * queried.
 */
size_t sgemm_workspace_size(int config);

/*
 * The configuration sgemm_general_ws would pick for a plain product with a workspace
 * of workspace_bytes (as sgemm_select_config otherwise; queries the current device's
 * compute-unit count when workspace_bytes > 0).
 */
int sgemm_select_config_ws(int M, int N, int K, float alpha,
                           const float *A, int lda,
                           const float *B, int ldb,
                           const float *C, int ldc,
                           size_t workspace_bytes);

/*
 * The configuration the library would pick for any call form (host logic only): opA/opB
 * as for sgemm_op, strides and batch as for sgemm_strided_batched_op (batch == 1 for the
 * single-matrix entry points, strides then ignored), and the workspace size as for
 * sgemm_general_ws (used only when batch == 1; it queries the current device's
 * compute-unit count when nonzero). Arguments are not validated. Returns -1 when no
 * matrix kernel would run (M, N, K or batch <= 0, or alpha == 0).
 */
int sgemm_select_config_general(int opA, int opB, int M, int N, int K, float alpha,
                                const float *A, int lda, long long strideA,
                                const float *B, int ldb, long long strideB,
                                const float *C, int ldc, long long strideC,
                                int batch, size_t workspace_bytes);

/* Number of kernel configurations compiled into the library. */
int sgemm_config_count(void);

/* Short name of configuration `config` (e.g. "mfma_256x256x16_w2x4"), or NULL if out of range. */
const char *sgemm_config_name(int config);

/*
 * One static line of space-separated key=value fields describing configuration
 * `config`, or NULL if it is out of range. The fields are the tile parameters that a
 * tiled kernel is built from ("Micro_gemm_4x4 - cuBLAS micro GEMM skeleton", section
 * "Tile parameters"), as this library sizes them:
 *   name          as sgemm_config_name
 *   kind          tile16 (one output per thread), mfma (one workgroup per tile),
 *                 streamk (whole-tile rounds, then equal shares of the remaining tiles x
 *                 K-tiles per compute unit), valu
 *                 (register micro-tile on vector FMAs)
 *   tile          BMxBNxBK: the workgroup's output tile and the k depth of one LDS stage
 *   waves         WGMxWGN: waves over the tile (1x1 for the non-matrix kinds)
 *   kgroups       wave groups splitting each stage's k range
 *   threads       threads per workgroup
 *   ahead         K-tiles whose loads run ahead of the one being multiplied
 *   loader        direct-16B (HBM -> LDS copies), staged-16B (through registers), or the
 *                 element-wise forms of tile16 and valu
 *   lds_bytes     static LDS per workgroup
 *   band          tile rows per band of the workgroup order
 *   unaligned     the form run when rows are only 4-byte aligned: direct-16B-unaligned
 *                 (the same 16-byte direct copies from 4-byte aligned addresses, with the
 *                 K-tile that holds the end of K copied in 4-byte words), staged-4B
 *                 (16-byte loads through registers, the chunk that crosses a row's end
 *                 read float by float), or for a register-staged streamk configuration
 *                 data-parallel-staged-4B (the data-parallel kernel of its tile)
 *   unaligned_bk  the K-tile of that form
 *   compute       the instruction that does the multiply-adds
 * The string is owned by the library and valid for the life of the process.
 */
const char *sgemm_config_describe(int config);

/*
 * The configuration sgemm would use for these arguments (host logic only; no GPU
 * call). Returns an id in [0, sgemm_config_count()), or -1 when no kernel would
 * run (M == 0 or N == 0) or the quick-return scaling kernel would (K == 0 or alpha == 0
 * counts as -1 too).
 */
int sgemm_select_config(int M, int N, int K, float alpha,
                        const float *A, int lda,
                        const float *B, int ldb,
                        const float *C, int ldc);

/*
 * Launch shape of configuration `config` for an M x N x K product (host logic only).
 * Writes grid[3] and block[3] (dim3 order x, y, z). Data-parallel matrix configurations
 * launch one workgroup per BM x BN tile; when N mod BN = r is 1..8, the whole tiles
 * number at least 256 (over the batch, in a batched call; the shape reported here is for
 * one product) and the fringe workgroups' memory round trips, ceil(K / (64 x (threads / 64) x U))
 * (U = 4 for r <= 2, 2 for r <= 4, 1 for r <= 8), times the rounds they run in (ceil(M / 2) of
 * them over 256 CUs, as many per CU as the configuration's LDS and 32 waves allow), are at most
 * 3, the tiles stop at column N - r and ceil(M / 2) more workgroups follow them,
 * each computing two rows of the last r columns (fringe columns; they also require row
 * strides under 2^20 floats, which this query, having no strides, assumes). Stream-K
 * configurations launch one
 * workgroup per tile of the whole rounds they run unsplit (direct-copy ones: 256 x
 * floor((tiles - 1) / 256)), then one per compute unit for the shared tiles, and at most
 * one per K-tile step of those; the shape reported for them assumes MI355X's 256 compute
 * units. Returns 0, SGEMM_ERROR_BAD_CONFIG,
 * SGEMM_ERROR_TOO_LARGE, or -1/-2/-3 for a negative M/N/K.
 */
int sgemm_launch_shape(int config, int M, int N, int K, int grid[3], int block[3]);

/* Static message for a status code returned by any entry point. */
const char *sgemm_status_string(int status);

/* Library version string. */
const char *sgemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TILED_FP32_GEMM_SGEMM_H */
