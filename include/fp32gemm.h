/*
 * fp32gemm — single-precision GEMM and small-M GEMV for AMD MI355X (gfx950).
 *
 * C ABI of libfp32gemm.so.  Plain pointers and sizes only; no HIP or torch
 * header is needed to call it (the stream is an opaque pointer that is
 * ABI-identical to hipStream_t).
 *
 * The operation is the one defined on the page "GPU GEMM 优化完全拆解（一）：
 * 从朴素 Kernel 到共享内存分块", section "什么是 GEMM" (A is M x K, B is K x N,
 * C is M x N, alpha and beta scalars, C <- alpha * A B + beta * C), with the
 * row-major element update of the naive kernel in "CUDA 矩阵乘法优化：从朴素
 * Kernel 到接近 cuBLAS", section "1. Kernel 1: 朴素实现".  The small-M
 * product is the decode-phase matrix-vector shape of the first page's
 * section "LLM 推理本质上是 GEMM 的串联" (M = batch, usually 1 to 8).
 *
 * Conventions shared by every entry point:
 *  - Layout: row-major fp32.  Element (i, k) of A is A[i * lda + k], element
 *    (k, j) of B is B[k * ldb + j], element (i, j) of C is C[i * ldc + j].
 *  - Memory: A, B and C are device pointers (hipMalloc / torch CUDA tensors)
 *    owned by the caller.  The library keeps no reference after the call's
 *    kernels finish.  C must not overlap A or B.
 *  - Arithmetic: fp32 throughout (fp32 MFMA or fp32 FMA); no conversion to a
 *    narrower format.  The order of the k-sum is unspecified, so results may
 *    differ from a sequential loop by rounding.  Repeated calls with the same
 *    arguments and configuration give bit-identical results (no atomics on
 *    floats).
 *  - Reads: when beta == 0, C is not read (NaN in C does not propagate).
 *    When alpha == 0 or K == 0, A and B are not read (they may be NULL) and
 *    C <- beta * C.  When M == 0 or N == 0 the call does nothing.
 *  - Alignment: any 4-byte alignment is accepted.  The 128-bit load path is
 *    used when A and B are 16-byte aligned and K, N, lda and ldb are
 *    multiples of 4; otherwise a 32-bit load path computes the same result.
 *  - Asynchrony: work is enqueued on `stream` (NULL = the null stream) and
 *    the call returns without synchronising.
 *  - Return value: 0 on success; -p when argument p (1-based, in the order of
 *    the routine's own parameter list) is invalid; FP32GEMM_ERR_CONFIG for an
 *    unknown configuration id; a positive hipError_t value when a HIP call or
 *    kernel launch fails.  Nothing is enqueued when a negative code is
 *    returned.
 *  - Threads: every entry point is reentrant; calls on different streams
 *    may run concurrently.  The library allocates no device memory at run
 *    time; the split-K decode kernel (see sgemv) uses device memory reserved
 *    statically when the library is loaded, per stream.
 */
#ifndef FP32GEMM_H
#define FP32GEMM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *fp32gemm_stream_t;

#define FP32GEMM_OK 0
#define FP32GEMM_ERR_CONFIG (-100)
#define FP32GEMM_ERR_SCRATCH (-101)

/*
 * C[M x N] <- alpha * A[M x K] . B[K x N] + beta * C.
 * Argument checks: M, N, K >= 0; lda >= max(1, K); ldb >= max(1, N);
 * ldc >= max(1, N); A and B non-NULL when alpha != 0 and K > 0; C non-NULL
 * when M > 0 and N > 0.  M <= 8 is routed to the GEMV kernel (sgemv), and
 * M = 9..128 to the skinny MFMA kernel where it is the faster (M <= 48
 * and M = 65..80 always, M <= 96 up to N = 8192, otherwise while the tiled
 * kernel has fewer than 160 64x64 tiles);
 * larger M runs the LDS-tiled fp32 MFMA kernel with the tile configuration
 * that the per-shape table selects for (M, N, K).
 */
int sgemm(int M, int N, int K, float alpha, const float *A, int lda,
          const float *B, int ldb, float beta, float *C, int ldc,
          fp32gemm_stream_t stream);

/*
 * The same operation for 1 <= M <= 128 (the decode shape: X = A is M x K, the
 * weight W = B is K x N, Y = C is M x N; M is the number of sequences
 * decoded at once).  Bandwidth-bound: the time is one pass over W.  The
 * library picks the kernel by shape:
 *  - large W with few 256-column blocks (for example 4096 x 4096 at any
 *    M up to 8): K is split across workgroups, each reading 1 KB runs of W's
 *    rows over a chunk of K; the chunks' partial sums are added in chunk
 *    order by the last workgroup of each column block, in the same kernel.
 *    The partial sums and arrival counters live in device memory the
 *    library reserves statically (about 16 MB per device, in 8 slots); each
 *    stream gets its own slot on its first call, so calls on different
 *    streams never share one.  Calls on further streams run a form without
 *    scratch that adds the same partial sums in the same order
 *    (bit-identical results).  A call captured in a HIP graph keeps the
 *    capturing stream's slot: two replays of it must not run concurrently
 *    with each other or with calls on that stream.
 *  - otherwise each workgroup streams a narrow block of W's columns over
 *    all of K, its waves split K, and the partial sums are added inside the
 *    workgroup; up to M = 32 the multiply can run on the vector ALUs
 *    (128-bit loads of W), up to M = 128 on the matrix cores (16-column
 *    stripes, v_mfma_f32_16x16x4_f32).
 * Every path adds in a fixed order (integer atomics only, none on floats),
 * so repeated calls give bit-identical results.  Returns -1 when M is
 * outside 1..128.
 */
int sgemv(int M, int N, int K, float alpha, const float *A, int lda,
          const float *B, int ldb, float beta, float *C, int ldc,
          fp32gemm_stream_t stream);

/*
 * Transposed operands.  op(X) = X for FP32GEMM_OP_N and X^T for FP32GEMM_OP_T.
 * C[M x N] <- alpha * op(A)[M x K] . op(B)[K x N] + beta * C, row-major
 * storage: A is M x K (lda >= K) for N, or stored K x M (lda >= M) with
 * op(A)[i][k] = A[k * lda + i] for T; B is K x N (ldb >= N) for N, or stored
 * N x K (ldb >= K) with op(B)[k][j] = B[j * ldb + k] for T.  These are the
 * projection products of a transformer layer ("GPU GEMM 优化完全拆解（一）",
 * section "LLM 推理本质上是 GEMM 的串联": QKV, Q K^T, FFN), where weights and
 * keys are commonly stored transposed.  The 128-bit path needs 16-byte
 * aligned operands whose contiguous dimension and leading dimension are
 * multiples of 4.  M <= 8 runs a GEMV kernel: with op(B) = B the one sgemm
 * uses; with op(B) = B^T (a linear layer's weight stored N x K, y = x W^T) a
 * row-dot kernel that streams each stored row of B contiguously.  Either
 * takes op(A) = A^T as well, up to lda = 2^17 (beyond that the tiled kernel
 * runs).  Both reduce in a fixed order, so results are bit-reproducible.
 * Argument positions for error codes: transA 1,
 * transB 2, M 3, N 4, K 5, alpha 6, A 7, lda 8, B 9, ldb 10, beta 11, C 12,
 * ldc 13, stream 14.
 */
#define FP32GEMM_OP_N 0
#define FP32GEMM_OP_T 1
int sgemm_ex(int transA, int transB, int M, int N, int K, float alpha,
             const float *A, int lda, const float *B, int ldb, float beta,
             float *C, int ldc, fp32gemm_stream_t stream);

/*
 * batch_count independent products of the same shape: entry b uses
 * A + b * strideA, B + b * strideB and C + b * strideC (element strides).
 * strideA or strideB may be 0 (one operand shared by every entry); the C
 * entries must not overlap: strideC >= (M - 1) * ldc + N when
 * batch_count > 1.  Per-head attention products (Q K^T and P V for every
 * head) are this shape; with M <= 8 (decode: one query row per head) the
 * entries run on the GEMV kernels, with one grid over all entries.
 * 0 <= batch_count <= 65535; batch_count == 0 does nothing.  Argument positions: transA 1, transB 2, M 3, N 4, K 5, alpha 6,
 * A 7, lda 8, strideA 9, B 10, ldb 11, strideB 12, beta 13, C 14, ldc 15,
 * strideC 16, batch_count 17, stream 18.
 */
int sgemm_strided_batched(int transA, int transB, int M, int N, int K,
                          float alpha, const float *A, int lda,
                          long long strideA, const float *B, int ldb,
                          long long strideB, float beta, float *C, int ldc,
                          long long strideC, int batch_count,
                          fp32gemm_stream_t stream);

/*
 * Fused epilogue: C[i][j] <- act(alpha * (op(A) op(B))[i][j] + beta * C[i][j]
 * + bias[j]), operands as in sgemm_ex.  This is the operator fusion of "GPU
 * 基础原理" (a translation of "Basic facts about GPUs"), section "4.1 算子融合":
 * the elementwise chain (the page's example is y = relu(x + 1)) runs on the
 * product in registers, so C is stored once instead of being written, read
 * and written again by separate kernels.
 *
 * bias: device pointer to N floats, one per column of C (a linear layer's
 * output features), owned by the caller; NULL = no bias.  act:
 * FP32GEMM_ACT_NONE or FP32GEMM_ACT_RELU (v < 0 becomes 0; NaN and -0.0 pass
 * unchanged).  The bias is added first, then the activation is applied.
 * alpha = 0 or K = 0 still applies the epilogue to beta * C.  Routing as in
 * sgemm_ex (M <= 8 takes a GEMV kernel).  Argument positions for error
 * codes: as sgemm_ex for 1..13, bias 14, act 15 (unknown activation),
 * stream 16.
 */
#define FP32GEMM_ACT_NONE 0
#define FP32GEMM_ACT_RELU 1
int sgemm_fused(int transA, int transB, int M, int N, int K, float alpha,
                const float *A, int lda, const float *B, int ldb, float beta,
                float *C, int ldc, const float *bias, int act,
                fp32gemm_stream_t stream);

/*
 * Split-K: the same product as sgemm_ex, computed as `splits` partial
 * products over consecutive chunks of K that run as one grid, then added in
 * ascending chunk order (so results are bit-reproducible) with alpha and
 * beta applied once.  This is the K split of "CUDA 矩阵乘法优化：从朴素
 * Kernel 到接近 cuBLAS", section "10. cuBLAS 领先的性能差异", for shapes
 * whose C has too few tiles to fill the GPU but whose K is long.
 *
 * splits = 0 lets the library choose (fp32gemm_splitk_splits); otherwise
 * 1 <= splits <= 65535, rounded so that every chunk is a multiple of 32
 * values of K (the call may use fewer chunks than asked).  With one chunk,
 * or M <= 8, the call is exactly sgemm_ex and needs no workspace.
 *
 * workspace: device memory owned by the caller, at least
 * sgemm_splitk_workspace_size(M, N, K, splits) bytes, 16-byte aligned for
 * the fastest path; it holds the partial products (chunks x M x N floats,
 * packed) between the two kernels, must not overlap A, B or C, and must not
 * be used by another call until this one has completed on its stream.  The
 * library allocates nothing.
 *
 * Argument positions for error codes: transA 1, transB 2, M 3, N 4, K 5,
 * alpha 6, A 7, lda 8, B 9, ldb 10, beta 11, C 12, ldc 13, splits 14,
 * workspace 15 (NULL when needed), workspace_bytes 16 (too small),
 * stream 17.
 */
int sgemm_splitk(int transA, int transB, int M, int N, int K, float alpha,
                 const float *A, int lda, const float *B, int ldb, float beta,
                 float *C, int ldc, int splits, float *workspace,
                 size_t workspace_bytes, fp32gemm_stream_t stream);

/*
 * sgemm_splitk for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, kernels and summation order as sgemm_splitk with the
 * same splits (bit-identical results), but the partial products go to a
 * scratch array the library holds in device memory, 16 MiB on each GPU it
 * runs on, kept until the process ends.  No hipMalloc, hipFree or other
 * allocating call is made.
 *
 * Limit: chunks x M x N floats (the chunk count as sgemm_splitk would use
 * it, see sgemm_splitk_workspace_size / 4) must be at most 4 Mi; larger
 * calls return FP32GEMM_ERR_SCRATCH and enqueue nothing.  Calls that need
 * no scratch (one chunk, M <= 8, quick returns) run as sgemm_ex does.
 *
 * All calls on one GPU share its scratch array, which keeps the last call's
 * contents: calls that overlap in time on one GPU (on different streams,
 * or graph replays running concurrently) race and give undefined results.
 * Calls in sequence on one stream are safe.
 *
 * Argument positions for error codes: transA 1, transB 2, M 3, N 4, K 5,
 * alpha 6, A 7, lda 8, B 9, ldb 10, beta 11, C 12, ldc 13, splits 14,
 * stream 15.
 */
int sgemm_splitk_noalloc(int transA, int transB, int M, int N, int K,
                         float alpha, const float *A, int lda, const float *B,
                         int ldb, float beta, float *C, int ldc, int splits,
                         fp32gemm_stream_t stream);

/*
 * Stream-K: the same product as sgemm_ex, as one persistent grid whose
 * workgroups each take an equal run of the product's (C tile, K slice)
 * units, crossing tile boundaries; a tile shared by several workgroups is
 * finished in the same kernel by the last of them to arrive, which adds the
 * others' partial tiles in K order and applies alpha, beta.  This is the
 * pages' remedy for grids that leave compute units idle ("CUDA 矩阵乘法优化：
 * 从朴素 Kernel 到接近 cuBLAS", section "10. cuBLAS 领先的性能差异": split
 * K where the tiles of C alone do not fill the GPU), without split-K's
 * second kernel and with every workgroup doing the same amount of work.
 * Results are bit-reproducible (the order of the additions depends only on
 * the shape).
 *
 * workspace: device memory owned by the caller, at least
 * sgemm_streamk_workspace_size(M, N, K) bytes; it holds partial tiles (two
 * per workgroup at most) and must not overlap A, B or C or be used by
 * another call until this one has completed on its stream.  Arrival
 * counters live in device memory the library reserves statically per
 * stream (8 streams per device, up to 4096 C tiles per call; past either
 * limit they go to the end of the workspace, cleared by a small kernel
 * before the main one).  M <= 8 runs the GEMV kernels as sgemm_ex does and
 * needs no workspace.
 *
 * Argument positions for error codes: transA 1, transB 2, M 3, N 4, K 5,
 * alpha 6, A 7, lda 8, B 9, ldb 10, beta 11, C 12, ldc 13, workspace 14
 * (NULL), workspace_bytes 15 (too small), stream 16.
 */
int sgemm_streamk(int transA, int transB, int M, int N, int K, float alpha,
                  const float *A, int lda, const float *B, int ldb, float beta,
                  float *C, int ldc, float *workspace, size_t workspace_bytes,
                  fp32gemm_stream_t stream);

/* Workspace bytes sgemm_streamk needs for this shape (0 when M <= 8). */
size_t sgemm_streamk_workspace_size(int M, int N, int K);

/* Workspace bytes sgemm_splitk needs for this shape and splits (0 = the
 * library's choice); 0 when the call runs as a single chunk. */
size_t sgemm_splitk_workspace_size(int M, int N, int K, int splits);

/* The number of K chunks sgemm_splitk uses with splits = 0: a model of the
 * tiled kernel's rate for the enlarged grid plus the reduction's traffic. */
int fp32gemm_splitk_splits(int M, int N, int K);

/* Human-readable text for a return code (static storage, never NULL). */
const char *fp32gemm_strerror(int code);

/*
 * Tuning and testing hooks.  These expose the per-shape parameter search of
 * "CUDA 矩阵乘法优化：从朴素 Kernel 到接近 cuBLAS", section "8. Kernel 9:
 * 参数自动调优": the tile parameters (block tile, K depth, wave tile) are
 * enumerated, each candidate is timed on the target GPU, and the fastest per
 * shape goes into a table, because the best choice differs between GPUs.
 * The tuner (fp32_gemm_06_amd/tune.py) drives the sweep through these calls.
 * kind 0 = the SGEMM kernel family, kind 1 = the GEMV family.
 * Configurations are numbered 0 .. fp32gemm_num_configs(kind)-1 and named by
 * fp32gemm_config_name (NULL for an unknown id); an unknown kind gives 0
 * configurations, NULL names and FP32GEMM_ERR_CONFIG selections.
 */
int fp32gemm_num_configs(int kind);
const char *fp32gemm_config_name(int kind, int cfg);

/* The configuration sgemm()/sgemv() would pick for this shape (kind as above). */
int fp32gemm_select_config(int kind, int M, int N, int K);

/* The largest M a configuration runs (kind as above; -1 for an unknown id):
 * 8, 32, 64 or 128 for the GEMV family, INT_MAX for the tiled family. */
int fp32gemm_config_max_rows(int kind, int cfg);

/* Whether the tiled kernel runs this product (batch entries of M x N x K) as
 * two launches: 0 = one launch; 1 = columns [0, *first) of C in whole rounds
 * of 256x256 tiles, then the remaining columns; 2 = the same over rows.
 * *first (may be NULL) receives the split point, 0 for one launch. */
int fp32gemm_round_split(int M, int N, int K, int batch, int *first);

/*
 * sgemm / sgemv with a forced configuration (cfg = -1 picks as the plain
 * entry point does).  Same contract and codes as sgemm; the M <= 8 routing
 * is not applied: fp32gemm_sgemm_with_config always runs the MFMA kernel and
 * fp32gemm_sgemv_with_config always the GEMV family (M must be 1..128, and at
 * most fp32gemm_config_max_rows of the configuration, else
 * FP32GEMM_ERR_CONFIG).
 */
int fp32gemm_sgemm_with_config(int cfg, int M, int N, int K, float alpha,
                               const float *A, int lda, const float *B,
                               int ldb, float beta, float *C, int ldc,
                               fp32gemm_stream_t stream);
int fp32gemm_sgemv_with_config(int cfg, int M, int N, int K, float alpha,
                               const float *A, int lda, const float *B,
                               int ldb, float beta, float *C, int ldc,
                               fp32gemm_stream_t stream);

/*
 * Stream-K tuning and testing hooks.  Tiles are numbered 0 ..
 * (number of names) - 1 and named by fp32gemm_streamk_tile_name (NULL past
 * the end).  fp32gemm_streamk_plan reports the plan for a shape with a
 * forced tile and / or workgroup count (-1 / 0 = the library's choice): the
 * tile, workgroups and K slices per workgroup, and returns the workspace
 * bytes it needs (0 for invalid arguments).  fp32gemm_streamk_with_config
 * runs sgemm_streamk with that plan, for any M >= 1; error positions as
 * sgemm_streamk shifted by two (tile 1, groups 2; FP32GEMM_ERR_CONFIG for an
 * unknown tile).
 */
const char *fp32gemm_streamk_tile_name(int tile);
size_t fp32gemm_streamk_plan(int M, int N, int K, int tile, int groups,
                             int *tile_out, int *groups_out, int *ipw_out);
int fp32gemm_streamk_with_config(int tile, int groups, int transA, int transB,
                                 int M, int N, int K, float alpha,
                                 const float *A, int lda, const float *B,
                                 int ldb, float beta, float *C, int ldc,
                                 float *workspace, size_t workspace_bytes,
                                 fp32gemm_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FP32GEMM_H */
