/*
 * CPU oracle for single-precision GEMM: C_ref = alpha * A.B + beta * C0.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or helper with the HIP
 * library and includes no GPU header.
 *
 * What it follows (the pages, by title and section):
 *  - "GPU GEMM 优化完全拆解（一）：从朴素 Kernel 到共享内存分块",
 *    section "什么是 GEMM": A is M x K, B is K x N, C is M x N, alpha and
 *    beta are scalars; element (i, j) of the product is the inner product of
 *    row i of A with column j of B (the display formula itself was lost in
 *    extraction; the prose around it and the store of the naive kernel in
 *    "CUDA 线程层次" fix the update C = alpha * (A B) + beta * C).
 *  - "CUDA 矩阵乘法优化：从朴素 Kernel 到接近 cuBLAS", section
 *    "1. Kernel 1: 朴素实现": one output element is the dot product over
 *    k = 0..K-1 followed by the alpha/beta update, row-major storage.
 *  - "GPU 基础原理", section "4.2 分块": a tiled sum is the same sum over k
 *    regrouped, so the plain (untiled) definition is the reference.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - leading dimensions: row-major with a row stride >= the row length
 *    (the pages only show packed storage);
 *  - beta == 0 does not read C0 and alpha == 0 (or K == 0) does not read A
 *    or B: the usual BLAS convention; the pages always evaluate
 *    alpha * tmp + beta * C;
 *  - arithmetic: every fp32 operand is widened to double, each product is
 *    exact in double (24 + 24 significant bits <= 53), the sum runs over k in
 *    ascending order in double, and alpha * acc + beta * c0 is evaluated in
 *    double.  The result is returned in double, unrounded.
 *
 * The bound array Bnd = |alpha| * (|A| |B|) + |beta| * |C0| is what the
 * acceptance test scales its tolerance by.
 *
 * oracle_epilogue adds the fused bias + activation of the pages' operator
 * fusion example (see its comment) to those results.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no -ffast-math: the order of the
 * double sum must stay as written).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Optional planted mistakes, used only by the CPU tests that check the
 * pins catch them.  0 = the faithful oracle. */
#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

/* Element (i, j) of A.B as a double sum over k = 0..K-1, ascending. */
static double dot_ij(int64_t i, int64_t j, int64_t K, const float *A,
                     int64_t lda, const float *B, int64_t ldb) {
  double acc = 0.0;
  int64_t kend = K;
#if ORACLE_MUTANT == 1 /* drops the last term of the sum */
  kend = K > 0 ? K - 1 : 0;
#endif
  for (int64_t k = 0; k < kend; ++k) {
#if ORACLE_MUTANT == 2 /* reads B transposed */
    acc += (double)A[i * lda + k] * (double)B[j * ldb + k];
#else
    acc += (double)A[i * lda + k] * (double)B[k * ldb + j];
#endif
  }
  return acc;
}

/* The update of one element from its dot product. */
static double update(double alpha, double acc, double beta, const float *C0,
                     int64_t i, int64_t j, int64_t ldc, int64_t K) {
  double r;
  if (alpha == 0.0 || K == 0)
    r = 0.0;
  else
    r = alpha * acc;
#if ORACLE_MUTANT == 3 /* wrong sign on the beta term */
  if (beta != 0.0) r -= beta * (double)C0[i * ldc + j];
#else
  if (beta != 0.0) r += beta * (double)C0[i * ldc + j];
#endif
  return r;
}

/*
 * Full product.  out[i * ldo + j] (double) receives the reference value for
 * i < M, j < N.  A, B may be NULL when alpha == 0 or K == 0; C0 may be NULL
 * when beta == 0.  Rows are distributed over OpenMP threads; each element's
 * sum is still the plain ascending-k sum.
 */
void oracle_sgemm(int M, int N, int K, float alpha, const float *A, int64_t lda,
                  const float *B, int64_t ldb, float beta, const float *C0,
                  int64_t ldc, double *out, int64_t ldo) {
  const double a = (double)alpha, b = (double)beta;
  const int use_ab = (alpha != 0.0f && K > 0);
#if ORACLE_MUTANT == 4 /* assumes C0 is packed (ignores its leading dimension) */
  ldc = N;
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < M; ++i) {
    double *row = out + i * ldo;
    /* i-k-j order: the row accumulator receives the terms of every sum in
     * ascending k, which is the same sum as dot_ij() evaluates. */
    for (int64_t j = 0; j < N; ++j) row[j] = 0.0;
    if (use_ab) {
      int64_t kend = K;
#if ORACLE_MUTANT == 1
      kend = K - 1;
#endif
      for (int64_t k = 0; k < kend; ++k) {
        const double aik = (double)A[i * lda + k];
#if ORACLE_MUTANT == 2
        for (int64_t j = 0; j < N; ++j) row[j] += aik * (double)B[j * ldb + k];
#else
        const float *brow = B + k * ldb;
        for (int64_t j = 0; j < N; ++j) row[j] += aik * (double)brow[j];
#endif
      }
    }
    for (int64_t j = 0; j < N; ++j) row[j] = update(a, row[j], b, C0, i, j, ldc, K);
  }
}

/*
 * Selected elements only: out[t] = reference value of element
 * (rows[t], cols[t]).  Used where the full product is too slow for a test.
 */
void oracle_sgemm_entries(int count, const int *rows, const int *cols, int K,
                          float alpha, const float *A, int64_t lda,
                          const float *B, int64_t ldb, float beta,
                          const float *C0, int64_t ldc, double *out) {
  const double a = (double)alpha, b = (double)beta;
  const int use_ab = (alpha != 0.0f && K > 0);
#pragma omp parallel for schedule(static)
  for (int t = 0; t < count; ++t) {
    const int64_t i = rows[t], j = cols[t];
    const double acc = use_ab ? dot_ij(i, j, K, A, lda, B, ldb) : 0.0;
    out[t] = update(a, acc, b, C0, i, j, ldc, K);
  }
}

/*
 * Tolerance scale: bnd[i * ldo + j] = |alpha| * sum_k |A[i,k]| |B[k,j]|
 *                                     + |beta| * |C0[i,j]|.
 * Terms that the update does not read (alpha == 0, beta == 0) contribute 0.
 */
void oracle_bound(int M, int N, int K, float alpha, const float *A, int64_t lda,
                  const float *B, int64_t ldb, float beta, const float *C0,
                  int64_t ldc, double *bnd, int64_t ldo) {
  const double aa = fabs((double)alpha), bb = fabs((double)beta);
  const int use_ab = (alpha != 0.0f && K > 0);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < M; ++i) {
    double *row = bnd + i * ldo;
    for (int64_t j = 0; j < N; ++j) row[j] = 0.0;
    if (use_ab) {
      for (int64_t k = 0; k < K; ++k) {
        const double aik = fabs((double)A[i * lda + k]);
        const float *brow = B + k * ldb;
        for (int64_t j = 0; j < N; ++j) row[j] += aik * fabs((double)brow[j]);
      }
      for (int64_t j = 0; j < N; ++j) row[j] *= aa;
    }
    if (beta != 0.0f)
      for (int64_t j = 0; j < N; ++j) row[j] += bb * fabs((double)C0[i * ldc + j]);
  }
}

/* The bound for selected elements (same definition as oracle_bound). */
void oracle_bound_entries(int count, const int *rows, const int *cols, int K,
                          float alpha, const float *A, int64_t lda,
                          const float *B, int64_t ldb, float beta,
                          const float *C0, int64_t ldc, double *out) {
  const double aa = fabs((double)alpha), bb = fabs((double)beta);
  const int use_ab = (alpha != 0.0f && K > 0);
#pragma omp parallel for schedule(static)
  for (int t = 0; t < count; ++t) {
    const int64_t i = rows[t], j = cols[t];
    double s = 0.0;
    if (use_ab) {
      for (int64_t k = 0; k < K; ++k)
        s += fabs((double)A[i * lda + k]) * fabs((double)B[k * ldb + j]);
      s *= aa;
    }
    if (beta != 0.0f) s += bb * fabs((double)C0[i * ldc + j]);
    out[t] = s;
  }
}

/*
 * Fused epilogue, applied to values the functions above produced.  The pages
 * fuse an elementwise chain into the kernel that produces its input ("GPU
 * 基础原理", section "4.1 算子融合": y = relu(x + 1) in one pass, the
 * intermediate never stored); on a GEMM output the chain is a linear layer's
 * epilogue:
 *
 *   vals[t] <- act(vals[t] + bias[cols[t]])
 *
 * with one bias value per column of C (NULL = no bias) and act 0 = identity,
 * 1 = ReLU: v < 0 gives 0, anything else (including NaN and -0.0) passes
 * unchanged.  The bias is added in double, then the activation is applied.
 * bnd[t] (may be NULL) receives + |bias[cols[t]]|, the matching tolerance
 * scale; ReLU moves two values no further apart, so it adds nothing.
 * rows[] is unused by the faithful oracle (the bias does not depend on the
 * row).
 */
void oracle_epilogue(int count, const int *rows, const int *cols, const float *bias, int act,
                     double *vals, double *bnd) {
  (void)rows;
  for (int t = 0; t < count; ++t) {
#if ORACLE_MUTANT == 5 /* bias indexed by the row */
    const double b = bias ? (double)bias[rows[t]] : 0.0;
#else
    const double b = bias ? (double)bias[cols[t]] : 0.0;
#endif
    double v = vals[t];
#if ORACLE_MUTANT == 6 /* activation before the bias */
    if (act == 1 && v < 0.0) v = 0.0;
    v += b;
#else
    v += b;
    if (act == 1 && v < 0.0) v = 0.0;
#endif
    vals[t] = v;
    if (bnd) bnd[t] += fabs(b);
  }
}

/* Number of OpenMP threads the parallel loops above will use. */
int oracle_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sets the number of OpenMP threads the loops above use (n >= 1) and
 * returns the number in effect afterwards; for timing the oracle on fewer
 * cores than the host has. */
int oracle_set_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  if (n >= 1) omp_set_num_threads(n);
#endif
  return oracle_threads();
}
