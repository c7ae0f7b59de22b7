// C-ABI entry points of libfp32gemm.so: argument checks, quick returns,
// routing (M <= 8 to the GEMV kernel), configuration choice and launch.
// The host-side launch mirrors the pages' launch step (grid over C tiles,
// asynchronous launch that returns at once; "CUDA 矩阵乘法优化", section
// "1. Kernel 1: 朴素实现"), with the grid shape taken from the chosen tile.
#include "../../include/fp32gemm.h"
#include "common.h"

using namespace fp32gemm;

namespace {

// Largest leading dimension accepted: keeps every in-tile byte offset the
// kernels form (at most 256 rows x ld x 4 bytes) inside 32 bits.
constexpr int kMaxLd = 1 << 20;

int imax(int a, int b) { return a > b ? a : b; }

int check_args(int M, int N, int K, float alpha, const float *A, int lda, const float *B,
               int ldb, float beta, float *C, int ldc) {
  (void)beta;
  if (M < 0) return -1;
  if (N < 0) return -2;
  if (K < 0) return -3;
  if (lda < imax(1, K) || lda > kMaxLd) return -6;
  if (ldb < imax(1, N) || ldb > kMaxLd) return -8;
  if (ldc < imax(1, N) || ldc > kMaxLd) return -11;
  const bool reads_ab = alpha != 0.0f && K > 0 && M > 0 && N > 0;
  if (reads_ab && A == nullptr) return -5;
  if (reads_ab && B == nullptr) return -7;
  if (M > 0 && N > 0 && C == nullptr) return -10;
  return 0;
}

// Quick returns shared by both families.  Returns 1 when the call is done
// (result code in *rc), 0 when the main kernel has to run.
int quick_return(const GemmArgs &a, hipStream_t s, int *rc) {
  if (a.M == 0 || a.N == 0) {
    *rc = 0;
    return 1;
  }
  if (a.alpha == 0.0f || a.K == 0) {
    *rc = (a.beta == 1.0f) ? 0 : (int)launch_scale(a, s);
    return 1;
  }
  return 0;
}

int run_gemm(int cfg, const GemmArgs &a, hipStream_t s) {
  int ntiles = 0;
  const GemmConfig *tiles = gemm_configs(&ntiles);
  if (cfg < 0) cfg = select_gemm_config(a.M, a.N, a.K);
  if (cfg >= ntiles * kNumGroups) return FP32GEMM_ERR_CONFIG;
  const GemmConfig &c = tiles[cfg / kNumGroups];
  return (int)c.launch(a, vec4_ok(a), kGroups[cfg % kNumGroups], s);
}

int run_gemv(int cfg, const GemmArgs &a, hipStream_t s) {
  int n = 0;
  const GemvConfig *cfgs = gemv_configs(&n);
  if (cfg < 0) cfg = select_gemv_config(a.M, a.N, a.K);
  if (cfg >= n) return FP32GEMM_ERR_CONFIG;
  return (int)cfgs[cfg].launch(a, s);
}

GemmArgs pack(int M, int N, int K, float alpha, const float *A, int lda, const float *B,
              int ldb, float beta, float *C, int ldc) {
  GemmArgs a;
  a.M = M; a.N = N; a.K = K;
  a.alpha = alpha; a.beta = beta;
  a.A = A; a.B = B; a.C = C;
  a.lda = lda; a.ldb = ldb; a.ldc = ldc;
  return a;
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

int sgemm(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
          float beta, float *C, int ldc, fp32gemm_stream_t stream) {
  int rc = check_args(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  if (rc) return rc;
  const GemmArgs a = pack(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (quick_return(a, s, &rc)) return rc;
  if (M <= 8) return run_gemv(-1, a, s);
  return run_gemm(-1, a, s);
}

int sgemv(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
          float beta, float *C, int ldc, fp32gemm_stream_t stream) {
  if (M < 1 || M > 8) return -1;
  int rc = check_args(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  if (rc) return rc;
  const GemmArgs a = pack(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (quick_return(a, s, &rc)) return rc;
  return run_gemv(-1, a, s);
}

const char *fp32gemm_strerror(int code) {
  switch (code) {
    case 0: return "success";
    case -1: return "invalid argument 1 (M)";
    case -2: return "invalid argument 2 (N)";
    case -3: return "invalid argument 3 (K)";
    case -4: return "invalid argument 4 (alpha)";
    case -5: return "invalid argument 5 (A is NULL but referenced)";
    case -6: return "invalid argument 6 (lda < max(1,K) or lda > 2^20)";
    case -7: return "invalid argument 7 (B is NULL but referenced)";
    case -8: return "invalid argument 8 (ldb < max(1,N) or ldb > 2^20)";
    case -9: return "invalid argument 9 (beta)";
    case -10: return "invalid argument 10 (C is NULL)";
    case -11: return "invalid argument 11 (ldc < max(1,N) or ldc > 2^20)";
    case -12: return "invalid argument 12 (stream)";
    case FP32GEMM_ERR_CONFIG: return "unknown configuration id";
    default: break;
  }
  if (code > 0) return hipGetErrorString(static_cast<hipError_t>(code));
  return "unknown error code";
}

int fp32gemm_num_configs(int kind) {
  if (kind == 0) return num_gemm_config_ids();
  if (kind == 1) {
    int n = 0;
    (void)gemv_configs(&n);
    return n;
  }
  return 0;
}

const char *fp32gemm_config_name(int kind, int cfg) {
  if (kind == 0) return gemm_config_name(cfg);
  if (kind == 1) {
    int n = 0;
    const GemvConfig *c = gemv_configs(&n);
    return (cfg >= 0 && cfg < n) ? c[cfg].name : nullptr;
  }
  return nullptr;
}

int fp32gemm_select_config(int kind, int M, int N, int K) {
  if (kind == 0) return select_gemm_config(M, N, K);
  if (kind == 1) return select_gemv_config(M, N, K);
  return FP32GEMM_ERR_CONFIG;
}

int fp32gemm_sgemm_with_config(int cfg, int M, int N, int K, float alpha, const float *A,
                               int lda, const float *B, int ldb, float beta, float *C, int ldc,
                               fp32gemm_stream_t stream) {
  if (cfg < -1 || cfg >= num_gemm_config_ids()) return FP32GEMM_ERR_CONFIG;
  int rc = check_args(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  if (rc) return rc;
  const GemmArgs a = pack(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (quick_return(a, s, &rc)) return rc;
  return run_gemm(cfg, a, s);
}

int fp32gemm_sgemv_with_config(int cfg, int M, int N, int K, float alpha, const float *A,
                               int lda, const float *B, int ldb, float beta, float *C, int ldc,
                               fp32gemm_stream_t stream) {
  if (cfg < -1 || cfg >= fp32gemm_num_configs(1)) return FP32GEMM_ERR_CONFIG;
  if (M < 1 || M > 8) return -1;
  int rc = check_args(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  if (rc) return rc;
  const GemmArgs a = pack(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (quick_return(a, s, &rc)) return rc;
  return run_gemv(cfg, a, s);
}

}  // extern "C"
#pragma GCC visibility pop
