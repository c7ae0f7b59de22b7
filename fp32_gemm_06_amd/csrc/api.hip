// C-ABI entry points of libfp32gemm.so: argument checks, quick returns,
// routing (M <= 8 to the GEMV kernel), configuration choice and launch.
// The host-side launch mirrors the pages' launch step (grid over C tiles,
// asynchronous launch that returns at once; "CUDA 矩阵乘法优化", section
// "1. Kernel 1: 朴素实现"), with the grid shape taken from the chosen tile.
#include <mutex>

#include "../../include/fp32gemm.h"
#include "common.h"

using namespace fp32gemm;

namespace {

// Largest leading dimension accepted: keeps every in-tile byte offset the
// kernels form (at most 256 rows x ld x 4 bytes) inside 32 bits.
constexpr int kMaxLd = 1 << 20;
// Most K chunks of a split-K call (one grid dimension).
constexpr int kMaxSplits = 65535;

int imax(int a, int b) { return a > b ? a : b; }

// 1-based positions of the arguments in a routine's parameter list (0 when
// the routine has no such argument), for BLAS-style -p error codes.
struct Pos {
  int ta, tb, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, batch;
};
constexpr Pos kPosSgemm = {0, 0, 1, 2, 3, 5, 6, 0, 7, 8, 0, 10, 11, 0, 0};
constexpr Pos kPosSgemmEx = {1, 2, 3, 4, 5, 7, 8, 0, 9, 10, 0, 12, 13, 0, 0};
constexpr Pos kPosBatched = {1, 2, 3, 4, 5, 7, 8, 9, 10, 11, 12, 14, 15, 16, 17};

int check_args(const Pos &p, int ta, int tb, const GemmArgs &a) {
  if (ta != 0 && ta != 1) return -p.ta;
  if (tb != 0 && tb != 1) return -p.tb;
  if (a.M < 0) return -p.M;
  if (a.N < 0) return -p.N;
  if (a.K < 0) return -p.K;
  if (a.lda < imax(1, ta ? a.M : a.K) || a.lda > kMaxLd) return -p.lda;
  if (p.sA && a.sA < 0) return -p.sA;
  if (a.ldb < imax(1, tb ? a.K : a.N) || a.ldb > kMaxLd) return -p.ldb;
  if (p.sB && a.sB < 0) return -p.sB;
  if (a.ldc < imax(1, a.N) || a.ldc > kMaxLd) return -p.ldc;
  if (p.batch && a.batch < 0) return -p.batch;
  // batch entries of C must not overlap
  if (p.sC && a.batch > 1 && a.M > 0 && a.N > 0 && a.sC < (long long)(a.M - 1) * a.ldc + a.N)
    return -p.sC;
  const bool work = a.M > 0 && a.N > 0 && a.batch > 0;
  const bool reads_ab = work && a.alpha != 0.0f && a.K > 0;
  if (reads_ab && a.A == nullptr) return -p.A;
  if (reads_ab && a.B == nullptr) return -p.B;
  if (work && a.C == nullptr) return -p.C;
  return 0;
}

// Quick returns shared by every routine.  Returns 1 when the call is done
// (result code in *rc), 0 when the main kernel has to run.
int quick_return(const GemmArgs &a, hipStream_t s, int *rc) {
  if (a.M == 0 || a.N == 0 || a.batch == 0) {
    *rc = 0;
    return 1;
  }
  if (a.alpha == 0.0f || a.K == 0) {
    const bool noop = a.beta == 1.0f && a.bias == nullptr && a.act == kActNone;
    *rc = noop ? 0 : (int)launch_scale(a, s);
    return 1;
  }
  return 0;
}

int run_gemm(int cfg, int ta, int tb, const GemmArgs &a, hipStream_t s) {
  int ntiles = 0;
  const GemmConfig *tiles = gemm_configs(&ntiles);
  if (cfg < 0) cfg = select_gemm_config(a.M, a.N, a.K, a.batch);
  if (cfg >= ntiles * kNumGroups) return FP32GEMM_ERR_CONFIG;
  const GemmConfig &c = tiles[cfg / kNumGroups];
  return (int)c.launch[2 * ta + tb](a, vec4_ok(a, ta, tb), kGroups[cfg % kNumGroups], s);
}

int run_gemv(int cfg, int ta, const GemmArgs &a, hipStream_t s) {
  int n = 0;
  const GemvConfig *cfgs = gemv_configs(&n);
  if (cfg < 0) cfg = select_gemv_config(a.M, a.N, a.K);
  if (cfg >= n) return FP32GEMM_ERR_CONFIG;
  return (int)cfgs[cfg].launch(a, ta, s);
}

// The tiled kernel with the configuration the dispatcher picks, as one launch
// or as two over column or row ranges of C (plan_round_split).  The second
// product starts at an offset of 256 k1 elements along N or M: B (op(B) = B
// as given: columns; B^T: storage rows), A (op(A) = A: rows; A^T: storage
// columns), C and the bias move with it, and the strides between batch
// entries stay.
int run_tiled(int ta, int tb, const GemmArgs &a, hipStream_t s) {
  const RoundSplit sp = plan_round_split(a.M, a.N, a.K, a.batch);
  if (sp.dim == 0) return run_gemm(-1, ta, tb, a, s);
  const size_t f = (size_t)sp.first;
  GemmArgs p = a, q = a;
  if (sp.dim == 1) {
    p.N = sp.first;
    q.N = a.N - sp.first;
    q.B = tb ? a.B + f * (size_t)a.ldb : a.B + f;
    q.C = a.C + f;
    if (a.bias) q.bias = a.bias + f;
  } else {
    p.M = sp.first;
    q.M = a.M - sp.first;
    q.A = ta ? a.A + f : a.A + f * (size_t)a.lda;
    q.C = a.C + f * (size_t)a.ldc;
  }
  const int rc = run_gemm(sp.main_cfg, ta, tb, p, s);
  if (rc) return rc;
  return run_gemm(-1, ta, tb, q, s);
}

// M = 9..128: the skinny MFMA kernel (N / 16 workgroups or fewer, each over
// all of K), or the tiled kernel, whose 64x64 tiles number only
// ceil(M / 64) * ceil(N / 64) and each walk all of K.  Measured over N =
// 4096..16384, K = 4096 (cold weights, both layouts of W, one GPU), the
// skinny kernel is faster
//  * for every M <= 48 (4096^2, M = 16: 21.4 against 99.7 us; N = 16384,
//    M = 33: 68.7 against 83.7);
//  * for M = 65..80, where the tiled kernel computes up to twice the rows
//    (N = 11008, M = 80: 121 against 132; N = 16384: 123 against 134);
//  * for M <= 96 while its 32-column stripes fit one round of workgroups
//    (N = 8192, M = 96: 71.1 against 74.5);
//  * while the tiled kernel has fewer than 160 tiles (4096^2, M = 128: 59.4
//    against 75.3).
// Otherwise the tiled kernel is (N = 11008, M = 64: 79.0 against 86.1 with
// W stored N x K; M = 96: 132 against 138; N = 8192, M = 128: 79.0 against
// 90.4).
// Short K comes first: the skinny kernel's fixed cost (staging X and adding
// the waves' M x 16 NB partial sums in LDS) grows with the row blocks, and
// below K = 5 M the tiled kernel's walk over K is the shorter.  Measured over
// N = 128, 1024 and 4096, both layouts of W, M = 33..128 and K = 128..1024
// (one GPU, back-to-back calls), the two are level at K = 200-250 for
// M = 33..48, 320 for M = 64, 640 for M = 128; at K = 128 the tiled kernel
// takes 5.2-5.7 us against 6.8 (M = 33) to 11.0 (M = 128).  Up to 32 rows
// (two row blocks) the skinny kernel is the faster at every K (M = 32,
// K = 128: 4.5 against 5.1 us).
bool skinny_pays(const GemmArgs &a) {
  if (a.M > 32 && a.K < 5 * a.M) return false;
  if (a.M <= 48 || (a.M > 64 && a.M <= 80)) return true;
  if (a.M <= 96 && (long long)a.N * a.batch <= 256 * 32) return true;
  const long long tiles = (long long)((a.M + 63) / 64) * ((a.N + 63) / 64) * a.batch;
  return tiles < 160;
}

// The product on the kernel that suits it: M <= 8 on a GEMV kernel (row dots
// when op(B) = B^T, column stripes otherwise; a.batch entries in one grid),
// M = 9..128 on the skinny MFMA kernel where it pays, and everything else
// (and op(A) = A^T with a very large lda) on the tiled kernel.
int run_product(int ta, int tb, const GemmArgs &a, hipStream_t s) {
  if (gemv_supported(a, ta)) {
    if (tb) return (int)launch_gemv_rows(a, ta, -1, s);
    return run_gemv(select_gemv_config_batched(a.M, a.N, a.K, a.batch), ta, a, s);
  }
  if (skinny_supported(a, ta) && skinny_pays(a)) {
    if (tb) return (int)launch_skinny_tb(a, ta, s);
    return run_gemv(select_gemv_config_batched(a.M, a.N, a.K, a.batch), ta, a, s);
  }
  return run_tiled(ta, tb, a, s);
}

// Split-K as two kernels over a workspace of chunks x M x N floats (packed
// planes): chunk c of K as batch entry c, raw sums into plane c, then
// C <- alpha * (the planes added in order) + beta * C.
int run_splitk(int transA, int transB, const GemmArgs &a, int chunks, int kc, float *workspace,
               hipStream_t s) {
  const int M = a.M, N = a.N;
  GemmArgs p = a;
  p.K = kc;
  p.k_total = a.K;
  p.alpha = 1.0f;
  p.beta = 0.0f;
  p.C = workspace;
  p.ldc = N;
  p.sA = transA ? (long long)kc * a.lda : (long long)kc;
  p.sB = transB ? (long long)kc : (long long)kc * a.ldb;
  p.sC = (long long)M * N;
  p.batch = chunks;
  const int rc = run_gemm(model_gemm_config(M, N, kc, chunks, nullptr), transA, transB, p, s);
  if (rc) return rc;
  return (int)launch_splitk_reduce(workspace, chunks, M, N, a.alpha, a.beta, a.C, a.ldc, s);
}

// ---- scratch of sgemm_splitk_noalloc ---------------------------------------
// For callers that cannot allocate (code under HIP graph capture, serving
// loops, harnesses that forbid hipMalloc): the split-K partial products go
// to this file-scope array instead of a caller workspace.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code
// the array's name only stands for the device symbol; its device address
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is passed to kernels.
constexpr size_t kScratchFloats = (size_t)4 << 20;  // 16 MiB
__device__ __attribute__((aligned(256))) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_ptr(float **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float *>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

GemmArgs pack(int M, int N, int K, float alpha, const float *A, int lda, const float *B,
              int ldb, float beta, float *C, int ldc) {
  GemmArgs a;
  a.M = M; a.N = N; a.K = K;
  a.alpha = alpha; a.beta = beta;
  a.A = A; a.B = B; a.C = C;
  a.lda = lda; a.ldb = ldb; a.ldc = ldc;
  a.sA = a.sB = a.sC = 0;
  a.batch = 1;
  a.k_total = 0;
  a.bias = nullptr;
  a.act = kActNone;
  return a;
}

// Stream-K call shared by sgemm_streamk and its forced-plan hook; `base` is
// the 1-based position of transA in the caller's parameter list.
int streamk_call(int tile, int groups, int base, int transA, int transB, int M, int N, int K,
                 float alpha, const float *A, int lda, const float *B, int ldb, float beta,
                 float *C, int ldc, float *workspace, size_t workspace_bytes, hipStream_t s,
                 bool forced) {
  GemmArgs a = pack(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  const int off = base - 1;
  const Pos p = {1 + off, 2 + off, 3 + off, 4 + off, 5 + off, 7 + off, 8 + off, 0,
                 9 + off, 10 + off, 0, 12 + off, 13 + off, 0, 0};
  int rc = check_args(p, transA, transB, a);
  if (rc) return rc;
  if (quick_return(a, s, &rc)) return rc;
  if (!forced && M <= 8) return run_product(transA, transB, a, s);  // the GEMV kernels
  const SkPlan plan = streamk_plan(M, N, K, tile, groups);
  if (plan.tile < 0) return FP32GEMM_ERR_CONFIG;
  if (workspace == nullptr) return -(14 + off);
  if (workspace_bytes < streamk_workspace_bytes(plan)) return -(15 + off);
  return (int)launch_streamk(transA, transB, a, plan, workspace, s);
}
}  // namespace

#pragma GCC visibility push(default)
extern "C" {

int sgemm(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
          float beta, float *C, int ldc, fp32gemm_stream_t stream) {
  const GemmArgs a = pack(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  int rc = check_args(kPosSgemm, 0, 0, a);
  if (rc) return rc;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (quick_return(a, s, &rc)) return rc;
  return run_product(0, 0, a, s);
}

int sgemv(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
          float beta, float *C, int ldc, fp32gemm_stream_t stream) {
  if (M < 1 || M > kSkinnyMaxRows) return -1;
  const GemmArgs a = pack(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  int rc = check_args(kPosSgemm, 0, 0, a);
  if (rc) return rc;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (quick_return(a, s, &rc)) return rc;
  return run_gemv(-1, 0, a, s);
}

int sgemm_ex(int transA, int transB, int M, int N, int K, float alpha, const float *A, int lda,
             const float *B, int ldb, float beta, float *C, int ldc, fp32gemm_stream_t stream) {
  const GemmArgs a = pack(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  int rc = check_args(kPosSgemmEx, transA, transB, a);
  if (rc) return rc;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (quick_return(a, s, &rc)) return rc;
  return run_product(transA, transB, a, s);
}

int sgemm_strided_batched(int transA, int transB, int M, int N, int K, float alpha,
                          const float *A, int lda, long long strideA, const float *B, int ldb,
                          long long strideB, float beta, float *C, int ldc, long long strideC,
                          int batch_count, fp32gemm_stream_t stream) {
  GemmArgs a = pack(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  a.sA = strideA;
  a.sB = strideB;
  a.sC = strideC;
  a.batch = batch_count;
  int rc = check_args(kPosBatched, transA, transB, a);
  if (rc) return rc;
  if (batch_count > 65535) return -kPosBatched.batch;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (quick_return(a, s, &rc)) return rc;
  return run_product(transA, transB, a, s);
}

int sgemm_fused(int transA, int transB, int M, int N, int K, float alpha, const float *A, int lda,
                const float *B, int ldb, float beta, float *C, int ldc, const float *bias, int act,
                fp32gemm_stream_t stream) {
  GemmArgs a = pack(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  int rc = check_args(kPosSgemmEx, transA, transB, a);
  if (rc) return rc;
  if (act != FP32GEMM_ACT_NONE && act != FP32GEMM_ACT_RELU) return -15;
  a.bias = bias;
  a.act = act == FP32GEMM_ACT_RELU ? kActRelu : kActNone;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (quick_return(a, s, &rc)) return rc;
  return run_product(transA, transB, a, s);
}

size_t sgemm_splitk_workspace_size(int M, int N, int K, int splits) {
  if (M <= 8 || N <= 0 || K <= 0 || splits < 0 || splits > kMaxSplits) return 0;
  int kc = 0;
  const int chunks = splitk_chunk(K, splits > 0 ? splits : splitk_pick(M, N, K), &kc);
  return chunks > 1 ? (size_t)chunks * (size_t)M * (size_t)N * sizeof(float) : 0;
}

int fp32gemm_splitk_splits(int M, int N, int K) {
  if (M <= 8 || N <= 0 || K <= 0) return 1;
  int kc = 0;
  return splitk_chunk(K, splitk_pick(M, N, K), &kc);
}

int sgemm_splitk(int transA, int transB, int M, int N, int K, float alpha, const float *A, int lda,
                 const float *B, int ldb, float beta, float *C, int ldc, int splits, float *workspace,
                 size_t workspace_bytes, fp32gemm_stream_t stream) {
  GemmArgs a = pack(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  int rc = check_args(kPosSgemmEx, transA, transB, a);
  if (rc) return rc;
  if (splits < 0 || splits > kMaxSplits) return -14;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (quick_return(a, s, &rc)) return rc;
  int kc = 0;
  const int chunks = M <= 8 ? 1 : splitk_chunk(K, splits > 0 ? splits : splitk_pick(M, N, K), &kc);
  if (chunks <= 1) return run_product(transA, transB, a, s);  // the plain routine, no workspace
  if (workspace == nullptr) return -15;
  if (workspace_bytes < (size_t)chunks * (size_t)M * (size_t)N * sizeof(float)) return -16;
  return run_splitk(transA, transB, a, chunks, kc, workspace, s);
}

int sgemm_splitk_noalloc(int transA, int transB, int M, int N, int K, float alpha, const float *A,
                         int lda, const float *B, int ldb, float beta, float *C, int ldc,
                         int splits, fp32gemm_stream_t stream) {
  GemmArgs a = pack(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  int rc = check_args(kPosSgemmEx, transA, transB, a);
  if (rc) return rc;
  if (splits < 0 || splits > kMaxSplits) return -14;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int kc = 0;
  const bool work = a.M > 0 && a.N > 0 && a.alpha != 0.0f && a.K > 0;
  const int chunks =
      !work || M <= 8 ? 1 : splitk_chunk(K, splits > 0 ? splits : splitk_pick(M, N, K), &kc);
  // checked before anything is enqueued, quick returns included
  if (chunks > 1 && (size_t)chunks * (size_t)M * (size_t)N > kScratchFloats)
    return FP32GEMM_ERR_SCRATCH;
  if (quick_return(a, s, &rc)) return rc;
  if (chunks <= 1) return run_product(transA, transB, a, s);  // no scratch needed
  float *ws = nullptr;
  const hipError_t e = scratch_ptr(&ws);
  if (e != hipSuccess) return (int)e;
  return run_splitk(transA, transB, a, chunks, kc, ws, s);
}

size_t sgemm_streamk_workspace_size(int M, int N, int K) {
  if (M <= 8 || N <= 0 || K <= 0) return 0;
  return streamk_workspace_bytes(streamk_plan(M, N, K, -1, 0));
}

int sgemm_streamk(int transA, int transB, int M, int N, int K, float alpha, const float *A,
                  int lda, const float *B, int ldb, float beta, float *C, int ldc,
                  float *workspace, size_t workspace_bytes, fp32gemm_stream_t stream) {
  return streamk_call(-1, 0, 1, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                      workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream), false);
}

size_t fp32gemm_streamk_plan(int M, int N, int K, int tile, int groups, int *tile_out,
                             int *groups_out, int *ipw_out) {
  if (M <= 0 || N <= 0 || K <= 0 || tile < -1 || tile >= streamk_num_tiles() || groups < 0)
    return 0;
  const SkPlan p = streamk_plan(M, N, K, tile, groups);
  if (tile_out) *tile_out = p.tile;
  if (groups_out) *groups_out = p.groups;
  if (ipw_out) *ipw_out = p.ipw;
  return streamk_workspace_bytes(p);
}

const char *fp32gemm_streamk_tile_name(int tile) { return streamk_tile_name(tile); }

int fp32gemm_streamk_with_config(int tile, int groups, int transA, int transB, int M, int N,
                                 int K, float alpha, const float *A, int lda, const float *B,
                                 int ldb, float beta, float *C, int ldc, float *workspace,
                                 size_t workspace_bytes, fp32gemm_stream_t stream) {
  if (tile < -1 || tile >= streamk_num_tiles()) return FP32GEMM_ERR_CONFIG;
  if (groups < 0) return -2;
  return streamk_call(tile, groups, 3, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C,
                      ldc, workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream),
                      true);
}

const char *fp32gemm_strerror(int code) {
  static const char *const bad[] = {
      "invalid argument 1",  "invalid argument 2",  "invalid argument 3",
      "invalid argument 4",  "invalid argument 5",  "invalid argument 6",
      "invalid argument 7",  "invalid argument 8",  "invalid argument 9",
      "invalid argument 10", "invalid argument 11", "invalid argument 12",
      "invalid argument 13", "invalid argument 14", "invalid argument 15",
      "invalid argument 16", "invalid argument 17", "invalid argument 18"};
  static const char *const bad_high[] = {"invalid argument 19", "invalid argument 20"};
  if (code == 0) return "success";
  if (code == -19 || code == -20) return bad_high[-code - 19];
  if (code == FP32GEMM_ERR_CONFIG) return "unknown configuration id";
  if (code == FP32GEMM_ERR_SCRATCH)
    return "the split-K partial products exceed the 16 MiB static scratch of "
           "sgemm_splitk_noalloc (chunks x M x N floats must be at most 4 Mi)";
  if (code < 0 && code >= -18) return bad[-code - 1];
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
  if (kind == 0) return select_gemm_config(M, N, K, 1);
  if (kind == 1) return select_gemv_config(M, N, K);
  return FP32GEMM_ERR_CONFIG;
}

int fp32gemm_config_max_rows(int kind, int cfg) {
  if (kind == 1) {
    int n = 0;
    const GemvConfig *c = gemv_configs(&n);
    return (cfg >= 0 && cfg < n) ? c[cfg].max_rows : -1;
  }
  if (kind == 0) return (cfg >= 0 && cfg < num_gemm_config_ids()) ? 0x7fffffff : -1;
  return -1;
}

int fp32gemm_round_split(int M, int N, int K, int batch, int *first) {
  const RoundSplit sp = plan_round_split(M, N, K, batch);
  if (first) *first = sp.dim ? sp.first : 0;
  return sp.dim;
}

int fp32gemm_sgemm_with_config(int cfg, int M, int N, int K, float alpha, const float *A,
                               int lda, const float *B, int ldb, float beta, float *C, int ldc,
                               fp32gemm_stream_t stream) {
  if (cfg < -1 || cfg >= num_gemm_config_ids()) return FP32GEMM_ERR_CONFIG;
  const GemmArgs a = pack(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  int rc = check_args(kPosSgemm, 0, 0, a);
  if (rc) return rc;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (quick_return(a, s, &rc)) return rc;
  return cfg < 0 ? run_tiled(0, 0, a, s) : run_gemm(cfg, 0, 0, a, s);
}

int fp32gemm_sgemv_with_config(int cfg, int M, int N, int K, float alpha, const float *A,
                               int lda, const float *B, int ldb, float beta, float *C, int ldc,
                               fp32gemm_stream_t stream) {
  if (cfg < -1 || cfg >= fp32gemm_num_configs(1)) return FP32GEMM_ERR_CONFIG;
  if (M < 1 || M > kSkinnyMaxRows) return -1;
  if (cfg >= 0) {
    int n = 0;
    if (!gemv_config_runs(gemv_configs(&n)[cfg], M)) return FP32GEMM_ERR_CONFIG;
  }
  const GemmArgs a = pack(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  int rc = check_args(kPosSgemm, 0, 0, a);
  if (rc) return rc;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (quick_return(a, s, &rc)) return rc;
  return run_gemv(cfg, 0, a, s);
}

}  // extern "C"
#pragma GCC visibility pop
