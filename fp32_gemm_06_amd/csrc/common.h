// Internal declarations shared by the kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp32gemm {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// Arguments of one C <- alpha A B + beta C call, already validated.
struct GemmArgs {
  int M, N, K;
  float alpha, beta;
  const float *A;
  const float *B;
  float *C;
  int lda, ldb, ldc;
  long long sA, sB, sC;  // element strides between batch entries
  int batch;             // number of products (1 for a single GEMM)
  // Split-K: when > 0, entry b of the batch reduces over k in
  // [b * K, min((b + 1) * K, k_total)) of the whole product (its operands are
  // already offset by sA, sB); 0 for ordinary calls.
  int k_total;
  // Fused epilogue: C[i][j] = act(alpha acc + beta C0 + bias[j]); bias may be
  // NULL (no bias), act is kActNone or kActRelu.
  const float *bias;
  int act;
};

constexpr int kActNone = 0;
constexpr int kActRelu = 1;

// The activation of the fused epilogue: ReLU maps v < 0 to 0 and passes
// everything else (NaN and -0.0 included) unchanged.
__device__ __forceinline__ float apply_act(float v, int act) {
  return (act == kActRelu && v < 0.0f) ? 0.0f : v;
}

// Buffer-resource word 3 for gfx9-family raw buffers: 32-bit data format,
// no swizzle, no index stride.  With a raw resource a load whose byte offset
// is at or past num_records returns zero and a store there is dropped; the
// kernels use that to mask rows/columns outside the matrix without branches.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kRsrcRange = 0x7ffffff0;
constexpr uint32_t kOob = 0x80000000u;  // an offset the range check rejects

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, kRsrcRange,
                                           kRsrcWord3);
}

// One 16-byte-per-lane DMA from a buffer into LDS at dst + 16 * lane
// (buffer_load_dwordx4 ... lds).  The body exists only in the device pass:
// the host pass cannot form an LDS address-space pointer, and the kernels'
// host launch stubs must still be emitted.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, float *dst, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) void lds_void_t;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)dst, 16, off, 0, 0, 0);
#else
  (void)rs; (void)dst; (void)off;
#endif
}

// Whether the 128-bit (DMA) load path may be used: 16-byte aligned operands
// and row lengths / strides that keep every float4 inside one row.  A as
// given moves float4s along K, A^T along M; B as given along N, B^T along K.
inline bool vec4_ok(const GemmArgs &a, bool ta, bool tb) {
  const bool okA = ((uintptr_t)a.A % 16 == 0) && a.lda % 4 == 0 && (ta ? a.M : a.K) % 4 == 0 &&
                   a.sA % 4 == 0;
  const bool okB = ((uintptr_t)a.B % 16 == 0) && a.ldb % 4 == 0 && (tb ? a.K : a.N) % 4 == 0 &&
                   a.sB % 4 == 0;
  return okA && okB && a.k_total % 4 == 0;
}

// Scratch slots kept per (device, stream): a stream gets slot 0..7 on its
// first call that needs one, and keeps it; -1 when all are taken.
constexpr int kStreamSlots = 8;
int stream_slot(hipStream_t s);

// Stream-K work assignment of the tiled kernel (sgemm_kernel.h): workgroup g
// takes units [g ipw, (g + 1) ipw) of the tile-major (tile, K slice) units;
// part holds 2 x grid partial tiles, cnt one arrival counter per tile.
struct SkArgs {
  int ipw;
  float *part;
  unsigned *cnt;
};

// ---- SGEMM (fp32 MFMA) family ---------------------------------------------
typedef hipError_t (*GemmLaunchFn)(const GemmArgs &, bool dma, int group_m, hipStream_t);
struct GemmConfig {
  const char *name;
  int BM, BN, BK, WM, WN;
  int wgs_per_cu;          // workgroups one CU holds (LDS and register limits, 128-bit path)
  GemmLaunchFn launch[4];  // index 2 * transA + transB
};
const GemmConfig *gemm_configs(int *count);
// Per operand-layout combination, in tile-list order (sgemm_nn.hip, ...).
void launchers_nn(GemmLaunchFn *out);
void launchers_nt(GemmLaunchFn *out);
void launchers_tn(GemmLaunchFn *out);
void launchers_tt(GemmLaunchFn *out);
// Stream-K launchers of the tiles in FP32GEMM_SK_TILES, same order.
typedef hipError_t (*SkLaunchFn)(const GemmArgs &, bool dma, int group_m, int groups,
                                 const SkArgs &, hipStream_t);
void sk_launchers_nn(SkLaunchFn *out);
void sk_launchers_nt(SkLaunchFn *out);
void sk_launchers_tn(SkLaunchFn *out);
void sk_launchers_tt(SkLaunchFn *out);

// ---- GEMV (M <= 32) family ------------------------------------------------
struct GemvConfig {
  const char *name;
  int cbw;          // columns of W per workgroup
  int waves;        // waves per workgroup (they split K)
  int unroll;       // rows of W per lane per pass (0: the MFMA kernel)
  int max_rows;     // largest M the configuration runs
  hipError_t (*launch)(const GemmArgs &, int transA, hipStream_t);
};
const GemvConfig *gemv_configs(int *count);

// The GEMV kernels take 1 <= M <= 8, and lda <= 2^17 when op(A) = A^T.
bool gemv_supported(const GemmArgs &a, int transA);
// The column-stripe kernel also takes 9 <= M <= kGemvMaxRows, on row
// capacities 12, 16, 24 and 32 (gemv_row_capacity), in the configurations
// for which gemv_config_runs says so.
constexpr int kGemvMaxRows = 32;
bool gemv_wide_supported(const GemmArgs &a, int transA);
int gemv_row_capacity(int M);
bool gemv_config_runs(const GemvConfig &c, int M);

// Skinny MFMA kernel (skinny.hip), op(A) = A^T up to lda = 2^17; op(B) = B:
// stripes of 16 columns of W for M <= 128, of 32 for M <= 64, of 64 for
// M <= 32.
constexpr int kSkinnyMaxRows = 128;
bool skinny_supported(const GemmArgs &a, int transA);
hipError_t launch_skinny16(const GemmArgs &a, int transA, hipStream_t s);
hipError_t launch_skinny32(const GemmArgs &a, int transA, hipStream_t s);
hipError_t launch_skinny64(const GemmArgs &a, int transA, hipStream_t s);
// The same for op(B) = B^T (W stored N x K), 16 stored rows of W per workgroup.
hipError_t launch_skinny_tb(const GemmArgs &a, int transA, hipStream_t s);
// Stripe widths in blocks of 16 columns (1, 2 or 4) for batch products of N
// columns: the skinny MFMA kernel's for M rows, and the column-stripe GEMV's.
int skinny_stripe_blocks(int M, int N, int batch, bool transposed_w);
int gemv_stripe_blocks(int N, int batch);

// Small-M product with W stored K x N, K split across workgroups
// (gemv_split.hip): 256-column blocks x K chunks, the chunks' partial sums
// added in chunk order inside the same kernel.  gemv_split_pays: whether the
// dispatcher takes it for this shape (one product, M <= 8).  The
// _serial form walks the chunks in one workgroup per column block and needs
// no scratch; its results are bit-identical.
// gemv_split_waves: the pipeline for the shape's chunk length (4 or 8 waves).
bool gemv_split_pays(int M, int N, int K, int batch);
int gemv_split_waves(int N, int K);
hipError_t launch_gemv_split4(const GemmArgs &a, int transA, hipStream_t s);
hipError_t launch_gemv_split4_serial(const GemmArgs &a, int transA, hipStream_t s);
hipError_t launch_gemv_split8(const GemmArgs &a, int transA, hipStream_t s);
hipError_t launch_gemv_split8_serial(const GemmArgs &a, int transA, hipStream_t s);

// Small-M product with op(B) = B^T (B stored N x K): row-dot kernel.
// rows_per_wave is 1 or 2; <= 0 picks from M.
hipError_t launch_gemv_rows(const GemmArgs &a, int transA, int rows_per_wave, hipStream_t s);

// C <- beta * C (beta == 0 writes zeros without reading C).
hipError_t launch_scale(const GemmArgs &a, hipStream_t s);

// Split-K (csrc/splitk.hip).  The K range is cut into chunks of kc floats (a
// multiple of 32); splitk_chunk returns kc for `splits` requested chunks and
// the number of chunks that leaves.  C <- alpha * sum_s ws[s] + beta * C,
// summed in ascending s, where ws holds `splits` packed M x N partials.
int splitk_chunk(int K, int splits, int *kc);
int splitk_pick(int M, int N, int K);
hipError_t launch_splitk_reduce(const float *ws, int splits, int M, int N, float alpha, float beta,
                                float *C, int ldc, hipStream_t s);

// Stream-K (streamk.hip): plan (tile index into FP32GEMM_SK_TILES, number of
// workgroups, units per workgroup, tiles of C; tile -1 when none), the
// workspace it needs, and the launch.  tile < 0 / groups <= 0 choose.
struct SkPlan {
  int tile, groups, ipw;
  long long tiles;
};
SkPlan streamk_plan(int M, int N, int K, int tile, int groups);
size_t streamk_workspace_bytes(const SkPlan &p);
hipError_t launch_streamk(int ta, int tb, const GemmArgs &a, const SkPlan &p, float *workspace,
                          hipStream_t s);
int streamk_num_tiles();
const char *streamk_tile_name(int t);

// SGEMM configuration ids combine a tile shape with the tile-ordering group
// (tile-rows per strip): id = tile_index * kNumGroups + group_index.
constexpr int kNumGroups = 4;
constexpr int kGroups[kNumGroups] = {1, 2, 4, 8};

int num_gemm_config_ids();
const char *gemm_config_name(int id);

// Per-shape table (generated by the tuning sweep; single products) and the
// fallback model over the tiles of all `batch` entries.
int select_gemm_config(int M, int N, int K, int batch);
// The fallback model alone, for a grid of `mult` products of M x N x K (batch
// entries or split-K chunks); *rate receives the modelled TFLOP/s.
int model_gemm_config(int M, int N, int K, int mult, double *rate);
// A tiled product as two launches over ranges of C: columns (dim 1) or rows
// (dim 2) [0, first) in whole rounds of 256x256 tiles with configuration
// main_cfg, the rest as a second product with its own configuration.
// dim 0: one launch.
struct RoundSplit {
  int dim, first, main_cfg;
};
RoundSplit plan_round_split(int M, int N, int K, int batch);
int select_gemv_config(int M, int N, int K);
// GEMV choice for `batch` products of M x N (the grid is stripes x batch).
int select_gemv_config_batched(int M, int N, int K, int batch);

}  // namespace fp32gemm
