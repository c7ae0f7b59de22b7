// Stream-K: C <- alpha op(A) op(B) + beta C as one persistent grid that
// splits the product's (tile, K slice) units evenly over its workgroups.
//
// The pages credit part of the vendor library's lead to splitting K on grids
// that would leave SMs idle ("CUDA 矩阵乘法优化：从朴素 Kernel 到接近
// cuBLAS", section "10. cuBLAS 领先的性能差异").  Split-K (splitk.hip) cuts
// every tile into the same number of chunks and adds them in a second
// kernel; here the units of all tiles are dealt out in equal runs, so a
// workgroup may finish one tile, do whole tiles, and start another, and a
// tile shared by several workgroups is completed in the same kernel by the
// last of them to arrive (sgemm_kernel.h, SK form).  The partial tiles go to
// the caller's workspace; the arrival counters live in device memory the
// library reserves per stream (zero between calls, put back to zero by the
// kernel), or, when a call has no slot, in the workspace, cleared by a small
// kernel first.  Either way the partial tiles are added in K order, so the
// result depends only on the shape and the plan.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "sgemm_kernel.h"

namespace fp32gemm {
namespace {

constexpr int kSkMaxTiles = 4096;  // tiles per call with reserved counters
constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) unsigned g_sk_counters[kStreamSlots][kSkMaxTiles] = {};
std::mutex g_sk_mu;
unsigned *g_sk_counters_ptr[kMaxDevices] = {};

// Device address of this device's counter array (looked up once per device).
hipError_t counters_base(unsigned **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_sk_mu);
  if (g_sk_counters_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_sk_counters));
    if (e != hipSuccess) return e;
    g_sk_counters_ptr[dev] = static_cast<unsigned *>(p);
  }
  *out = g_sk_counters_ptr[dev];
  return hipSuccess;
}

__global__ void __launch_bounds__(256) zero_counters(unsigned *p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

struct SkTile {
  const char *name;
  int bm, bn, occ;
};
const SkTile kSkTiles[] = {
#define FP32GEMM_SK_ROW(BM, BN, BK, WM, WN, KS, P, OCC, MF) \
  {#BM "x" #BN "x" #BK "_w" #WM "x" #WN, BM, BN, OCC},
    FP32GEMM_SK_TILES(FP32GEMM_SK_ROW)
#undef FP32GEMM_SK_ROW
};
constexpr int kNumSkTiles = sizeof(kSkTiles) / sizeof(kSkTiles[0]);
constexpr int kSliceK = 32;  // every stream-K tile takes K slices of 32

// Time of one K slice of one workgroup (us) with w workgroups of the tile
// per CU, w = 1 .. the tile's occupancy: measured at 4096^3 with whole
// tiles per workgroup (all workgroups at the same K position).
const double kSkSliceUs[kNumSkTiles][4] = {{1.903, 0.0, 0.0, 0.0},
                                           {0.602, 1.059, 1.580, 2.015}};

long long tiles_of(int t, int M, int N) {
  return (long long)((M + kSkTiles[t].bm - 1) / kSkTiles[t].bm) *
         ((N + kSkTiles[t].bn - 1) / kSkTiles[t].bn);
}

}  // namespace

int streamk_num_tiles() { return kNumSkTiles; }
const char *streamk_tile_name(int t) {
  return t >= 0 && t < kNumSkTiles ? kSkTiles[t].name : nullptr;
}

// The plan: tile shape, number of workgroups and units per workgroup.
// Candidates are one round of w workgroups per CU (256 w, w up to the
// tile's occupancy; fewer when there are fewer units), or the caller's
// tile and / or count.  The estimate: the units of one workgroup at the
// measured slice time for w per CU, plus about 3 us of launch, first loads
// and epilogue; when tiles are shared, 2 us for publishing and counting,
// 0.5 us per segment the last workgroup reads back, and up to 15% slower
// slices when the workgroups' K positions differ (they no longer read the
// same A and B slices at the same time, so fewer of their loads hit L2;
// measured as 69% -> 26% L2 hits at 1536^3).
SkPlan streamk_plan(int M, int N, int K, int tile, int groups) {
  SkPlan best = {-1, 0, 0, 0};
  double best_t = 0.0;
  const long long nk = (K + kSliceK - 1) / kSliceK;
  for (int t = 0; t < kNumSkTiles; ++t) {
    if (tile >= 0 && t != tile) continue;
    const long long tiles = tiles_of(t, M, N);
    const long long units = tiles * nk;
    for (int w = 1; w <= kSkTiles[t].occ; ++w) {
      if (groups > 0 && w > 1) break;
      long long g = groups > 0 ? groups : 256LL * w;
      if (g > units) g = units;
      const long long ipw = (units + g - 1) / g;
      g = (units + ipw - 1) / ipw;
      const int per_cu = (int)std::min<long long>((g + 255) / 256, kSkTiles[t].occ);
      const double slice = kSkSliceUs[t][per_cu - 1];
      double est = ipw * slice + 3.0;
      if (ipw % nk != 0) {
        long long a = ipw % nk, b = nk;  // distinct K positions: nk / gcd(ipw mod nk, nk)
        while (b != 0) {
          const long long r = a % b;
          a = b;
          b = r;
        }
        const double phases = (double)std::min<long long>(nk / a, 16);
        const double nseg = ipw < nk ? (double)((nk + ipw - 1) / ipw + 1) : 2.0;
        est = ipw * slice * (1.0 + 0.15 * phases / 16.0) + 3.0 + 2.0 + 0.5 * nseg;
      }
      if (best.tile < 0 || est < best_t) {
        best = {t, (int)g, (int)ipw, tiles};
        best_t = est;
      }
    }
  }
  return best;
}

size_t streamk_workspace_bytes(const SkPlan &p) {
  if (p.tile < 0) return 0;
  const size_t part = 2 * (size_t)p.groups * kSkTiles[p.tile].bm * kSkTiles[p.tile].bn;
  return (part + (size_t)p.tiles + 64) * sizeof(float);
}

hipError_t launch_streamk(int ta, int tb, const GemmArgs &a, const SkPlan &p, float *workspace,
                          hipStream_t s) {
  static SkLaunchFn fns[4][kNumSkTiles];
  static std::once_flag once;
  std::call_once(once, [] {
    sk_launchers_nn(fns[0]);
    sk_launchers_nt(fns[1]);
    sk_launchers_tn(fns[2]);
    sk_launchers_tt(fns[3]);
  });
  if (p.tile < 0 || p.tile >= kNumSkTiles) return hipErrorInvalidValue;
  SkArgs sk;
  sk.ipw = p.ipw;
  sk.part = workspace;
  const size_t part = 2 * (size_t)p.groups * kSkTiles[p.tile].bm * kSkTiles[p.tile].bn;
  const int slot = p.tiles <= kSkMaxTiles ? stream_slot(s) : -1;
  if (slot >= 0) {
    unsigned *base = nullptr;
    const hipError_t e = counters_base(&base);
    if (e != hipSuccess) return e;
    sk.cnt = base + (size_t)slot * kSkMaxTiles;
  } else {
    // counters after the partial tiles, 256-byte aligned, cleared first
    const size_t off = (part + 63) / 64 * 64;
    sk.cnt = reinterpret_cast<unsigned *>(workspace + off);
    const int n = (int)p.tiles;
    hipLaunchKernelGGL(zero_counters, dim3((n + 255) / 256), dim3(256), 0, s, sk.cnt, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return fns[2 * ta + tb][p.tile](a, vec4_ok(a, ta, tb), 8, p.groups, sk, s);
}

}  // namespace fp32gemm
