// Small-M product Y[M x N] <- alpha X[M x K] W[K x N] + beta Y, 1 <= M <= 8,
// with K split across workgroups and the partial sums added inside the same
// kernel.
//
// This is the decode shape of "GPU GEMM 优化完全拆解（一）", section "LLM 推理
// 本质上是 GEMM 的串联": the time is the time to stream W once from HBM.  With
// W stored K x N, a workgroup that owns a column block over all of K reads a
// short piece of every row (64 bytes for 16 columns at N = 4096, which gives
// the 256 workgroups that fill the GPU); the memory system serves such
// pieces far slower than long runs.  Here a workgroup owns 256 columns (one
// 1 KB run of a row per wave instruction) over a chunk of K, so N = 4096
// still gives 16 column blocks x 16 chunks = 256 workgroups.  The chunks'
// partial sums are added in a fixed order by the last workgroup of each
// column block to finish, in the same kernel: the K split with a reduction
// step of "CUDA 矩阵乘法优化：从朴素 Kernel 到接近 cuBLAS", section "10. cuBLAS
// 领先的性能差异", without the second launch.
//
// Cross-workgroup protocol (no spin-wait; every workgroup runs to the end):
//  1. each workgroup writes its partial sums with agent-scope atomic stores,
//     which the compiler emits as stores with the sc1 bit: they write
//     through the XCD's L2, so they are visible to every XCD once complete;
//  2. it waits for its own stores to complete (s_waitcnt vmcnt(0)), then one
//     thread adds 1 to the column block's counter (agent-scope atomic add);
//  3. the workgroup that reads count - 1 is the last: its loads of the
//     partials are agent-scope atomic loads (sc1), which do not return stale
//     copies from its own L2.  It adds chunk 0, 1, 2, ... in that order,
//     applies alpha, beta, the bias and the activation, stores Y and puts
//     the counter back to 0 for the next call.
// An agent-scope release fence would also write back every dirty line of
// the XCD's L2 (buffer_wbl2) and an acquire fence would invalidate it
// (buffer_inv); both serialise per workgroup and cost far more than the
// whole product.  They are not needed here: every value published across
// workgroups is written and read by agent-scope atomics, and the wait in
// step 2 orders their completion before the counter update.
//
// Scratch: partial sums and counters live in file-scope device arrays, in
// slots; each stream gets its own slot on first use (8 per device), so
// calls on one stream reuse it in stream order and calls on different
// streams never share one.  With every slot taken, the same kernel runs
// with one workgroup per column block that walks the chunks itself and adds
// their partial sums in the same order: bit-identical results, no scratch.
// Either way the summation order depends only on the shape, never on timing.
#include <mutex>
#include <vector>

#include "common.h"

namespace fp32gemm {
namespace {

constexpr int kSplitCW = 256;          // columns per workgroup (64 lanes x float4)
constexpr int kSplitMaxRowsM = 8;      // largest M
constexpr int kSplitMaxGroups = 256;   // column blocks x chunks per call with scratch
constexpr int kSplitKcMax = 1024;      // rows of K per chunk (X chunk staged in LDS)

// Partial sums: [column block][chunk][row m][column], MR rows per call.
__device__ __attribute__((aligned(256)))
float g_split_partials[kStreamSlots][(size_t)kSplitMaxGroups * kSplitMaxRowsM * kSplitCW];
// Arrival counters, one per column block; zero between calls.
__device__ __attribute__((aligned(256))) unsigned g_split_counters[kStreamSlots][kSplitMaxGroups] =
    {};

// Stream -> slot, per device.  Slots are never released: a stream keeps its
// slot for the life of the process.
std::mutex g_slot_mu;
struct SlotOwner {
  int dev;
  hipStream_t stream;
};
std::vector<SlotOwner> g_slot_owners;

}  // namespace

int stream_slot(hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  std::lock_guard<std::mutex> lk(g_slot_mu);
  int used = 0;
  for (const SlotOwner &o : g_slot_owners) {
    if (o.dev != dev) continue;
    if (o.stream == s) return used;
    ++used;
  }
  if (used >= kStreamSlots) return -1;
  g_slot_owners.push_back({dev, s});
  return used;
}

namespace {

// A compile-time count, to pass group sizes to a generic lambda.
template <int V> struct Count { static constexpr int value = V; };

// Workgroup (column block cb, chunk s): rows [s KC, (s + 1) KC) of K, 256
// columns.  Wave w of a pass takes U consecutive rows, each wave instruction
// one 1 KB run of a row (lane l: columns 4 l .. 4 l + 3).  D passes of
// loads are in flight while one is multiplied; the chunk's passes run in
// blocks of D, starting at a block that depends on the column block.  Workgroup ids run over the
// chunks of one column block first; the hardware deals consecutive ids to
// the 8 XCDs in turn, so each XCD streams whole rows of its chunks (timed
// at 4096 x 4096, M = 1, against consecutive column blocks of one chunk:
// 16.4 against 17.3 us).
template <int MR, bool VEC, int NW, int U, int D, bool SERIAL>
__global__ void __launch_bounds__(NW * 64)
gemv_split_kernel(GemmArgs a, int transA, int S, int KC, int slot) {
  constexpr int CW = kSplitCW;
  constexpr int THREADS = NW * 64;
  constexpr int ROWS = NW * U;                 // rows of W per pass
  constexpr int OUTS = MR * CW;                // outputs of a column block
  constexpr int OPT = (OUTS + THREADS - 1) / THREADS;  // outputs per thread
  constexpr int XS = MR * kSplitKcMax;         // X chunk
  constexpr int XPT = (XS + THREADS - 1) / THREADS;    // X values staged per thread
  constexpr int RS = NW * MR * CW;             // per-wave sums
  static_assert(U % 4 == 0, "X is read in float4 pieces");
  __shared__ __attribute__((aligned(16))) float smem[XS > RS ? XS : RS];
  __shared__ int last;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = a.N, K = a.K;
  const int id = blockIdx.x;
  const int cb = SERIAL ? id : id / S;
  const int s_first = SERIAL ? 0 : id % S;
  const int s_end = SERIAL ? S : s_first + 1;
  const int n0 = cb * CW;
  const int c0 = 4 * lane;                     // first column of this lane in the block
  // X element (m, k) sits at A + k * xk + m * xm
  const uint32_t xk = transA ? (uint32_t)a.lda : 1u, xm = transA ? 1u : (uint32_t)a.lda;
  const float alpha = a.alpha, beta = a.beta;

  float total[OPT];
#pragma unroll
  for (int j = 0; j < OPT; ++j) total[j] = 0.0f;

  for (int s = s_first; s < s_end; ++s) {
    const int k0 = s * KC;
    const int kend = min(K, k0 + KC);

    // rows k0 + r0 + wave * U + u of this lane's four columns (zeros past
    // the chunk); the wave's first row goes into the buffer base so byte
    // offsets stay small
    auto load_w = [&](float (&w)[U][4], int r0) {
      const int rw = k0 + r0 + wave * U;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.B + (size_t)rw * a.ldb + n0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool row_ok = rw + u < kend;
        if constexpr (VEC) {
          const uint32_t off = (row_ok & (n0 + c0 < N)) ? (uint32_t)(u * a.ldb + c0) * 4u : kOob;
          const floatx4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) w[u][e] = v[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t off =
                (row_ok & (n0 + c0 + e < N)) ? (uint32_t)(u * a.ldb + c0 + e) * 4u : kOob;
            w[u][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
          }
        }
      }
    };

    // X(m, k0 .. k0 + KC) as [m][kk] (zeros past the chunk): its loads go
    // out first, then the first D passes of W, so the two latencies overlap
    float xr[XPT];
    {
      const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.A + (size_t)k0 * xk);
#pragma unroll
      for (int j = 0; j < XPT; ++j) {
        const int i = tid + j * THREADS, m = i / KC, kk = i - m * KC;
        const bool ok = (i < MR * KC) & (k0 + kk < kend);
        const uint32_t off = ok ? ((uint32_t)kk * xk + (uint32_t)m * xm) * 4u : kOob;
        xr[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, off, 0, 0));
      }
    }
    // the chunk's blocks of D passes start at a phase that depends on the
    // column block, so the column blocks of one chunk do not all read the
    // same rows at the same time
    const int nblk = KC / (D * ROWS);
    const int phase = (cb % 4) * nblk / 4;
    float w[D][U][4];
#pragma unroll
    for (int d = 0; d < D; ++d) load_w(w[d], phase * D * ROWS + d * ROWS);
    __syncthreads();  // the previous chunk's sums have been read (SERIAL)
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int i = tid + j * THREADS;
      if (i < MR * KC) smem[i] = xr[j];
    }
    __syncthreads();

    float acc[MR][4];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[m][e] = 0.0f;
    // every lane of a wave uses the same rows, so the X reads are broadcasts
    auto multiply = [&](const float (&wv)[U][4], int r0) {
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int q = 0; q < U / 4; ++q) {
          const floatx4 xv =
              *reinterpret_cast<const floatx4 *>(&smem[m * KC + r0 + wave * U + 4 * q]);
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[m][e] += xv[t] * wv[4 * q + t][e];
        }
    };
    // KC is a multiple of D passes; each multiply frees its registers for
    // the pass D ahead (after the last block: out-of-range offsets, no
    // traffic)
    for (int it = 0; it < nblk; ++it) {
      const int r0 = ((it + phase) % nblk) * D * ROWS;
      const int rn = it + 1 < nblk ? ((it + 1 + phase) % nblk) * D * ROWS : KC + D * ROWS;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        multiply(w[d], r0 + d * ROWS);
        __builtin_amdgcn_sched_barrier(0);
        load_w(w[d], rn + d * ROWS);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // per-wave sums into LDS (the X chunk is no longer read), then the waves
    // in wave order
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MR; ++m)
      *reinterpret_cast<floatx4 *>(&smem[(wave * MR + m) * CW + c0]) =
          floatx4{acc[m][0], acc[m][1], acc[m][2], acc[m][3]};
    __syncthreads();
#pragma unroll
    for (int j = 0; j < OPT; ++j) {
      const int o = tid + j * THREADS;
      if (OUTS % THREADS == 0 || o < OUTS) {
        float p = smem[o];
#pragma unroll
        for (int w2 = 1; w2 < NW; ++w2) p += smem[w2 * OUTS + o];
        if constexpr (SERIAL) {
          total[j] = (s == 0) ? p : total[j] + p;
        } else {
          float *ws = &g_split_partials[slot][((size_t)cb * S + s) * OUTS];
          __hip_atomic_store(&ws[o], p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }

  if constexpr (!SERIAL) {
    // publish: this workgroup's partial sums have completed, then count it
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      const unsigned before = __hip_atomic_fetch_add(&g_split_counters[slot][cb], 1u,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = before == (unsigned)(S - 1);
    }
    __syncthreads();
    if (!last) return;
    asm volatile("" ::: "memory");
    const float *ws = &g_split_partials[slot][(size_t)cb * S * OUTS];
    // Chunks in order, in groups of 16, 8, 4, 2 and 1 chunks (at most 64
    // loads per thread, over all of the thread's outputs).  A group's loads
    // have no conditions, so they are issued back to back and cost one
    // memory round trip; the output index is clamped into this column
    // block's partial sums (threads past OUTS load a valid value they do not
    // use).
    constexpr int GMAX = 64 / OPT >= 16 ? 16 : (64 / OPT > 0 ? 64 / OPT : 1);
    auto group = [&](auto size, int s0) {
      constexpr int GG = decltype(size)::value;
      float v[OPT][GG];
#pragma unroll
      for (int j = 0; j < OPT; ++j) {
        const int o = min(tid + j * THREADS, OUTS - 1);
#pragma unroll
        for (int i = 0; i < GG; ++i)
          v[j][i] = __hip_atomic_load(&ws[(size_t)(s0 + i) * OUTS + o], __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int j = 0; j < OPT; ++j)
#pragma unroll
        for (int i = 0; i < GG; ++i) total[j] = s0 + i == 0 ? v[j][i] : total[j] + v[j][i];
    };
    int s0 = 0;
    for (; s0 + GMAX <= S; s0 += GMAX) group(Count<GMAX>{}, s0);
    if constexpr (GMAX > 8) {
      if (s0 + 8 <= S) group(Count<8>{}, s0), s0 += 8;
    }
    if constexpr (GMAX > 4) {
      if (s0 + 4 <= S) group(Count<4>{}, s0), s0 += 4;
    }
    if constexpr (GMAX > 2) {
      if (s0 + 2 <= S) group(Count<2>{}, s0), s0 += 2;
    }
    if constexpr (GMAX > 1) {
      if (s0 < S) group(Count<1>{}, s0);
    }
    if (tid == 0)
      __hip_atomic_store(&g_split_counters[slot][cb], 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }

  // alpha / beta update, bias and activation
#pragma unroll
  for (int j = 0; j < OPT; ++j) {
    const int o = tid + j * THREADS;
    const int m = o / CW, n = n0 + o % CW;
    if ((OUTS % THREADS == 0 || o < OUTS) && n < N) {
      float *y = a.C + (size_t)m * a.ldc + n;
      float out = alpha * total[j];
      if (beta != 0.0f) out += beta * *y;
      if (a.bias) out += a.bias[n];
      *y = apply_act(out, a.act);
    }
  }
}

// Chunking for a shape: about `target` workgroups, chunks a multiple of
// `step` rows (whole groups of D passes) and at most kSplitKcMax.
struct SplitPlan {
  int ncb, S, KC;
};

SplitPlan split_plan(int N, int K, int target, int step) {
  SplitPlan p;
  p.ncb = (N + kSplitCW - 1) / kSplitCW;
  int s = target / p.ncb;
  if (s < 1) s = 1;
  int kc = (K + s - 1) / s;
  kc = (kc + step - 1) / step * step;
  const int kc_max = kSplitKcMax / step * step;
  if (kc > kc_max) kc = kc_max;
  p.KC = kc;
  p.S = (K + kc - 1) / kc;
  return p;
}

template <bool VEC, int NW, int U, int D, bool SERIAL>
hipError_t launch_split_m(const GemmArgs &a, int transA, const SplitPlan &p, int slot,
                          hipStream_t s) {
  const dim3 grid((unsigned)(SERIAL ? p.ncb : p.ncb * p.S)), block(NW * 64);
  switch (a.M) {
#define FP32GEMM_SPLIT_CASE(MR)                                                               \
  case MR:                                                                                    \
    hipLaunchKernelGGL((gemv_split_kernel<MR, VEC, NW, U, D, SERIAL>), grid, block, 0, s, a,  \
                       transA, p.S, p.KC, slot);                                              \
    break;
    FP32GEMM_SPLIT_CASE(1)
    FP32GEMM_SPLIT_CASE(2)
    FP32GEMM_SPLIT_CASE(3)
    FP32GEMM_SPLIT_CASE(4)
    FP32GEMM_SPLIT_CASE(5)
    FP32GEMM_SPLIT_CASE(6)
    FP32GEMM_SPLIT_CASE(7)
    FP32GEMM_SPLIT_CASE(8)
#undef FP32GEMM_SPLIT_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Two pipelines, 4 rows per pass and 4 passes in flight: 4 waves (64 KB
// of W in flight per workgroup) or 8 waves (128 KB).  Timed at 4096 x 4096,
// M = 1, cold, in one run: 14.7 us on 4 waves against 15.2 on 8, and
// 16.0 / 15.7 without the phases; phases on every pass instead of every 4
// passes took 22 us.  Between GPUs the two pipelines trade places by a few
// per cent (4096^2: 15.8 / 16.1 us on another); the swept shapes take the
// faster one from the per-shape table, other shapes 4 waves for chunks of
// up to 256 rows and 8 beyond (4096 x 8192, M = 1: 26.9 us on 8 against
// 28.8 on 4).  FORCE_SERIAL: the scratch-free form even when a slot is
// free (tests).
constexpr int kSplitU = 4, kSplitD = 4;
constexpr int kSplitStep = 8 * kSplitU * kSplitD;  // chunk granularity, both pipelines

template <int NW, bool FORCE_SERIAL>
hipError_t launch_split(const GemmArgs &a, int transA, hipStream_t s) {
  if (!gemv_supported(a, transA) || a.batch != 1) return hipErrorInvalidValue;
  const SplitPlan p = split_plan(a.N, a.K, kSplitMaxGroups, kSplitStep);
  const bool vec = ((uintptr_t)a.B % 16 == 0) && a.N % 4 == 0 && a.ldb % 4 == 0;
  int slot = -1;
  if (!FORCE_SERIAL && p.ncb * p.S <= kSplitMaxGroups) slot = stream_slot(s);
  constexpr int U = kSplitU, D = kSplitD;
  if (slot >= 0)
    return vec ? launch_split_m<true, NW, U, D, false>(a, transA, p, slot, s)
               : launch_split_m<false, NW, U, D, false>(a, transA, p, slot, s);
  return vec ? launch_split_m<true, NW, U, D, true>(a, transA, p, -1, s)
             : launch_split_m<false, NW, U, D, true>(a, transA, p, -1, s);
}

}  // namespace

// Where the split kernel is chosen (W stored K x N, one product): timed
// against the column-stripe and skinny kernels over 25 swept shapes, cold
// weights.  For M <= 4 it wins from about 12 M weights on (M = 1: 3072 x
// 4096 13.1 against 18.1 us; 4096^2 15.3 against 17.8; 4096 x 11008 33.1
// against 43.7; 2048 x 8192 15.8 against 30.4) and loses on small products
// (2048^2: 7.1 against 6.0), where its fixed cost (partial sums, counter,
// final sum: about 2 us) is a larger share.  For M = 5..8 it wins while the
// weight has at most 16 column blocks (4096^2, M = 8: 19.2 against 20.2 on
// the skinny MFMA kernel; 4096 x 11008: 38.7 against 48.9); with more
// column blocks the skinny kernel keeps it (8192^2: 48.0 against 50.1;
// 11008 x 4096: 37.0 against 37.8).  Above 64 column blocks the other
// kernels have enough workgroups without a split (1 x 32000 x 4096: 92.7
// against 96.1).
bool gemv_split_pays(int M, int N, int K, int batch) {
  if (batch != 1 || M < 1 || M > kSplitMaxRowsM) return false;
  const SplitPlan p = split_plan(N, K, kSplitMaxGroups, kSplitStep);
  if (p.S < 2 || p.ncb * p.S > kSplitMaxGroups || p.ncb > 64) return false;
  const long long w = (long long)N * K;
  if (M <= 4) return w >= (12LL << 20);
  return p.ncb <= 16 && w >= (16LL << 20);
}

int gemv_split_waves(int N, int K) {
  return split_plan(N, K, kSplitMaxGroups, kSplitStep).KC <= 256 ? 4 : 8;
}

hipError_t launch_gemv_split4(const GemmArgs &a, int transA, hipStream_t s) {
  return launch_split<4, false>(a, transA, s);
}
hipError_t launch_gemv_split4_serial(const GemmArgs &a, int transA, hipStream_t s) {
  return launch_split<4, true>(a, transA, s);
}
hipError_t launch_gemv_split8(const GemmArgs &a, int transA, hipStream_t s) {
  return launch_split<8, false>(a, transA, s);
}
hipError_t launch_gemv_split8_serial(const GemmArgs &a, int transA, hipStream_t s) {
  return launch_split<8, true>(a, transA, s);
}

}  // namespace fp32gemm
