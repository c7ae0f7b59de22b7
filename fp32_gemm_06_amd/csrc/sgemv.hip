// Small-M product Y[M x N] <- alpha X[M x K] W[K x N] + beta Y, 1 <= M <= 8.
//
// This is the decode-phase shape of "GPU GEMM 优化完全拆解（一）", section
// "LLM 推理本质上是 GEMM 的串联": M is the batch, and the work is bound by
// the bandwidth needed to stream W once, not by arithmetic.  The pages give
// no kernel for it; the design applies their coalescing rule ("GPU 基础原理",
// section "4.3 合并加载"; 128-bit loads as in "CUDA 矩阵乘法优化", section
// "7. Kernel 6") and the split-K reduction that the worklog credits for
// small problems ("CUDA 矩阵乘法优化", section "10. cuBLAS 领先的性能差异",
// split-K and a reduction step), with a deterministic reduction order.
//
// Mapping.  A workgroup owns a column block of 64 lanes x 4 columns (one
// 1 KB row segment of W per wave instruction) and a range of R rows of W
// (the K split).  Its waves take interleaved chunks of U rows; each lane
// keeps U 128-bit loads in flight and M x 4 fp32 accumulators.  X values are
// the same for the whole wave and come in through scalar loads.  The waves'
// partial sums are added in LDS in wave order; with one split the workgroup
// writes Y directly, otherwise it writes its partial sums to a workspace and
// the last workgroup of the column block to finish (counted with an atomic
// counter) adds the splits in split order, applies alpha / beta and resets
// the counter.  No float atomics: the result does not depend on timing.
#include "common.h"

namespace fp32gemm {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

template <int MR, bool VEC, int U>
__global__ void __launch_bounds__(kThreads)
sgemv_kernel(GemmArgs a, int rows_per_split, float *work, unsigned *counters) {
  constexpr int VW = VEC ? 4 : 1;   // columns per lane
  constexpr int CB = 64 * VW;       // columns per workgroup
  __shared__ float red[kWaves][MR][CB];
  __shared__ int is_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cb = blockIdx.x, sp = blockIdx.y, splits = gridDim.y;
  const int n0 = cb * CB;
  const int kb = sp * rows_per_split;
  const int ke = min(a.K, kb + rows_per_split);

  // Column validity is fixed per lane: a lane outside N gets the rejected
  // offset and loads zeros.
  const int col = lane * VW;
  const bool col_ok = n0 + col < a.N;

  float acc[MR][VW];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int e = 0; e < VW; ++e) acc[m][e] = 0.0f;

  const size_t ldb = (size_t)a.ldb;
  for (int k = kb + wave * U; k < ke; k += kWaves * U) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.B + (size_t)k * ldb + n0);
    if (k + U <= ke) {
      float w[U][VW];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t off = col_ok ? (uint32_t)(u * a.ldb + col) * 4u : kOob;
        if constexpr (VEC) {
          const floatx4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) w[u][e] = v[e];
        } else {
          w[u][0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          const float x = a.A[(size_t)m * a.lda + k + u];
#pragma unroll
          for (int e = 0; e < VW; ++e) acc[m][e] += x * w[u][e];
        }
    } else {
      for (int u = 0; u < ke - k; ++u) {
        const uint32_t off = col_ok ? (uint32_t)(u * a.ldb + col) * 4u : kOob;
        float w[VW];
        if constexpr (VEC) {
          const floatx4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = v[e];
        } else {
          w[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          const float x = a.A[(size_t)m * a.lda + k + u];
#pragma unroll
          for (int e = 0; e < VW; ++e) acc[m][e] += x * w[e];
        }
      }
    }
  }

  // Sum the waves' partial results in wave order.
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int e = 0; e < VW; ++e) red[wave][m][col + e] = acc[m][e];
  __syncthreads();

  constexpr int OUTS = MR * CB;                      // outputs of this workgroup
  constexpr int PER = (OUTS + kThreads - 1) / kThreads;
  float part[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int o = tid + p * kThreads;
    float s = 0.0f;
    if (o < OUTS) {
      const int m = o / CB, c = o % CB;
      s = red[0][m][c];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) s += red[w][m][c];
    }
    part[p] = s;
  }

  const float alpha = a.alpha, beta = a.beta;
  auto finish = [&](int o, float s) {
    const int m = o / CB, c = o % CB;
    if (n0 + c >= a.N) return;
    float *y = a.C + (size_t)m * a.ldc + n0 + c;
    float out = alpha * s;
    if (beta != 0.0f) out += beta * *y;
    *y = out;
  };

  if (splits == 1) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int o = tid + p * kThreads;
      if (o < OUTS) finish(o, part[p]);
    }
    return;
  }

  // Publish this split's partial sums, then count arrivals for the column block.
  const size_t N = (size_t)a.N;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int o = tid + p * kThreads;
    if (o < OUTS) {
      const int m = o / CB, c = o % CB;
      if (n0 + c < a.N) work[((size_t)sp * MR + m) * N + n0 + c] = part[p];
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = atomicAdd(&counters[cb], 1u);
    is_last = (prev == (unsigned)(splits - 1));
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();

  // Last arrival: add the splits in split order.
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int o = tid + p * kThreads;
    if (o < OUTS) {
      const int m = o / CB, c = o % CB;
      if (n0 + c < a.N) {
        const float *src = work + (size_t)m * N + n0 + c;
        float s = src[0];
        for (int q = 1; q < splits; ++q) s += src[(size_t)q * MR * N];
        finish(o, s);
      }
    }
  }
  if (tid == 0) counters[cb] = 0u;  // ready for the next call on this stream
}

// C <- beta * C; beta == 0 stores zeros without reading C.
__global__ void __launch_bounds__(256) scale_kernel(float *C, int M, int N, int ldc, float beta) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= N) return;
  for (int i = blockIdx.y; i < M; i += gridDim.y) {
    float *p = C + (size_t)i * ldc + j;
    *p = (beta == 0.0f) ? 0.0f : beta * *p;
  }
}

template <int MR, bool VEC, int U>
void launch_one(dim3 grid, const GemmArgs &a, int R, float *work, unsigned *counters, hipStream_t s) {
  hipLaunchKernelGGL((sgemv_kernel<MR, VEC, U>), grid, dim3(kThreads), 0, s, a, R, work, counters);
}

template <bool VEC, int U>
void launch_m(dim3 grid, const GemmArgs &a, int R, float *work, unsigned *counters, hipStream_t s) {
  switch (a.M) {
    case 1: launch_one<1, VEC, U>(grid, a, R, work, counters, s); break;
    case 2: launch_one<2, VEC, U>(grid, a, R, work, counters, s); break;
    case 3: launch_one<3, VEC, U>(grid, a, R, work, counters, s); break;
    case 4: launch_one<4, VEC, U>(grid, a, R, work, counters, s); break;
    case 5: launch_one<5, VEC, U>(grid, a, R, work, counters, s); break;
    case 6: launch_one<6, VEC, U>(grid, a, R, work, counters, s); break;
    case 7: launch_one<7, VEC, U>(grid, a, R, work, counters, s); break;
    default: launch_one<8, VEC, U>(grid, a, R, work, counters, s); break;
  }
}

}  // namespace

const GemvConfig *gemv_configs(int *count) {
  static const GemvConfig table[] = {
      {"u8_wg512", kWaves, 8, 512},    {"u8_wg1024", kWaves, 8, 1024},
      {"u8_wg2048", kWaves, 8, 2048},  {"u16_wg512", kWaves, 16, 512},
      {"u16_wg1024", kWaves, 16, 1024}, {"u16_wg2048", kWaves, 16, 2048},
      {"u4_wg1024", kWaves, 4, 1024},  {"u4_wg2048", kWaves, 4, 2048},
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

// Workspace the K split may use, per (device, stream).
size_t gemv_work_floats() { return (size_t)4 << 20; }  // 16 MB
int gemv_max_counters() { return 65536; }

hipError_t launch_gemv_with(const GemvConfig &cfg, const GemmArgs &a, float *work,
                            unsigned *counters, hipStream_t s) {
  const bool vec = ((uintptr_t)a.B % 16 == 0) && a.N % 4 == 0 && a.ldb % 4 == 0;
  const int cbw = vec ? 256 : 64;
  const long long cbs = ((long long)a.N + cbw - 1) / cbw;
  if (cbs > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int U = cfg.unroll;
  // Split K so that about target_wgs workgroups run; each split is a
  // multiple of U rows; the workspace and counter limits cap the split.
  long long splits = (cfg.target_wgs + cbs - 1) / cbs;
  const long long max_by_rows = ((long long)a.K + U - 1) / U;
  if (splits > max_by_rows) splits = max_by_rows;
  if (splits > 65535) splits = 65535;
  if (work == nullptr || counters == nullptr || cbs > gemv_max_counters() ||
      splits * a.M * (long long)a.N > (long long)gemv_work_floats())
    splits = 1;
  if (splits < 1) splits = 1;
  long long R = ((a.K + splits - 1) / splits + U - 1) / U * U;
  if (R < U) R = U;
  splits = (a.K + R - 1) / R;
  if (splits < 1) splits = 1;
  const dim3 grid((unsigned)cbs, (unsigned)splits);
  const int Ri = (int)R;
  if (vec) {
    if (U == 4) launch_m<true, 4>(grid, a, Ri, work, counters, s);
    else if (U == 8) launch_m<true, 8>(grid, a, Ri, work, counters, s);
    else launch_m<true, 16>(grid, a, Ri, work, counters, s);
  } else {
    if (U == 4) launch_m<false, 4>(grid, a, Ri, work, counters, s);
    else if (U == 8) launch_m<false, 8>(grid, a, Ri, work, counters, s);
    else launch_m<false, 16>(grid, a, Ri, work, counters, s);
  }
  return hipGetLastError();
}

hipError_t launch_scale(const GemmArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)((a.N + 255) / 256), (unsigned)(a.M < 1024 ? a.M : 1024));
  hipLaunchKernelGGL(scale_kernel, grid, dim3(256), 0, s, a.C, a.M, a.N, a.ldc, a.beta);
  return hipGetLastError();
}

}  // namespace fp32gemm
