// Small-M product Y[M x N] <- alpha X[M x K] W[K x N] + beta Y, 1 <= M <= 8.
//
// This is the decode-phase shape of "GPU GEMM 优化完全拆解（一）", section
// "LLM 推理本质上是 GEMM 的串联": M is the batch, and the time is the time to
// stream W once from HBM.  The pages give no kernel for it; the design keeps
// their coalescing rule ("GPU 基础原理", section "4.3 合并加载"), 128-bit
// loads ("CUDA 矩阵乘法优化", section "7. Kernel 6") and a K split with a
// reduction step ("10. cuBLAS 领先的性能差异"), but the reduction never
// leaves the workgroup:
//
//  * a workgroup owns CBW columns of W over the whole of K, so it needs no
//    other workgroup's partial sums (a cross-workgroup reduction would need
//    an agent-scope release/acquire, which on this GPU writes back and
//    invalidates the XCD's whole L2 per workgroup);
//  * with CBW = 16 and N = 4096 that is 256 workgroups, one per CU; each row
//    segment is 64 bytes.  The two column blocks that share a 128-byte line
//    run on the same XCD (so the line is fetched once into that L2), and the
//    line pairs an XCD owns are spread across the row: a workgroup's stream
//    of rows keeps one address offset modulo the row stride, and with a
//    power-of-two stride (N = 4096: 16 KB) a contiguous window of columns
//    per XCD concentrates its traffic on few memory channels;
//  * lanes are grouped LPR to a row (one float4 each); a wave instruction
//    reads RPI = 64 / LPR rows; lane group g of wave w takes U consecutive
//    rows per pass, so its X values are U consecutive floats per batch row;
//  * every lane keeps U loads of W in flight and M x 4 fp32 accumulators;
//  * partial sums are added across the lane groups of a wave with a fixed
//    butterfly, then across waves in LDS in wave order: the summation order
//    does not depend on timing, so results are bit-reproducible.
#include "common.h"

namespace fp32gemm {
namespace {

template <int MR, bool VEC, bool XVEC, int CBW, int NW, int U>
__global__ void __launch_bounds__(NW * 64)
sgemv_kernel(GemmArgs a) {
  constexpr int VW = VEC ? 4 : 1;     // columns per lane
  constexpr int LPR = CBW / VW;       // lanes per row
  constexpr int RPI = 64 / LPR;       // rows per wave instruction
  constexpr int ROWS = NW * RPI * U;  // rows per workgroup pass
  static_assert(64 % LPR == 0 && CBW % VW == 0, "lane mapping");
  static_assert(!XVEC || U % 4 == 0, "X is read in float4 pieces");
  __shared__ float red[NW][MR][CBW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane / LPR;           // row group inside the wave
  const int cl = (lane % LPR) * VW;   // first column of this lane in the block

  // Column block: workgroups go to the XCDs round-robin by id (XCD = id % 8);
  // blocks 2j and 2j+1 go to XCD j % 8.  Ids past the last full group of 16
  // keep their own number.
  const int G = gridDim.x, bid = blockIdx.x;
  const int cb = bid < (G & ~15)
                     ? 2 * (8 * ((bid >> 3) >> 1) + (bid & 7)) + ((bid >> 3) & 1)
                     : bid;
  const int n0 = cb * CBW;
  const bool col_ok = n0 + cl < a.N;  // VEC: N % 4 == 0, so the float4 is whole

  float acc[MR][VW];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int e = 0; e < VW; ++e) acc[m][e] = 0.0f;

  const int ldb = a.ldb, lda = a.lda;
  for (int k0 = 0; k0 < a.K; k0 += ROWS) {
    // this lane's rows: k0 + wave * RPI * U + g * U + u, u < U.  The wave's
    // first row goes into the buffer base so byte offsets stay below 2^31.
    const int kw = k0 + wave * RPI * U;
    const int r0 = g * U;
    const int nrows = a.K - kw - r0;  // rows of this lane still inside K
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.B + (size_t)kw * ldb + n0);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.A + kw);
    float w[U][VW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = col_ok && u < nrows;
      const uint32_t off = ok ? (uint32_t)((r0 + u) * ldb + cl) * 4u : kOob;
      if constexpr (VEC) {
        const floatx4 v = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) w[u][e] = v[e];
      } else {
        w[u][0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, off, 0, 0));
      }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float x[U];
      if constexpr (XVEC) {
        // rows kw + r0 + u start on a multiple of 4 and K % 4 == 0, so each
        // float4 of X is entirely inside or entirely outside K
#pragma unroll
        for (int q = 0; q < U / 4; ++q) {
          const uint32_t off = 4 * q < nrows ? (uint32_t)(m * lda + r0 + 4 * q) * 4u : kOob;
          const floatx4 v = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) x[4 * q + e] = v[e];
        }
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t off = u < nrows ? (uint32_t)(m * lda + r0 + u) * 4u : kOob;
          x[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, off, 0, 0));
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < VW; ++e) acc[m][e] += x[u] * w[u][e];
    }
  }

  // Butterfly over the row groups of the wave (lane bits above the column bits).
#pragma unroll
  for (int s = LPR; s < 64; s <<= 1)
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int e = 0; e < VW; ++e) acc[m][e] += __shfl_xor(acc[m][e], s, 64);
  if (g == 0) {
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int e = 0; e < VW; ++e) red[wave][m][cl + e] = acc[m][e];
  }
  __syncthreads();

  // Waves in wave order, then the alpha/beta update.
  const float alpha = a.alpha, beta = a.beta;
  for (int o = tid; o < MR * CBW; o += NW * 64) {
    const int m = o / CBW, c = o % CBW;
    if (n0 + c >= a.N) continue;
    float s = red[0][m][c];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) s += red[w2][m][c];
    float *y = a.C + (size_t)m * a.ldc + n0 + c;
    float out = alpha * s;
    if (beta != 0.0f) out += beta * *y;
    *y = out;
  }
}

// C <- beta * C for every batch entry (blockIdx.z); beta == 0 stores zeros
// without reading C.
__global__ void __launch_bounds__(256)
scale_kernel(float *C, int M, int N, int ldc, long long sC, float beta) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= N) return;
  float *Cz = C + (long long)blockIdx.z * sC;
  for (int i = blockIdx.y; i < M; i += gridDim.y) {
    float *p = Cz + (size_t)i * ldc + j;
    *p = (beta == 0.0f) ? 0.0f : beta * *p;
  }
}

template <bool VEC, bool XVEC, int CBW, int NW, int U>
hipError_t launch_cfg(const GemmArgs &a, hipStream_t s) {
  const long long blocks = ((long long)a.N + CBW - 1) / CBW;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks), block(NW * 64);
  switch (a.M) {
#define FP32GEMM_GEMV_CASE(MR)                                                                  \
  case MR:                                                                                      \
    hipLaunchKernelGGL((sgemv_kernel<MR, VEC, XVEC, CBW, NW, U>), grid, block, 0, s, a); break;
    FP32GEMM_GEMV_CASE(1)
    FP32GEMM_GEMV_CASE(2)
    FP32GEMM_GEMV_CASE(3)
    FP32GEMM_GEMV_CASE(4)
    FP32GEMM_GEMV_CASE(5)
    FP32GEMM_GEMV_CASE(6)
    FP32GEMM_GEMV_CASE(7)
    FP32GEMM_GEMV_CASE(8)
#undef FP32GEMM_GEMV_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// 128-bit loads of W need B 16-byte aligned and N, ldb multiples of 4; of X,
// A 16-byte aligned and K, lda multiples of 4.
template <int CBW, int NW, int U>
hipError_t launch_gemv(const GemmArgs &a, hipStream_t s) {
  const bool vec = ((uintptr_t)a.B % 16 == 0) && a.N % 4 == 0 && a.ldb % 4 == 0;
  const bool xvec = ((uintptr_t)a.A % 16 == 0) && a.K % 4 == 0 && a.lda % 4 == 0;
  if (vec)
    return xvec ? launch_cfg<true, true, CBW, NW, U>(a, s) : launch_cfg<true, false, CBW, NW, U>(a, s);
  return xvec ? launch_cfg<false, true, CBW, NW, U>(a, s) : launch_cfg<false, false, CBW, NW, U>(a, s);
}

}  // namespace

const GemvConfig *gemv_configs(int *count) {
  static const GemvConfig table[] = {
      {"c16_w8_u8", 16, 8, 8, &launch_gemv<16, 8, 8>},
      {"c16_w8_u4", 16, 8, 4, &launch_gemv<16, 8, 4>},
      {"c16_w16_u4", 16, 16, 4, &launch_gemv<16, 16, 4>},
      {"c16_w4_u8", 16, 4, 8, &launch_gemv<16, 4, 8>},
      {"c16_w8_u16", 16, 8, 16, &launch_gemv<16, 8, 16>},
      {"c16_w16_u8", 16, 16, 8, &launch_gemv<16, 16, 8>},
      {"c32_w8_u8", 32, 8, 8, &launch_gemv<32, 8, 8>},
      {"c64_w16_u8", 64, 16, 8, &launch_gemv<64, 16, 8>},
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

hipError_t launch_scale(const GemmArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)((a.N + 255) / 256), (unsigned)(a.M < 1024 ? a.M : 1024),
                  (unsigned)a.batch);
  hipLaunchKernelGGL(scale_kernel, grid, dim3(256), 0, s, a.C, a.M, a.N, a.ldc, a.sC, a.beta);
  return hipGetLastError();
}

}  // namespace fp32gemm
