// Small-M product Y[M x N] <- alpha X[M x K] W[K x N] + beta Y, 1 <= M <= 32.
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
//    rows per pass of ROWS = NW * RPI * U rows;
//  * passes run two deep: the W values and the X chunk of pass p + 1 are in
//    flight while pass p is multiplied (W in two register sets, X through a
//    double buffer in LDS, read back as float4 over a lane group's U rows).
//    The loop body has no branches: rows past K read zeros through an
//    out-of-range buffer offset, so passes run in whole pairs;
//  * partial sums are added across the lane groups of a wave with a fixed
//    butterfly, then across waves in LDS in wave order: the summation order
//    does not depend on timing, so results are bit-reproducible;
//  * M from 1 to 8 has a kernel per M; M from 9 to 32 (several decode
//    sequences at once) runs on row capacities 12, 16, 24 and 32 with the
//    rows past M masked: no X loads, no stores.  The multiply is then
//    4 MR FMAs per 16 bytes of W, which the vector ALUs still keep up with
//    at N = K = 4096 up to about M = 16.
#include "common.h"

namespace fp32gemm {
namespace {

// Largest lda for op(A) = A^T that keeps a pass's X offsets within 31 bits
// (both GEMV kernels stage at most 2048 values of K at a time).
constexpr int kGemvMaxLdaT = 1 << 17;

template <int MR, bool VEC, int CBW, int NW, int U>
__global__ void __launch_bounds__(NW * 64)
sgemv_kernel(GemmArgs a, int transA) {
  constexpr bool CAP = MR > 8;        // a row capacity: rows m >= M are masked
  constexpr int VW = VEC ? 4 : 1;     // columns per lane
  constexpr int LPR = CBW / VW;       // lanes per row
  constexpr int RPI = 64 / LPR;       // rows per wave instruction
  constexpr int ROWS = NW * RPI * U;  // rows of W per pass
  constexpr int THREADS = NW * 64;
  constexpr int XN = MR * ROWS;                        // X values per pass
  constexpr int XPT = (XN + THREADS - 1) / THREADS;    // staged per thread
  static_assert(64 % LPR == 0 && CBW % VW == 0, "lane mapping");
  static_assert(U % 4 == 0, "X is read back in float4 pieces");
  __shared__ __attribute__((aligned(16))) float xs[2][MR][ROWS];
  __shared__ float red[NW][MR][CBW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane / LPR;           // row group inside the wave
  const int cl = (lane % LPR) * VW;   // first column of this lane in the block

  // Work item (batch entry, column block): workgroups go to the XCDs
  // round-robin by their linear id over the whole grid (XCD = id % 8);
  // items 2j and 2j+1 (the two stripes of a 128-byte line when CBW = 16) go
  // to XCD j % 8, so the line is fetched once into that XCD's L2.  Ids past
  // the last full group of 16 keep their own number.
  const int G = gridDim.x;
  const long long L = (long long)blockIdx.y * G + blockIdx.x;
  const long long T = (long long)gridDim.y * G;
  const long long w = L < (T & ~15LL) ? 2 * (8 * ((L >> 3) >> 1) + (L & 7)) + ((L >> 3) & 1) : L;
  const long long bz = w / G;         // batch entry (0 for a single product)
  const int cb = (int)(w - bz * G);   // column block
  a.A += bz * a.sA;
  a.B += bz * a.sB;
  a.C += bz * a.sC;
  const int n0 = cb * CBW;
  const bool col_ok = n0 + cl < a.N;  // VEC: N % 4 == 0, so the float4 is whole
  const int K = a.K;
  const int wrow = wave * RPI * U;    // first row of this wave in a pass
  const int rl = wrow + g * U;        // first row of this lane in a pass
  // X element (m, k) sits at A + k * xk + m * xm
  const uint32_t xk = transA ? (uint32_t)a.lda : 1u, xm = transA ? 1u : (uint32_t)a.lda;

  // W rows k0 + rl + u of this lane's columns; the wave's first row goes
  // into the buffer base so byte offsets stay small
  auto load_w = [&](float (&w)[U][VW], int k0) {
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.B + (size_t)(k0 + wrow) * a.ldb + n0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = col_ok & (k0 + rl + u < K);  // "&": no short circuit, no branch
      const uint32_t off = ok ? (uint32_t)((g * U + u) * a.ldb + cl) * 4u : kOob;
      if constexpr (VEC) {
        const floatx4 v = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) w[u][e] = v[e];
      } else {
        w[u][0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, off, 0, 0));
      }
    }
  };
  // X of the pass at k0: value i = m * ROWS + kk for i = tid + j * THREADS
  // (consecutive threads read consecutive k of one row of op(A))
  auto load_x = [&](float (&x)[XPT], int k0) {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.A + (size_t)k0 * xk);
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int i = tid + j * THREADS, m = i / ROWS, kk = i % ROWS;
      const bool ok = (i < XN) & (k0 + kk < K) & (!CAP | (m < a.M));
      const uint32_t off = ok ? ((uint32_t)kk * xk + (uint32_t)m * xm) * 4u : kOob;
      x[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, off, 0, 0));
    }
  };
  auto store_x = [&](const float (&x)[XPT], int buf) {
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int i = tid + j * THREADS;
      if (XN % THREADS == 0 || i < XN) (&xs[buf][0][0])[i] = x[j];
    }
  };

  float acc[MR][VW];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int e = 0; e < VW; ++e) acc[m][e] = 0.0f;
  auto multiply = [&](const float (&w)[U][VW], int buf) {
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int q = 0; q < U / 4; ++q) {
        const floatx4 xv = *reinterpret_cast<const floatx4 *>(&xs[buf][m][rl + 4 * q]);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int e = 0; e < VW; ++e) acc[m][e] += xv[t] * w[4 * q + t][e];
      }
  };

  float wa[U][VW], wb[U][VW];
  float xr[XPT];
  load_x(xr, 0);
  load_w(wa, 0);
  store_x(xr, 0);
  __syncthreads();
  // the scheduling barriers keep each prefetch ahead of the multiply that
  // waits on the previous pass
  for (int k0 = 0; k0 < K; k0 += 2 * ROWS) {
    load_x(xr, k0 + ROWS);
    load_w(wb, k0 + ROWS);
    __builtin_amdgcn_sched_barrier(0);
    multiply(wa, 0);
    store_x(xr, 1);
    __syncthreads();
    load_x(xr, k0 + 2 * ROWS);
    load_w(wa, k0 + 2 * ROWS);
    __builtin_amdgcn_sched_barrier(0);
    multiply(wb, 1);
    store_x(xr, 0);
    __syncthreads();
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
    if (n0 + c >= a.N || (CAP && m >= a.M)) continue;
    float s = red[0][m][c];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) s += red[w2][m][c];
    float *y = a.C + (size_t)m * a.ldc + n0 + c;
    float out = alpha * s;
    if (beta != 0.0f) out += beta * *y;
    if (a.bias) out += a.bias[n0 + c];
    *y = apply_act(out, a.act);
  }
}

// ---------------------------------------------------------------------------
// Small-M product with the weight stored transposed: op(B) = B^T, B stored
// N x K (the usual layout of a linear layer's weight, y = x W^T).  Output
// (m, n) is the dot product of row m of op(A) with row n of the stored B, a
// contiguous run of K floats, so the weight streams with 1 KB wave
// instructions (64 lanes x 16 bytes) and none of the column-stripe pattern of
// the other layout.  Each wave owns RW consecutive rows of B and walks K in
// chunks of CH floats, two chunks deep: the weights and the X values of chunk
// c + 1 are in flight while chunk c is multiplied (X through a double buffer
// in LDS, weights in two register sets).  The loop body has no branches:
// loads past K (or past N) take an out-of-range buffer offset and read zeros,
// so a pair of chunks always runs whole and the over-fetch adds exact zeros.
// Partial dot products stay in registers and are added across the wave with
// a fixed butterfly, so the result does not depend on timing.
// ---------------------------------------------------------------------------
constexpr int kRowsWaves = 4;
constexpr int kRowsThreads = kRowsWaves * 64;

template <int MR, bool VEC, int RW, int LPR, int CH, bool XV>
__global__ void __launch_bounds__(kRowsThreads)
sgemv_rows_kernel(GemmArgs a, int transA) {
  constexpr int VW = VEC ? 4 : 1;            // weight floats per lane per position
  constexpr int RPI = 64 / LPR;              // rows per wave instruction
  constexpr int STEP = LPR * VW;             // k covered by one lane group per instruction
  constexpr int POS = CH / STEP;             // positions per chunk
  constexpr int XN = MR * CH;                // X values staged per chunk
  constexpr int XW = XV ? 4 : 1;             // X values per staging load
  constexpr int XPT = (XN / XW + kRowsThreads - 1) / kRowsThreads;  // staging loads per thread
  static_assert(64 % LPR == 0 && CH % STEP == 0 && MR * RW <= LPR, "row-dot lane mapping");
  __shared__ __attribute__((aligned(16))) float xs[2][MR * CH];

  // batch entry (strided batches; 0 for a single product)
  const long long bz = blockIdx.y;
  a.A += bz * a.sA;
  a.B += bz * a.sB;
  a.C += bz * a.sC;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = lane / LPR, li = lane % LPR;  // row slot of the instruction; lane in it
  // this wave owns rows nw + r * RPI + slot, r < RW
  const int nw = (blockIdx.x * kRowsWaves + wave) * RPI * RW;
  const int K = a.K;
  // X element (m, k0 + kk) sits at A + k0 * xk + kk * xk + m * xm
  const uint32_t xk = transA ? (uint32_t)a.lda : 1u, xm = transA ? 1u : (uint32_t)a.lda;

  // one buffer base per wave (at its first row); each lane group's row goes
  // into the offset
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.B + (nw < a.N ? (size_t)nw * a.ldb : 0));
  bool live[RW];
  uint32_t rowoff[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    live[r] = nw + r * RPI + slot < a.N;
    rowoff[r] = (uint32_t)(r * RPI + slot) * (uint32_t)a.ldb * 4u;
  }

  // weights of the chunk at k0: RW rows x POS positions, zeros past K or N
  auto load_w = [&](float (&w)[RW][POS][VW], int k0) {
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int p = 0; p < POS; ++p) {
        const int k = k0 + p * STEP + li * VW;
        const uint32_t off = (live[r] & (k < K)) ? rowoff[r] + (uint32_t)k * 4u : kOob;
        if constexpr (VEC) {
          const floatx4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) w[r][p][e] = v[e];
        } else {
          w[r][p][0] =
              __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
        }
      }
  };
  // X of the chunk at k0, elements i .. i + XW - 1 = m * CH + kk .. with
  // i = XW * (tid + j * threads) (consecutive lanes read consecutive k),
  // zeros past K.  XV: op(A) = A with 16-byte aligned rows and K % 4 == 0,
  // so each float4 is all inside or all outside K.
  auto load_x = [&](floatx4 (&x)[XPT], int k0) {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.A + (size_t)k0 * xk);
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int i = XW * (tid + j * kRowsThreads), m = i / CH, kk = i % CH;
      const bool ok = ((XN % (XW * kRowsThreads) == 0) | (i < XN)) & (k0 + kk < K);
      const uint32_t off = ok ? ((uint32_t)kk * xk + (uint32_t)m * xm) * 4u : kOob;
      if constexpr (XV)
        x[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
      else
        x[j][0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, off, 0, 0));
    }
  };
  auto store_x = [&](const floatx4 (&x)[XPT], int buf) {
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int i = XW * (tid + j * kRowsThreads);
      if (XN % (XW * kRowsThreads) == 0 || i < XN) {
        if constexpr (XV)
          *reinterpret_cast<floatx4 *>(&xs[buf][i]) = x[j];
        else
          xs[buf][i] = x[j][0];
      }
    }
  };

  float acc[MR][RW];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int r = 0; r < RW; ++r) acc[m][r] = 0.0f;
  auto multiply = [&](const float (&w)[RW][POS][VW], int buf) {
#pragma unroll
    for (int p = 0; p < POS; ++p) {
      const int k = p * STEP + li * VW;
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        float x[VW];
        if constexpr (VEC) {
          const floatx4 v = *reinterpret_cast<const floatx4 *>(&xs[buf][m * CH + k]);
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = v[e];
        } else {
          x[0] = xs[buf][m * CH + k];
        }
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
          for (int e = 0; e < VW; ++e) acc[m][r] += x[e] * w[r][p][e];
      }
    }
  };

  const int nc = (K + CH - 1) / CH;
  float wa[RW][POS][VW], wb[RW][POS][VW];
  floatx4 xr[XPT];
  load_x(xr, 0);
  load_w(wa, 0);
  store_x(xr, 0);
  __syncthreads();
  // the scheduling barriers keep each prefetch ahead of the multiply that
  // waits on the previous chunk (left alone, the scheduler interleaves them
  // and the waits then cover the prefetch too)
  for (int c = 0; c < nc; c += 2) {
    load_x(xr, (c + 1) * CH);
    load_w(wb, (c + 1) * CH);
    __builtin_amdgcn_sched_barrier(0);
    multiply(wa, 0);
    store_x(xr, 1);
    __syncthreads();
    load_x(xr, (c + 2) * CH);
    load_w(wa, (c + 2) * CH);
    __builtin_amdgcn_sched_barrier(0);
    multiply(wb, 1);
    store_x(xr, 0);
    __syncthreads();
  }

  // butterfly over the LPR lanes of each row slot; lane li = m * RW + r of
  // the slot then writes output (m, row nw + r * RPI + slot)
#pragma unroll
  for (int sh = 1; sh < LPR; sh <<= 1)
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int r = 0; r < RW; ++r) acc[m][r] += __shfl_xor(acc[m][r], sh, 64);
  float sum = 0.0f;
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int r = 0; r < RW; ++r)
      if (li == m * RW + r) sum = acc[m][r];
  const int m = li / RW, n = nw + (li % RW) * RPI + slot;
  if (li < MR * RW && n < a.N) {
    float *y = a.C + (size_t)m * a.ldc + n;
    float out = a.alpha * sum;
    if (a.beta != 0.0f) out += a.beta * *y;
    if (a.bias) out += a.bias[n];
    *y = apply_act(out, a.act);
  }
}

template <bool VEC, int RW, int LPR, int CH_SHORT, bool XV>
hipError_t launch_rows_rw(const GemmArgs &a, int transA, hipStream_t s) {
  constexpr int RPW = (64 / LPR) * RW;  // rows per wave
  const long long wgs = ((long long)a.N + kRowsWaves * RPW - 1) / (kRowsWaves * RPW);
  if (wgs > 0x7fffffffLL || a.batch > 65535) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)wgs, (unsigned)a.batch), block(kRowsThreads);
  // K chunk: 1024 (512 for M > 4) with whole-wave rows, CH_SHORT with short rows
  switch (a.M) {
#define FP32GEMM_ROWS_CASE(MR)                                                                 \
  case MR:                                                                                     \
    hipLaunchKernelGGL((sgemv_rows_kernel<MR, VEC, RW, LPR,                                    \
                                          LPR == 64 ? (MR <= 4 ? 1024 : 512) : CH_SHORT, XV>), \
                       grid, block, 0, s, a, transA);                                          \
    break;
    FP32GEMM_ROWS_CASE(1)
    FP32GEMM_ROWS_CASE(2)
    FP32GEMM_ROWS_CASE(3)
    FP32GEMM_ROWS_CASE(4)
    FP32GEMM_ROWS_CASE(5)
    FP32GEMM_ROWS_CASE(6)
    FP32GEMM_ROWS_CASE(7)
    FP32GEMM_ROWS_CASE(8)
#undef FP32GEMM_ROWS_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool gemv_supported(const GemmArgs &a, int transA) {
  return a.M >= 1 && a.M <= 8 && (!transA || a.lda <= kGemvMaxLdaT);
}

bool gemv_wide_supported(const GemmArgs &a, int transA) {
  return a.M > 8 && a.M <= kGemvMaxRows && (!transA || a.lda <= kGemvMaxLdaT);
}

int gemv_row_capacity(int M) {
  return M <= 8 ? M : M <= 12 ? 12 : M <= 16 ? 16 : M <= 24 ? 24 : M <= 32 ? 32 : 0;
}

bool gemv_config_runs(const GemvConfig &c, int M) { return M >= 1 && M <= c.max_rows; }

// Rows per wave: one for M <= 3 (the most waves, which keeps the most loads
// in flight), two from M = 4 on (each staged X value then feeds two rows).
// Short rows share a wave instruction, 16 lanes (64 floats per instruction)
// to a row, with K chunks of 256: a whole wave per row leaves most lanes and
// most of each chunk masked at small K (K = 128: 57.7 against 15.0 us for
// 64 MB of weights).  Timing both variants over K from 256 to 2048 put the
// switch at K = 1024 (M <= 3: whole waves from 1024 on; M >= 4: from 2048).
hipError_t launch_gemv_rows(const GemmArgs &a, int transA, int rows_per_wave, hipStream_t s) {
  if (!gemv_supported(a, transA)) return hipErrorInvalidValue;
  const bool vec = ((uintptr_t)a.B % 16 == 0) && a.K % 4 == 0 && a.ldb % 4 == 0;
  // X staged with float4 loads when op(A) = A has 16-byte aligned rows
  const bool xv = vec && !transA && (uintptr_t)a.A % 16 == 0 && a.lda % 4 == 0;
  const int rw = rows_per_wave > 0 ? rows_per_wave : a.M >= 4 ? 2 : 1;
  const bool short_rows = a.K < 1024 || (a.M >= 4 && a.K == 1024);
  if (xv) {
    if (short_rows)
      return rw >= 2 ? launch_rows_rw<true, 2, 16, 256, true>(a, transA, s)
                     : launch_rows_rw<true, 1, 16, 256, true>(a, transA, s);
    return rw >= 2 ? launch_rows_rw<true, 2, 64, 0, true>(a, transA, s)
                   : launch_rows_rw<true, 1, 64, 0, true>(a, transA, s);
  }
  if (short_rows) {
    if (vec) return rw >= 2 ? launch_rows_rw<true, 2, 16, 256, false>(a, transA, s)
                            : launch_rows_rw<true, 1, 16, 256, false>(a, transA, s);
    return rw >= 2 ? launch_rows_rw<false, 2, 16, 256, false>(a, transA, s)
                   : launch_rows_rw<false, 1, 16, 256, false>(a, transA, s);
  }
  if (vec) return rw >= 2 ? launch_rows_rw<true, 2, 64, 0, false>(a, transA, s)
                          : launch_rows_rw<true, 1, 64, 0, false>(a, transA, s);
  return rw >= 2 ? launch_rows_rw<false, 2, 64, 0, false>(a, transA, s)
                 : launch_rows_rw<false, 1, 64, 0, false>(a, transA, s);
}

namespace {

// C <- beta * C for every batch entry (blockIdx.z); beta == 0 stores zeros
// without reading C.
__global__ void __launch_bounds__(256)
scale_kernel(float *C, int M, int N, int ldc, long long sC, float beta, const float *bias,
             int act) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= N) return;
  float *Cz = C + (long long)blockIdx.z * sC;
  const float bj = bias ? bias[j] : 0.0f;
  for (int i = blockIdx.y; i < M; i += gridDim.y) {
    float *p = Cz + (size_t)i * ldc + j;
    float v = (beta == 0.0f) ? 0.0f : beta * *p;
    if (bias) v += bj;
    *p = apply_act(v, act);
  }
}

// Configurations that also run M = 9..32 (row capacities): four rows of W per
// lane and at most 8 waves; the others spill their registers at 16+ rows.
template <int NW, int U>
constexpr bool kGemvWide = U == 4 && NW <= 8;

template <bool VEC, int CBW, int NW, int U>
hipError_t launch_cfg(const GemmArgs &a, int transA, hipStream_t s) {
  const long long blocks = ((long long)a.N + CBW - 1) / CBW;
  if (blocks > 0x7fffffffLL || a.batch > 65535) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks, (unsigned)a.batch), block(NW * 64);
  switch (a.M) {
#define FP32GEMM_GEMV_CASE(MR)                                                                   \
  case MR:                                                                                       \
    hipLaunchKernelGGL((sgemv_kernel<MR, VEC, CBW, NW, U>), grid, block, 0, s, a, transA); break;
    FP32GEMM_GEMV_CASE(1)
    FP32GEMM_GEMV_CASE(2)
    FP32GEMM_GEMV_CASE(3)
    FP32GEMM_GEMV_CASE(4)
    FP32GEMM_GEMV_CASE(5)
    FP32GEMM_GEMV_CASE(6)
    FP32GEMM_GEMV_CASE(7)
    FP32GEMM_GEMV_CASE(8)
    default:
      if constexpr (kGemvWide<NW, U>) {
        const int cap = gemv_row_capacity(a.M);
        switch (cap) {
          FP32GEMM_GEMV_CASE(12)
          FP32GEMM_GEMV_CASE(16)
          FP32GEMM_GEMV_CASE(24)
          FP32GEMM_GEMV_CASE(32)
          default: return hipErrorInvalidValue;
        }
        break;
      } else {
        return hipErrorInvalidValue;
      }
#undef FP32GEMM_GEMV_CASE
  }
  return hipGetLastError();
}

// 128-bit loads of W need B 16-byte aligned and N, ldb multiples of 4.
template <int CBW, int NW, int U>
hipError_t launch_gemv(const GemmArgs &a, int transA, hipStream_t s) {
  if (!gemv_supported(a, transA) && !(kGemvWide<NW, U> && gemv_wide_supported(a, transA)))
    return hipErrorInvalidValue;
  const bool vec = ((uintptr_t)a.B % 16 == 0) && a.N % 4 == 0 && a.ldb % 4 == 0;
  return vec ? launch_cfg<true, CBW, NW, U>(a, transA, s)
             : launch_cfg<false, CBW, NW, U>(a, transA, s);
}

}  // namespace

const GemvConfig *gemv_configs(int *count) {
  static const GemvConfig table[] = {
      {"c16_w8_u8", 16, 8, 8, 8, &launch_gemv<16, 8, 8>},
      {"c16_w8_u4", 16, 8, 4, kGemvMaxRows, &launch_gemv<16, 8, 4>},
      {"c16_w16_u4", 16, 16, 4, 8, &launch_gemv<16, 16, 4>},
      {"c16_w4_u8", 16, 4, 8, 8, &launch_gemv<16, 4, 8>},
      {"c16_w4_u16", 16, 4, 16, 8, &launch_gemv<16, 4, 16>},
      {"c32_w8_u4", 32, 8, 4, kGemvMaxRows, &launch_gemv<32, 8, 4>},
      {"c32_w8_u8", 32, 8, 8, 8, &launch_gemv<32, 8, 8>},
      {"c64_w8_u4", 64, 8, 4, kGemvMaxRows, &launch_gemv<64, 8, 4>},
      {"mfma16_w8", 16, 8, 0, 128, &launch_skinny16},
      {"mfma32_w8", 32, 8, 0, 128, &launch_skinny32},
      {"mfma64_w8", 64, 8, 0, 64, &launch_skinny64},
      {"split256_w4_u4", 256, 4, 4, 8, &launch_gemv_split4},
      {"split256_w4_u4_serial", 256, 4, 4, 8, &launch_gemv_split4_serial},
      {"split256_w8_u4", 256, 8, 4, 8, &launch_gemv_split8},
      {"split256_w8_u4_serial", 256, 8, 4, 8, &launch_gemv_split8_serial},
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

hipError_t launch_scale(const GemmArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)((a.N + 255) / 256), (unsigned)(a.M < 1024 ? a.M : 1024),
                  (unsigned)a.batch);
  hipLaunchKernelGGL(scale_kernel, grid, dim3(256), 0, s, a.C, a.M, a.N, a.ldc, a.sC, a.beta,
                     a.bias, a.act);
  return hipGetLastError();
}

}  // namespace fp32gemm
