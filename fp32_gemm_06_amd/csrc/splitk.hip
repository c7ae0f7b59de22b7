// Split-K across workgroups: C <- alpha * A B + beta * C computed as `splits`
// partial products over consecutive K chunks, then added in a fixed order.
//
// This is the K split the pages credit for part of the vendor library's lead
// on grids that leave SMs idle ("CUDA 矩阵乘法优化", section "10. cuBLAS 领先
// 的性能差异").  On MI355X it pays for shapes whose C has few tiles but whose
// K is long: the partial products multiply the number of workgroups, and the
// extra traffic (each partial is written once and read once) is small next to
// the K loop.  The cross-workgroup reduction is a second kernel, so that
// phase 1 is the batched tiled kernel unchanged for every tile shape and
// layout, and its fixed summation order keeps results bit-reproducible.  The
// in-kernel form, where the last workgroup of a tile adds the others' partial
// tiles, is stream-K (streamk.hip).
//
// Phase 1 is the tiled kernel launched as a batch: entry s reads A and B
// offset to chunk s and writes its raw sum to workspace plane s (packed
// M x N).  Phase 2 (below) adds the planes in ascending s and applies alpha
// and beta, with 128-bit accesses when the rows allow them.
#include <math.h>

#include "common.h"

namespace fp32gemm {
namespace {

constexpr int kChunkAlign = 32;  // chunks are whole K slices of every tile shape

template <bool VEC>
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float *ws, int splits, int M, int N, float alpha, float beta, float *C,
                     int ldc) {
  const long long plane = (long long)M * N;
  const int per_row = VEC ? N / 4 : N;
  const long long total = (long long)M * per_row;
  const long long stride = (long long)gridDim.x * 256;
  for (long long t = (long long)blockIdx.x * 256 + threadIdx.x; t < total; t += stride) {
    const int i = (int)(t / per_row), jj = (int)(t - (long long)i * per_row);
    if constexpr (VEC) {
      const float *p = ws + (long long)i * N + 4 * jj;
      floatx4 sum = *reinterpret_cast<const floatx4 *>(p);
      for (int q = 1; q < splits; ++q) sum += *reinterpret_cast<const floatx4 *>(p + q * plane);
      floatx4 *c = reinterpret_cast<floatx4 *>(C + (long long)i * ldc + 4 * jj);
      floatx4 out = alpha * sum;
      if (beta != 0.0f) out += beta * *c;
      *c = out;
    } else {
      const float *p = ws + (long long)i * N + jj;
      float sum = *p;
      for (int q = 1; q < splits; ++q) sum += p[q * plane];
      float *c = C + (long long)i * ldc + jj;
      float out = alpha * sum;
      if (beta != 0.0f) out += beta * *c;
      *c = out;
    }
  }
}

}  // namespace

int splitk_chunk(int K, int splits, int *kc) {
  if (splits < 1) splits = 1;
  long long c = ((long long)K + splits - 1) / splits;
  c = (c + kChunkAlign - 1) / kChunkAlign * kChunkAlign;
  if (c < kChunkAlign) c = kChunkAlign;
  *kc = (int)c;
  return (int)(((long long)K + c - 1) / c);
}

// Splits for the automatic choice: the tiled-kernel model (dispatch.hip) for a
// grid of `chunks` products, plus the reduction's traffic at an effective
// 5 TB/s and 3 us for the second launch; chunks of at least 256 values of K.
int splitk_pick(int M, int N, int K) {
  static const int cand[] = {1, 2, 3, 4, 6, 8, 12, 16, 24, 32};
  const double flops = 2.0 * M * N * (double)K;
  int best = 1;
  double best_t = -1.0;
  for (int s : cand) {
    int kc = 0;
    const int chunks = splitk_chunk(K, s, &kc);
    if (chunks > 1 && kc < 256) break;
    double rate = 0.0;
    model_gemm_config(M, N, kc, chunks, &rate);
    double t = flops / (rate * 1e12);
    if (chunks > 1) t += (2.0 * chunks + 2.0) * M * (double)N * 4.0 / 5e12 + 3e-6;
    if (best_t < 0.0 || t < best_t) {
      best_t = t;
      best = chunks;
    }
  }
  return best;
}

hipError_t launch_splitk_reduce(const float *ws, int splits, int M, int N, float alpha, float beta,
                                float *C, int ldc, hipStream_t s) {
  const bool vec = N % 4 == 0 && ldc % 4 == 0 && (uintptr_t)C % 16 == 0 && (uintptr_t)ws % 16 == 0;
  const long long total = (long long)M * (vec ? N / 4 : N);
  long long blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  if (vec)
    hipLaunchKernelGGL(splitk_reduce_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, ws, splits,
                       M, N, alpha, beta, C, ldc);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, ws,
                       splits, M, N, alpha, beta, C, ldc);
  return hipGetLastError();
}

}  // namespace fp32gemm
