// Matrix-core issue probe (measurement only; built into libmfmaprobe.so, not
// part of the GEMM library's ABI).
//
// The SGEMM kernels are bound by the fp32 matrix cores.  This kernel does
// nothing else: every wave issues `iters` x 32 independent MFMAs back to back
// (8 accumulator blocks of v_mfma_f32_32x32x2_f32, or 16 of
// v_mfma_f32_16x16x4_f32 four times as often), with no memory access and no
// barrier inside the loop.  Its rate is what the matrix cores deliver on this
// GPU at the clock they run at under that load, the ceiling a GEMM's inner
// loop can approach.  Each workgroup's thread 0 records the shader clock
// (s_memtime) and the 100 MHz wall clock (s_memrealtime) around its loop, so
// the clock under load is read from the kernel itself.
#include <hip/hip_runtime.h>

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <int MF>
__global__ void __launch_bounds__(512) mfma_issue(float *sink, unsigned long long *clocks,
                                                  int iters, float seed) {
  // distinct operand values per lane; the sums only keep the work alive
  const float a = seed + threadIdx.x * 1e-7f, b = seed - threadIdx.x * 1e-7f;
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long w0 = __builtin_amdgcn_s_memrealtime();
  float sum = 0.0f;
  if constexpr (MF == 32) {
    floatx16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = floatx16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[i], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) sum += acc[i][0] + acc[i][15];
  } else {
    floatx4 acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = floatx4{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[i], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += acc[i][0] + acc[i][3];
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long w1 = __builtin_amdgcn_s_memrealtime();
  sink[blockIdx.x * blockDim.x + threadIdx.x] = sum;
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = c1 - c0;
    clocks[2 * blockIdx.x + 1] = w1 - w0;
  }
}

}  // namespace

// `groups` workgroups of `waves` x 64 threads (waves 4 or 8: one or two per
// SIMD), each wave issuing iters x 32 MFMAs of the 32x32x2 (mf = 32) or
// iters x 64 of the 16x16x4 (mf = 16) form: 131,072 x iters FLOP per wave
// either way.  sink: groups x waves x 64 floats written; clocks: 2 x groups
// values written (shader clock cycles, then 10 ns wall-clock ticks, of the
// loop of each workgroup's first wave).  Returns 0, -1 for arguments the
// kernel does not take, or a positive hipError_t.
extern "C" __attribute__((visibility("default")))
int mfma_issue_rate(int mf, int groups, int waves, int iters, float *sink,
                    unsigned long long *clocks, hipStream_t s) {
  if ((mf != 32 && mf != 16) || (waves != 4 && waves != 8) || groups < 1 || iters < 1 ||
      sink == nullptr || clocks == nullptr)
    return -1;
  if (mf == 32)
    hipLaunchKernelGGL(mfma_issue<32>, dim3(groups), dim3(waves * 64), 0, s, sink, clocks, iters,
                       0.5f);
  else
    hipLaunchKernelGGL(mfma_issue<16>, dim3(groups), dim3(waves * 64), 0, s, sink, clocks, iters,
                       0.5f);
  return (int)hipGetLastError();
}
