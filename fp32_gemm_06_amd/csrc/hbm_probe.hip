// HBM streaming probe (measurement only; built into libhbmprobe.so, not part
// of the GEMM library's ABI).
//
// The decode kernels are bound by one pass over the weights.  This kernel
// does only that pass: workgroup g reads its own contiguous `per` floats of
// `src` with 128-bit buffer loads, U loads per lane per step and D steps in
// flight, and keeps a running sum so the loads cannot be dropped.  Its time
// for the same bytes and launch shape as a GEMV kernel is the ceiling that
// kernel's loads can reach on this GPU.  With `stamps`, each workgroup also
// records the wall clock (s_memrealtime, 100 MHz) when it starts and when its
// loads have all returned, which shows the dispatch ramp and the drain.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kOob = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7ffffff0,
                                           0x00020000);
}

template <int NW, int U, int D>
__global__ void __launch_bounds__(NW * 64)
stream_read(const float *src, long long per, float *sink, unsigned long long *stamps) {
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  constexpr int STEP = NW * 64 * 4;  // floats one load instruction covers over the workgroup
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rs = rsrc(src + (long long)blockIdx.x * per);
  const int nload = (int)(per / STEP);  // per is a multiple of STEP (checked on the host)
  auto load = [&](floatx4 (&r)[U], int step) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = step * U + u;
      const uint32_t off = k < nload ? (uint32_t)(k * STEP + tid * 4) * 4u : kOob;
      r[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    }
  };
  floatx4 v[D][U];
#pragma unroll
  for (int d = 0; d < D; ++d) load(v[d], d);
  float acc = 0.0f;
  for (int st = 0; st * U < nload; st += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
#pragma unroll
      for (int u = 0; u < U; ++u) acc += (v[d][u][0] + v[d][u][1]) + (v[d][u][2] + v[d][u][3]);
      __builtin_amdgcn_sched_barrier(0);
      load(v[d], st + d + D);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  sink[(long long)blockIdx.x * NW * 64 + tid] = acc;
  if (stamps != nullptr && tid == 0) {
    stamps[2 * blockIdx.x] = t0;
    stamps[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
  }
}

}  // namespace

// Reads n floats of src as `groups` contiguous pieces, one per workgroup of
// `waves` x 64 threads (waves 4 or 8; 4 float4 loads per lane per step, 2
// steps in flight).  n must split into pieces of a whole number of steps
// (n % (groups * waves * 256) == 0).  sink: groups x waves x 64 floats
// written; stamps: NULL or 2 x groups values.  Returns 0, -1 for a shape
// the kernel does not take, or a positive hipError_t.
extern "C" __attribute__((visibility("default")))
int hbm_stream_read(const float *src, long long n, int groups, int waves, float *sink,
                    unsigned long long *stamps, hipStream_t s) {
  if ((waves != 4 && waves != 8) || groups < 1 || n <= 0 ||
      n % ((long long)groups * waves * 256) != 0)
    return -1;
  const long long per = n / groups;
  if (per * 4 > 0x7fffffffLL) return -1;
  switch (waves) {
    case 4:
      hipLaunchKernelGGL((stream_read<4, 4, 2>), dim3(groups), dim3(256), 0, s, src, per, sink,
                         stamps);
      break;
    case 8:
      hipLaunchKernelGGL((stream_read<8, 4, 2>), dim3(groups), dim3(512), 0, s, src, per, sink,
                         stamps);
      break;
    default:
      return -1;
  }
  return (int)hipGetLastError();
}
