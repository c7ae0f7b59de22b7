// SGEMM kernels for op(A) = A, op(B) = B^T (see sgemm_kernel.h).
#include "sgemm_kernel.h"

namespace fp32gemm {
#define FP32GEMM_LAUNCHER(BM, BN, BK, WM, WN, KS, P, OCC, MF) &launch<Tile<BM, BN, BK, WM, WN, KS, P, MF>, false, true>,
// Fills out[] with this combination's launchers in tile-list order (a host
// function, so the device pass does not try to emit host function pointers).
void launchers_nt(GemmLaunchFn *out) {
  const GemmLaunchFn t[] = {FP32GEMM_TILES(FP32GEMM_LAUNCHER)};
  for (size_t i = 0; i < sizeof(t) / sizeof(t[0]); ++i) out[i] = t[i];
}
#undef FP32GEMM_LAUNCHER
#define FP32GEMM_SK_LAUNCHER(BM, BN, BK, WM, WN, KS, P, OCC, MF) \
  &launch_sk<Tile<BM, BN, BK, WM, WN, KS, P, MF>, false, true>,
void sk_launchers_nt(SkLaunchFn *out) {
  const SkLaunchFn t[] = {FP32GEMM_SK_TILES(FP32GEMM_SK_LAUNCHER)};
  for (size_t i = 0; i < sizeof(t) / sizeof(t[0]); ++i) out[i] = t[i];
}
#undef FP32GEMM_SK_LAUNCHER
}  // namespace fp32gemm
