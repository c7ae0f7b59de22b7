// The SGEMM configuration table: tile shapes from FP32GEMM_TILES with the
// launchers of the four operand-layout combinations.
#include <vector>

#include "sgemm_kernel.h"

namespace fp32gemm {

const GemmConfig *gemm_configs(int *count) {
  // Built once (thread-safe static initialisation), read-only afterwards.
  static const std::vector<GemmConfig> table = [] {
    std::vector<GemmConfig> t = {
#define FP32GEMM_ROW(BM, BN, BK, WM, WN, OCC) \
  {#BM "x" #BN "x" #BK "_w" #WM "x" #WN, BM, BN, BK, WM, WN, OCC, {nullptr, nullptr, nullptr, nullptr}},
        FP32GEMM_TILES(FP32GEMM_ROW)
#undef FP32GEMM_ROW
    };
    std::vector<GemmLaunchFn> nn(t.size()), nt(t.size()), tn(t.size()), tt(t.size());
    launchers_nn(nn.data());
    launchers_nt(nt.data());
    launchers_tn(tn.data());
    launchers_tt(tt.data());
    for (size_t i = 0; i < t.size(); ++i) {
      t[i].launch[0] = nn[i];
      t[i].launch[1] = nt[i];
      t[i].launch[2] = tn[i];
      t[i].launch[3] = tt[i];
    }
    return t;
  }();
  *count = (int)table.size();
  return table.data();
}

}  // namespace fp32gemm
