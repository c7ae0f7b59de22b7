// The SGEMM configuration table: tile shapes from FP32GEMM_TILES with the
// launchers of the four operand-layout combinations.
#include <string>
#include <vector>

#include "sgemm_kernel.h"

namespace fp32gemm {

const GemmConfig *gemm_configs(int *count) {
  // Built once (thread-safe static initialisation), read-only afterwards.
  // Names: BMxBNxBK_wWMxWN, then _k2 when two wave groups split K and _p2 /
  // _p4 for K slices per barrier.
  struct Shape {
    int bm, bn, bk, wm, wn, ks, p, occ, mf;
  };
  static const std::vector<std::string> names = [] {
    const Shape shapes[] = {
#define FP32GEMM_ROW(BM, BN, BK, WM, WN, KS, P, OCC, MF) {BM, BN, BK, WM, WN, KS, P, OCC, MF},
        FP32GEMM_TILES(FP32GEMM_ROW)
#undef FP32GEMM_ROW
    };
    std::vector<std::string> n;
    for (const Shape &t : shapes) {
      std::string s = std::to_string(t.bm) + "x" + std::to_string(t.bn) + "x" + std::to_string(t.bk) +
                      "_w" + std::to_string(t.wm) + "x" + std::to_string(t.wn);
      if (t.ks > 1) s += "_k" + std::to_string(t.ks);
      if (t.p > 1) s += "_p" + std::to_string(t.p);
      if (t.mf == 16) s += "_m16";
      n.push_back(s);
    }
    return n;
  }();
  static const std::vector<GemmConfig> table = [] {
    const Shape shapes[] = {
#define FP32GEMM_ROW(BM, BN, BK, WM, WN, KS, P, OCC, MF) {BM, BN, BK, WM, WN, KS, P, OCC, MF},
        FP32GEMM_TILES(FP32GEMM_ROW)
#undef FP32GEMM_ROW
    };
    std::vector<GemmConfig> t;
    for (size_t i = 0; i < names.size(); ++i) {
      const Shape &h = shapes[i];
      t.push_back({names[i].c_str(), h.bm, h.bn, h.bk, h.wm, h.wn, h.occ, {nullptr, nullptr, nullptr, nullptr}});
    }
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
