// Configuration naming and per-shape selection.
//
// The pages tune block and thread tile sizes per GPU with a search script
// and keep the best ("CUDA 矩阵乘法优化", section "8. Kernel 9: 参数自动调
// 优"), and note that the vendor library picks a specialised kernel by
// shape at run time ("10. cuBLAS 领先的性能差异").  Here the sweep
// (fp32_gemm_06_amd/tune.py) writes tune_table.inc with the best
// configuration per measured shape; other shapes fall back to a cost model
// over the same configurations.
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "common.h"

namespace fp32gemm {
namespace {

struct ShapeEntry {
  int M, N, K;
  const char *name;
};
#include "tune_table.inc"

std::once_flag g_names_once;
std::vector<std::string> g_gemm_names;

void build_names() {
  int n = 0;
  const GemmConfig *cfg = gemm_configs(&n);
  for (int t = 0; t < n; ++t)
    for (int g = 0; g < kNumGroups; ++g)
      g_gemm_names.push_back(std::string(cfg[t].name) + "_g" + std::to_string(kGroups[g]));
}

int find_gemm(const char *name) {
  std::call_once(g_names_once, build_names);
  for (size_t i = 0; i < g_gemm_names.size(); ++i)
    if (g_gemm_names[i] == name) return (int)i;
  return -1;
}

int find_gemv(const char *name) {
  int n = 0;
  const GemvConfig *cfg = gemv_configs(&n);
  for (int i = 0; i < n; ++i)
    if (strcmp(cfg[i].name, name) == 0) return i;
  return -1;
}

}  // namespace

int num_gemm_config_ids() {
  std::call_once(g_names_once, build_names);
  return (int)g_gemm_names.size();
}

const char *gemm_config_name(int id) {
  std::call_once(g_names_once, build_names);
  if (id < 0 || id >= (int)g_gemm_names.size()) return nullptr;
  return g_gemm_names[id].c_str();
}

// Size-class fallback: estimate each tile shape's time as the number of
// rounds of workgroups the 256 CUs run, times the work of one tile, divided
// by a per-shape efficiency (bigger tiles reuse more data per LDS byte), and
// take the cheapest.  Ties go to the earlier (larger) tile.
int select_gemm_config(int M, int N, int K) {
  for (const ShapeEntry &e : kGemmTable)
    if (e.M == M && e.N == N && e.K == K) {
      const int id = find_gemm(e.name);
      if (id >= 0) return id;
    }
  int n = 0;
  const GemmConfig *cfg = gemm_configs(&n);
  double best = 1e300;
  int best_t = 0;
  for (int t = 0; t < n; ++t) {
    const GemmConfig &c = cfg[t];
    const double tiles = (double)((M + c.BM - 1) / c.BM) * (double)((N + c.BN - 1) / c.BN);
    const int per_cu = c.lds_bytes <= 80 * 1024 ? 2 : 1;
    const double rounds = (double)(long long)((tiles + 256.0 * per_cu - 1) / (256.0 * per_cu));
    const double kpad = (double)((K + c.BK - 1) / c.BK) * c.BK;
    const double eff = (c.BM >= 256 || c.BN >= 256) ? 1.0 : (c.BM >= 128 ? 0.85 : 0.5);
    const double cost = rounds * c.BM * c.BN * kpad * per_cu / eff;
    if (cost < best * 0.999) {
      best = cost;
      best_t = t;
    }
  }
  return best_t * kNumGroups + 2;  // group of 4 tile-rows
}

int select_gemv_config(int M, int N, int K) {
  for (const ShapeEntry &e : kGemvTable)
    if (e.M == M && e.N == N && e.K == K) {
      const int id = find_gemv(e.name);
      if (id >= 0) return id;
    }
  // Narrow column blocks keep enough workgroups in flight unless N is huge.
  const int id = find_gemv(N >= 65536 ? "c64_w16_u8" : "c16_w8_u8");
  return id >= 0 ? id : 0;
}

}  // namespace fp32gemm
