// Configuration naming and per-shape selection.
//
// The pages tune block and thread tile sizes per GPU with a search script
// and keep the best ("CUDA 矩阵乘法优化", section "8. Kernel 9: 参数自动调
// 优"), and note that the vendor library picks a specialised kernel by
// shape at run time ("10. cuBLAS 领先的性能差异").  Here the sweep
// (fp32_gemm_06_amd/tune.py) writes tune_table.inc with the best
// configuration per measured shape; other shapes fall back to a cost model
// over the same configurations.
#include <math.h>
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

// Fallback for shapes the table does not list.  The pages observe that a grid
// with too few blocks leaves the GPU idle ("CUDA 矩阵乘法优化", section
// "10. cuBLAS 领先的性能差异"), and that edge tiles waste the part of the
// tile outside the matrix ("GPU 基础原理", section "最后一个考虑：分块的量化").
// The estimate per tile shape is its full-load rate on MI355X (measured by
// the sweep) scaled by the useful fraction of the work: each of the rounds
// of up to 256 tiles (one 8-wave workgroup per CU at full rate) costs a whole
// tile's work, of which M x N of the rounds' tile area is useful.  The 4-wave
// 64x64 tile gets a further factor for fewer than four workgroups per CU,
// which stops falling at one per CU (256 tiles).  Checked against the sweep,
// the estimate picks the measured best of the three tiles at 15 of the 16
// swept shapes (at 2048^3 the two it confuses are 1.7% apart); tiny shapes
// such as 128^3 get the 64x64 tile.
int model_gemm_config(int M, int N, int mult, double *rate_out) {
  struct Candidate {
    const char *name;
    int bm, bn;
    double full_rate;  // TFLOP/s with every CU busy
    bool small;        // 4-wave tile that needs several workgroups per CU
  };
  static const Candidate cands[] = {
      {"256x256x32_w128x64_g4", 256, 256, 145.0, false},
      {"128x128x32_w64x32_g4", 128, 128, 141.0, false},
      {"64x64x32_w32x32_g4", 64, 64, 133.0, true},
  };
  int best = -1;
  double best_rate = -1.0;
  for (const Candidate &c : cands) {
    const double tiles = (double)((M + c.bm - 1) / c.bm) * (double)((N + c.bn - 1) / c.bn) * mult;
    const double rounds = (double)(long long)((tiles + 255.0) / 256.0);
    // each round costs a whole tile's work per CU; only M x N x mult of it is useful
    double rate = c.full_rate / 256.0 * ((double)M * (double)N * mult) / (rounds * c.bm * c.bn);
    if (c.small && tiles < 1024.0) rate *= pow((tiles < 256.0 ? 256.0 : tiles) / 1024.0, 0.3);
    const int id = find_gemm(c.name);
    if (id >= 0 && rate > best_rate) {
      best_rate = rate;
      best = id;
    }
  }
  if (rate_out) *rate_out = best_rate;
  return best >= 0 ? best : 0;
}

// Fallback for shapes the table does not list.  The pages observe that a grid
// with too few blocks leaves the GPU idle ("CUDA 矩阵乘法优化", section
// "10. cuBLAS 领先的性能差异"), and that edge tiles waste the part of the
// tile outside the matrix ("GPU 基础原理", section "最后一个考虑：分块的量化").
// The estimate per tile shape is its full-load rate on MI355X (measured by
// the sweep) scaled by the useful fraction of the work: each of the rounds
// of up to 256 tiles (one 8-wave workgroup per CU at full rate) costs a whole
// tile's work, of which M x N of the rounds' tile area is useful.  The 4-wave
// 64x64 tile gets a further factor for fewer than four workgroups per CU,
// which stops falling at one per CU (256 tiles).  Checked against the sweep,
// the estimate picks the measured best of the three tiles at 15 of the 16
// swept shapes (at 2048^3 the two it confuses are 1.7% apart); tiny shapes
// such as 128^3 get the 64x64 tile.
int select_gemm_config(int M, int N, int K) {
  for (const ShapeEntry &e : kGemmTable)
    if (e.M == M && e.N == N && e.K == K) {
      const int id = find_gemm(e.name);
      if (id >= 0) return id;
    }
  return model_gemm_config(M, N, 1, nullptr);
}

int select_gemv_config(int M, int N, int K) { return select_gemv_config_batched(M, N, K, 1); }

int select_gemv_config_batched(int M, int N, int K, int batch) {
  if (batch == 1)
    for (const ShapeEntry &e : kGemvTable)
      if (e.M == M && e.N == N && e.K == K) {
        const int id = find_gemv(e.name);
        if (id >= 0) return id;
      }
  // the workgroup count is the stripes of N times the batch entries
  const long long NB = (long long)N * (batch > 1 ? batch : 1);
  // Wider column stripes read longer runs of each row of W (64, 128 or 256
  // bytes), which the memory system serves faster, but give fewer
  // workgroups.  The sweep over N from 1024 to 65536 is fastest with the
  // widest stripe that still leaves about 160 workgroups or more.
  (void)K;
  const char *name = NB >= 160 * 64   ? "c64_w8_u4"
                     : NB >= 256 * 32 ? "c32_w8_u4"
                     : M >= 4        ? "c16_w4_u8"
                                     : "c16_w8_u4";
  const int id = find_gemv(name);
  return id >= 0 ? id : 0;
}

}  // namespace fp32gemm
