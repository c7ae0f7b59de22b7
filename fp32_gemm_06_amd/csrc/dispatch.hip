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

#include <mutex>
#include <string>
#include <string_view>
#include <unordered_map>
#include <vector>

#include "common.h"

namespace fp32gemm {
namespace {

struct ShapeEntry {
  int M, N, K;
  const char *name;
};
#include "tune_table.inc"

// Configuration names and their ids, built once; the selection runs on every
// call, so names are looked up by hash, not by scanning the list.
std::once_flag g_names_once;
std::vector<std::string> g_gemm_names;
std::unordered_map<std::string_view, int> g_gemm_ids, g_gemv_ids;

void build_names() {
  int n = 0;
  const GemmConfig *cfg = gemm_configs(&n);
  for (int t = 0; t < n; ++t)
    for (int g = 0; g < kNumGroups; ++g)
      g_gemm_names.push_back(std::string(cfg[t].name) + "_g" + std::to_string(kGroups[g]));
  for (size_t i = 0; i < g_gemm_names.size(); ++i) g_gemm_ids.emplace(g_gemm_names[i], (int)i);
  const GemvConfig *gv = gemv_configs(&n);
  for (int i = 0; i < n; ++i) g_gemv_ids.emplace(gv[i].name, i);
}

int find_gemm(const char *name) {
  std::call_once(g_names_once, build_names);
  const auto it = g_gemm_ids.find(name);
  return it == g_gemm_ids.end() ? -1 : it->second;
}

int find_gemv(const char *name) {
  std::call_once(g_names_once, build_names);
  const auto it = g_gemv_ids.find(name);
  return it == g_gemv_ids.end() ? -1 : it->second;
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
// which stops falling at one per CU (256 tiles).  Each tile also has a fixed
// cost outside its K loop (filling the pipeline, writing C), priced as k0
// extra steps of K: about 12 us per round of 256x256 tiles at 4092^3, the
// time of 52 steps; 41 for the smaller tiles, from eight 2048 x 2048 x 128
// products (80.5 us on 128x128 tiles against 83.5 on 256x256).  It moves
// short-K products to the 128x128 tile: 8192^2 x 64 runs in 98 us there
// against 103 on 256x256.  Checked against the sweep,
// the estimate picks the measured best of the three tiles at 15 of the 16
// swept shapes (at 2048^3 the two it confuses are 0.3% apart); tiny shapes
// such as 128^3 get the 64x64 tile.
namespace {
struct ModelTile {
  const char *name;
  int bm, bn;
  double full_rate;  // TFLOP/s with every CU busy
  double k0;         // fixed cost per tile in steps of K
  bool small;        // 4-wave tile that needs several workgroups per CU
};
const ModelTile kModelTiles[] = {
    {"256x256x32_w128x64_g4", 256, 256, 145.0, 52.0, false},
    {"128x128x32_w64x32_g4", 128, 128, 141.0, 41.0, false},
    {"64x64x32_w32x32_g4", 64, 64, 133.0, 41.0, true},
};
}  // namespace

int model_gemm_config(int M, int N, int K, int mult, double *rate_out) {
  int best = -1;
  double best_rate = -1.0;
  for (const ModelTile &c : kModelTiles) {
    const double tiles = (double)((M + c.bm - 1) / c.bm) * (double)((N + c.bn - 1) / c.bn) * mult;
    const double rounds = (double)(long long)((tiles + 255.0) / 256.0);
    // each round costs a whole tile's work per CU; only M x N x mult of it is useful
    double rate = c.full_rate / 256.0 * ((double)M * (double)N * mult) / (rounds * c.bm * c.bn);
    if (c.small && tiles < 1024.0) rate *= pow((tiles < 256.0 ? 256.0 : tiles) / 1024.0, 0.3);
    rate *= (double)K / ((double)K + c.k0);
    const int id = find_gemm(c.name);
    if (id >= 0 && rate > best_rate) {
      best_rate = rate;
      best = id;
    }
  }
  if (rate_out) *rate_out = best_rate;
  return best >= 0 ? best : 0;
}

int select_gemm_config(int M, int N, int K, int batch) {
  if (batch == 1)
    for (const ShapeEntry &e : kGemmTable)
      if (e.M == M && e.N == N && e.K == K) {
        const int id = find_gemm(e.name);
        if (id >= 0) return id;
      }
  int best = model_gemm_config(M, N, K, batch, nullptr);
  // Where the model settles on the 4-wave 64x64 tile, a 96x96 tile (four
  // waves of 48x48 on 16x16x4 blocks) is taken when its tiles fill one or
  // two whole rounds of 256 (at least 89% of the last round's slots, at
  // least 95% of the tile area inside C): with one or two workgroups per CU
  // a wave's larger tile keeps the matrix cores busier.  Measured against
  // the best 64x64 form on one GPU: 1536^3 63.4 us against 73.0, 1536 x 1536
  // x 4096 160.7 against 187.5, 384 x 6144 x 4096 160.5 against 188.3,
  // 1536 x 3072 x 1536 109.3 against 121.2, 192 x 11008 x 4096 160.2 against
  // 188.2.  With four rounds (3072^3) it was 1% slower, with half a round
  // (768 x 1536 x 4096, 1152^3) 19-23% slower.
  if (best == find_gemm("64x64x32_w32x32_g4") && K >= 256) {
    const long long t96 = (long long)((M + 95) / 96) * ((N + 95) / 96) * batch;
    const long long r96 = (t96 + 255) / 256;
    const double fill = (double)t96 / (256.0 * (double)r96);
    const double inside = (double)M * (double)N * batch / ((double)t96 * 96.0 * 96.0);
    const int id = find_gemm("96x96x32_w48x48_m16_g8");
    if (id >= 0 && r96 <= 2 && fill >= 0.89 && inside >= 0.95) return id;
  }
  const double tiles64 = (double)((M + 63) / 64) * (double)((N + 63) / 64) * batch;
  // With fewer than 192 tiles of 64x64 most CUs would hold none or one
  // workgroup.  32x32 tiles (four waves of one 16x16x4 block each) give four
  // times as many workgroups.  With at most two rounds of them and a long K,
  // four K slices go in flight per stage; otherwise two (less LDS, more
  // workgroups per CU, a shorter pipeline to fill).  Measured against the
  // best 64x64 form on one GPU: 384^3 5.5 against 10.0 us, 512^3 6.5 against
  // 12.3, 768^3 15.0 against 17.0, 800^3 16.0 against 17.9, 512 x 512 x 8192
  // 59.9 against 141.6, 256 x 1024 x 4096 32.2 against 72.8, 64 x 11008 x
  // 4096 65.5 against 74.1; at 850^3 and 896^3 (196 tiles) they were within
  // 2% either way.
  if (best == find_gemm("64x64x32_w32x32_g4") && tiles64 < 192.0 && K >= 128) {
    const double t32 = (double)((M + 31) / 32) * (double)((N + 31) / 32) * batch;
    const bool deep = t32 <= 512.0 && K >= 1024;
    const int id = find_gemm(deep ? "32x32x32_w16x16_p4_m16_g8" : "32x32x32_w16x16_p2_m16_g8");
    if (id >= 0) return id;
  }
  // With at most one 64x64 tile per CU (16 < tiles <= 256) and K long enough,
  // the variant that stages two K slices per barrier keeps two slices of
  // loads in flight instead of one.  Where B comes from HBM (a weight read
  // once per call) it is much faster: 74.3 us against 99.7 plain at
  // 160 x 4096 x 4096, 195.6 against 259.1 at 256 x 4096 x 11008; with B
  // already in the caches it is 2-8% faster (73.4 against 75.7 at
  // 160 x 4096 x 4096).  The variant that also splits each slice between
  // two groups of waves times the same with B cached but 8-13% slower from
  // HBM.  At 320..512 tiles the plain tile is up to 3% faster, and with
  // K = 260 the staging covers too few slices.
  if (best == find_gemm("64x64x32_w32x32_g4") && tiles64 > 16.0 && tiles64 <= 256.0 && K >= 512) {
    const int p2 = find_gemm("64x64x32_w32x32_p2_g8");
    if (p2 >= 0) best = p2;
  }
  // With more 64x64 tiles than CUs, 32-row tiles (32 x 128, same area) cut
  // the rows computed past M by up to half where M % 64 is 1..32.  They are
  // taken when that saves a whole round of 256 tiles: 160 x 11008 x 4096
  // (430 tiles instead of 516 on 192 padded rows) 142.4 us against 190.8,
  // 96 x 13824 x 4096 134.6 against 142.4.  With the same rounds they gained
  // at most 4% and lost up to 2% (352 x 4096 x 4096, 608 x 4096 x 4096,
  // 288 x 11008 x 4096: their full rate is 2.7% lower, 1023 against 998 us
  // at 4096^3).
  if (best == find_gemm("64x64x32_w32x32_g4") && tiles64 > 256.0) {
    const long long t32 = (long long)((M + 31) / 32) * ((N + 127) / 128) * batch;
    const long long rounds64 = ((long long)tiles64 + 255) / 256, rounds32 = (t32 + 255) / 256;
    const int id = find_gemm("32x128x32_w32x32_g8");
    if (id >= 0 && rounds32 < rounds64) best = id;
  }
  // From two rounds of 64x64 tiles on, the same tile built from 16x16x4
  // blocks (four accumulator chains per wave instead of one) is faster:
  // 768 x 4096 x 4096 189.4 us against 203.9, 4096 x 2816 x 4096 666.4
  // against 695.2, 3000^3 406.7 against 424.4; between one and two rounds it
  // is about 3% slower (384 x 4096 x 4096 131.5 against 128.3).
  if (best == find_gemm("64x64x32_w32x32_g4") && tiles64 >= 512.0) {
    const int id = find_gemm("64x64x32_w32x32_m16_g8");
    if (id >= 0) best = id;
  }
  return best;
}

// Tile quantization across two launches.  When the 256x256 tiles of a
// product overflow whole rounds of 256 (one per CU), the last round runs
// partly empty, and the smaller tiles that fill the GPU better run at a lower
// rate.  Splitting C instead into the columns (or rows) that fill exact rounds
// of 256x256 tiles and the rest, run as a second product with its own tile,
// keeps most of the work on the fast tile.  The model above prices both
// launches, plus 3 us for the second one; the split is taken when it is
// estimated at least 1% faster.  Measured (one GPU, 18 shapes the model
// flags): never slower, and 2-4% faster where the rest or the single launch
// falls to the 64x64 tile (2048 x 11008 x 4096: 1357 -> 1308 us).
RoundSplit plan_round_split(int M, int N, int K, int batch) {
  RoundSplit r{0, 0, -1};
  const int big = find_gemm("256x256x32_w128x64_g8");
  if (big < 0 || batch < 1 || M < 1 || N < 1 || K < 1) return r;
  const double work = 2.0 * (double)K * (double)batch;  // flop per element of C
  double rate = 0.0;
  (void)model_gemm_config(M, N, K, batch, &rate);
  double best = work * (double)M * (double)N / (rate * 1e6) * 0.99;  // us
  const long long tm = (M + 255) / 256, tn = (N + 255) / 256;
  for (int dim = 1; dim <= 2; ++dim) {
    const long long across = dim == 1 ? tm : tn;  // tiles across the split
    const long long along = dim == 1 ? tn : tm;   // tiles along the split dimension
    long long k1 = along - 1;
    while (k1 >= 1 && (across * k1 * batch) % 256 != 0) --k1;
    if (k1 < 1) continue;
    const int first = (int)(256 * k1);
    const int m1 = dim == 1 ? M : first, n1 = dim == 1 ? first : N;
    const int m2 = dim == 1 ? M : M - first, n2 = dim == 1 ? N - first : N;
    double r1 = 0.0, r2 = 0.0;
    (void)model_gemm_config(m1, n1, K, batch, &r1);
    (void)model_gemm_config(m2, n2, K, batch, &r2);
    const double t = work * ((double)m1 * n1 / (r1 * 1e6) + (double)m2 * n2 / (r2 * 1e6)) + 3.0;
    if (t < best) {
      best = t;
      r = RoundSplit{dim, first, big};
    }
  }
  return r;
}

// Stripe width for a grid of one workgroup per stripe of 16 nb columns and
// batch entry.  Such a workgroup's time hardly depends on N, so the grid
// costs about its rounds of 256 workgroups (one per CU) times the time of
// one workgroup, which grows with the width: cost[i] for 16 << i columns,
// relative to 16.  The narrowest width reaches no lower estimate than a
// wider one, so ties go to the narrower stripe.
int stripe_blocks(int N, int batch, int widest, const double cost[3]) {
  int best = 1;
  double best_t = -1.0;
  for (int i = 0, nb = 1; i < 3 && nb <= widest; ++i, nb *= 2) {
    const long long wg = (long long)((N + 16 * nb - 1) / (16 * nb)) * (batch > 1 ? batch : 1);
    const double t = (double)((wg + 255) / 256) * cost[i];
    if (best_t < 0.0 || t < best_t) {
      best_t = t;
      best = nb;
    }
  }
  return best;
}

// The skinny kernel: 32-column stripes hold M <= 128 and 64-column ones
// M <= 64.  One workgroup's time relative to a 16-column one grows with the
// rows (W stored K x N, K = 4096, one round of workgroups each): 32 columns
// 1.1x at M <= 16, 1.35x to M = 48, 1.45x at 64, 1.5x above; 64 columns
// 1.65x to M = 32 and 2.2x above.  Swept over N = 2048..16384 and M = 9..128,
// this picks the fastest width at every point but one (within 2%); N = 4608
// to 7168 had taken 16 columns and two rounds, 1.2-1.5x slower than one
// round of 32, and M = 65..128 at N = 8192 runs 1.28x faster on 32 columns.
// Over W stored N x K the 64-column stripes cost more still above M = 32
// (N = 16384, M = 33: 82.5 us against 76.7 on 32 columns), so there they
// stop at M = 32.
int skinny_stripe_blocks(int M, int N, int batch, bool transposed_w) {
  static const double cost[4][3] = {
      {1.0, 1.1, 1.65}, {1.0, 1.35, 1.7}, {1.0, 1.45, 2.2}, {1.0, 1.5, 9.9}};
  const int row = M <= 16 ? 0 : M <= 48 ? 1 : M <= 64 ? 2 : 3;
  const int widest = M <= (transposed_w ? 32 : 64) ? 4 : 2;
  return stripe_blocks(N, batch, widest, cost[row]);
}

// The column-stripe GEMV (M <= 8): 1.1 and 1.5 times the 16-column time for
// 32 and 64 columns (N = 4096: 18.2, 20.2 and 27.9 us at M = 1).  N = 4608
// to 7168 then runs on 32 columns (M = 1, N = 6144: 23.7 us against 35.0 on
// 16) and N = 9216 on 64 (36.0 against 42.5 on 32); the sizes swept before
// (N = 1024..65536 in powers of two, 11008, 32000) keep their widths.
int gemv_stripe_blocks(int N, int batch) {
  static const double cost[3] = {1.0, 1.1, 1.5};
  return stripe_blocks(N, batch, 4, cost);
}

int select_gemv_config(int M, int N, int K) { return select_gemv_config_batched(M, N, K, 1); }

int select_gemv_config_batched(int M, int N, int K, int batch) {
  if (batch == 1)
    for (const ShapeEntry &e : kGemvTable)
      if (e.M == M && e.N == N && e.K == K) {
        const int id = find_gemv(e.name);
        if (id >= 0) return id;
      }
  if (M > 8) {
    // The skinny MFMA kernel (N = 11008, M = 16: 42.1 us on 64 columns
    // against 62.7 on 16; N = 4608, M = 48: 39.7 on 32 against 56.5 on 16).
    const int nb = skinny_stripe_blocks(M, N, batch, false);
    const char *mf = nb == 4 ? "mfma64_w8" : nb == 2 ? "mfma32_w8" : "mfma16_w8";
    const int id = find_gemv(mf);
    return id >= 0 ? id : 0;
  }
  // W of 16 M floats and more with few column blocks: K split across
  // workgroups in 1 KB runs of each row (gemv_split.hip).
  if (gemv_split_pays(M, N, K, batch)) {
    const int id =
        find_gemv(gemv_split_waves(N, K) == 4 ? "split256_w4_u4" : "split256_w8_u4");
    if (id >= 0) return id;
  }
  // From M = 5 on, while its stripes fit one round of workgroups, the skinny
  // MFMA kernel is the faster (4096^2, M = 8: 20.1 us against 22.1 on the
  // column stripes; 8 x 4096 x 11008: 48.9 against 50.7; at M = 4 they are
  // 2% apart and at N = 11008 the 64-column stripe is 1.5% ahead).
  if (M >= 5 && (long long)N * (batch > 1 ? batch : 1) <= 256 * 32) {
    const int snb = skinny_stripe_blocks(M, N, batch, false);
    const int id = find_gemv(snb == 4 ? "mfma64_w8" : snb == 2 ? "mfma32_w8" : "mfma16_w8");
    if (id >= 0) return id;
  }
  // Wider column stripes read longer runs of each row of W (64, 128 or 256
  // bytes), which the memory system serves faster, but give fewer
  // workgroups.
  const int nb = gemv_stripe_blocks(N, batch);
  const char *name = nb == 4              ? "c64_w8_u4"
                     : nb == 2            ? "c32_w8_u4"
                     : M >= 4 && M <= 8   ? "c16_w4_u8"
                                          : "c16_w8_u4";
  const int id = find_gemv(name);
  return id >= 0 ? id : 0;
}

}  // namespace fp32gemm
