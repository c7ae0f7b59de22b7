// SGEMM C <- alpha op(A) op(B) + beta C on gfx950 with the fp32 matrix cores.
// Included by sgemm_nn.hip, sgemm_nt.hip, sgemm_tn.hip and sgemm_tt.hip, which
// instantiate it for one operand-layout combination each.
//
// The structure follows the tiling the pages build up step by step, mapped
// onto CDNA4:
//  * a workgroup owns a BM x BN tile of C and walks K in slices of BK
//    ("GPU 基础原理", section "4.2 分块": the sum over k regrouped by tiles);
//  * each K slice of both operands is staged in LDS, loaded with 128-bit
//    coalesced reads ("GPU 基础原理", section "4.3 合并加载"; "CUDA 矩阵乘法
//    优化", section "7. Kernel 6: 向量化访存优化"), here with the
//    buffer_load ... lds DMA path that writes LDS without VGPR staging;
//  * LDS layouts are free of bank conflicts ("GPU GEMM 优化完全拆解（一）",
//    sections "32 个 bank" and "两种解法：Padding 与线性化"): k-contiguous
//    tiles use an XOR swizzle of 16-byte chunks, mn-contiguous tiles a gap
//    between their two k-halves;
//  * each 64-lane wave owns a WM x WN sub-tile of 32 x 32 blocks, the CDNA4
//    counterpart of warp tiling with per-thread register blocks ("CUDA 矩阵乘
//    法优化", sections "6. Kernel 5" and "9. Kernel 10: 线程束级分块"); the
//    outer product becomes v_mfma_f32_32x32x2_f32 (fp32 in, fp32 accumulate),
//    or, for tiles built from 16 x 16 blocks (MF = 16), v_mfma_f32_16x16x4_f32;
//  * slice k+1 is fetched while the matrix cores work on slice k, with two
//    LDS buffers and one barrier per slice (double buffering, "11. 探索未尽与
//    总结"; the two-barrier rule of "GPU GEMM 优化完全拆解（一）", section
//    "分块的思想"); small tiles may instead stage P slices per barrier, which
//    matters when a CU holds a single workgroup;
//  * optionally (KS = 2) two groups of waves split every K slice between them
//    and add their accumulators through LDS at the end, in group order: the
//    pages' split-K ("CUDA 矩阵乘法优化", section "10. cuBLAS 领先的性能差
//    异") kept inside the workgroup, so small grids get twice the waves per
//    SIMD without a workspace or any cross-workgroup synchronisation;
//  * tiles that overhang M, N or K are zero-filled by buffer loads whose
//    out-of-range offsets read zero, and stores outside C are dropped the same
//    way ("GPU 基础原理", section "最后一个考虑：分块的量化"), so interior and
//    edge tiles run one instruction stream;
//  * with beta = 0 the last K slice finishes one row of blocks at a time and
//    stores it while the next row's MFMAs run, so writing C overlaps the end
//    of the K loop instead of following it.
//
// Operand layouts.  op(A) is M x K and op(B) is K x N.  An operand is
// k-contiguous (KC) when its storage rows run along k: A as given, or B when
// op(B) = B^T (B stored N x K).  It is mn-contiguous (MC) when its rows run
// along m or n: A when op(A) = A^T (A stored K x M), or B as given.
//
// K order inside a slice.  For v_mfma_f32_32x32x2_f32 lane l supplies
// A[l % 32][k] and B[k][l % 32] with k = l / 32 of the instruction's pair.
// Any bijection between (step, lane half) and the BK values of k gives the
// same sum, so lane half h takes k = h * BK/2 + step.  A KC operand then has
// a lane's values for four consecutive steps next to each other in LDS (one
// ds_read_b128); an MC operand has the 32 lanes of a half reading 32
// consecutive floats of one k-row (one ds_read_b32 per step).
// For v_mfma_f32_16x16x4_f32 lane l supplies A[l % 16][k] and B[k][l % 16]
// with k = l / 16 of the instruction's four; lane quarter q takes
// k = 16 (q % 2) + 8 (q / 2) + step of a 32-wide slice, which keeps four
// steps of a KC operand in one chunk and puts the quarters that an LDS cycle
// serves together on the two sides of an MC tile's k-half gap.
#pragma once

#include "common.h"

namespace fp32gemm {
namespace {

// KS groups of WT waves each; group g takes MFMA step groups
// [g * NG / KS, (g + 1) * NG / KS) of every K slice (NG = BK / 8 groups of
// four MFMA steps).
// P > 1 (128-bit path): P K slices per barrier, i.e. stages of P slices in
// 2 P LDS buffers, the next stage in flight during the current one (the
// 32-bit staged path always uses one slice per barrier).
template <int BM_, int BN_, int BK_, int WM_, int WN_, int KS_ = 1, int P_ = 1, int MF_ = 32>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, KS = KS_, P = P_, MF = MF_;
  static constexpr int WAVES_N = BN / WN;
  static constexpr int WT = (BM / WM) * WAVES_N;  // waves per K group
  static constexpr int WAVES = WT * KS;
  static constexpr int NT = WAVES * 64;
  static constexpr int TM = WM / MF, TN = WN / MF;
  static constexpr int NGW = BK / (MF == 32 ? 8 : 16) / KS;  // step groups per wave per slice
  static constexpr int ACCN = MF == 32 ? 16 : 4;             // accumulator floats per block
  static_assert(MF == 32 || (MF == 16 && BK == 32), "16x16x4 blocks take 32-wide K slices");
  static_assert(BM % WM == 0 && BN % WN == 0 && WM % MF == 0 && WN % MF == 0, "wave tiling");
  static_assert(BK == 16 || BK == 32, "K slice of 16 or 32");
  static_assert(KS >= 1 && NGW >= 2 && NGW % 2 == 0, "fragment double buffering needs an even group count");
  static_assert(P >= 1 && P <= 4, "one to four K slices per barrier");
};

template <int MF> struct AccOf { typedef floatx16 type; };
template <> struct AccOf<16> { typedef floatx4 type; };

// Chunk swizzle of row r of a KC tile (float4 chunks of a BK-float row).
// Checked exhaustively to keep ds_read_b128 of 32 consecutive rows at one
// chunk conflict-free for 8-lane/32-bank and 16-lane/64-bank service.
template <int BK>
__device__ __forceinline__ int kc_swizzle(int r) {
  if constexpr (BK == 32) return (r & 7) ^ ((r >> 3) & 1);
  else return ((r >> 1) ^ (r >> 3)) & 3;
}

// One operand tile: `E` rows or columns along m/n (BM for A, BN for B) by BK
// along k, loaded by `WAVES` waves in whole 1 KB DMA instructions.  Lane l of
// instruction `inst` moves float4 chunk f = 64 inst + l of the tile, counted
// along the storage rows (CP chunks a row).
template <bool KC, int E, int BK, int WAVES>
struct Operand {
  // LDS floats of the tile
  static constexpr int FLOATS = KC ? E * BK : BK * E + 32;
  // DMA instructions per wave per slice (one instruction = 64 lanes x 16 bytes)
  static constexpr int NI = E * BK / 256 / WAVES;
  static_assert(E * BK % (256 * WAVES) == 0, "whole DMA instructions per wave");
  // KC: chunks per row (along k); MC: chunks per k-row (along m / n)
  static constexpr int CP = KC ? BK / 4 : E / 4;
  static_assert(!KC || 64 % CP == 0, "a KC instruction covers whole rows");
  static_assert(KC || (BK / 2) * CP % 64 == 0, "each k-half of an MC tile is whole instructions");

  // LDS float offset where instruction `inst` writes its 1 KB (MC: the second
  // k-half sits 32 floats further on)
  __device__ __forceinline__ static int dst(int inst) {
    if constexpr (KC) return inst * 256;
    else return inst * 256 + (inst * 64 >= (BK / 2) * CP ? 32 : 0);
  }
  // Source element (row along storage, column along storage) of the first of
  // the 4 floats this lane moves in instruction `inst`.  KC: (e, k); MC: (k, e).
  __device__ __forceinline__ static void src(int inst, int lane, int &row, int &col) {
    int c;  // chunk f % CP of the row
    if constexpr (64 % CP == 0) {
      row = inst * (64 / CP) + lane / CP;  // whole rows per instruction
      c = lane % CP;
    } else {
      const int f = inst * 64 + lane;
      row = f / CP;
      c = f % CP;
    }
    // KC: row along m / n, col along k; MC: row along k, col along m / n
    col = KC ? 4 * (c ^ kc_swizzle<BK>(row)) : 4 * c;
  }
};

// Stream-K work assignment (SK kernels only, SkArgs in common.h).  The
// product's tiles x nk K slices are numbered tile-major ("units"); logical
// workgroup g (ids renumbered XCD by XCD, as for tiles) takes units
// [g ipw, (g + 1) ipw).  A tile whose units several workgroups
// share is finished by the last of them to arrive, which adds the others'
// raw partial tiles in K order.  part: 2 x grid partial tiles of BM x BN
// floats (slot 2 g for a workgroup's first segment, 2 g + 1 for its last);
// cnt: one arrival counter per tile, zero between calls.

// The kernel: one BM x BN tile of C (of batch entry blockIdx.y) per workgroup,
// or (SK) the stream-K units of workgroup blockIdx.x.  DMA = 128-bit loads
// straight into LDS; otherwise 32-bit loads staged in registers and written
// to the same LDS positions (any alignment).
template <class T, bool TRANS_A, bool TRANS_B, bool DMA, bool SK = false>
__global__ void __launch_bounds__(T::NT) __attribute__((amdgpu_waves_per_eu(SK && T::WAVES <= 4 ? 4 : 1)))
sgemm_kernel(GemmArgs a, int tiles_m, int tiles_n, int group_m, SkArgs sk) {
  constexpr int BM = T::BM, BN = T::BN, BK = T::BK, WAVES = T::WAVES;
  constexpr bool KCA = !TRANS_A;  // A as given is k-contiguous
  constexpr bool KCB = TRANS_B;   // B^T storage is k-contiguous
  using OA = Operand<KCA, BM, BK, WAVES>;
  using OB = Operand<KCB, BN, BK, WAVES>;
  constexpr int STAGE = OA::FLOATS + OB::FLOATS;
  constexpr int NS = DMA ? 2 * T::P : 2;  // LDS buffers
  __shared__ __attribute__((aligned(16))) float lds[NS * STAGE];
  __shared__ int sk_last;  // stream-K: this workgroup finishes the tile
  (void)sk_last;

  // ---- batch and C tile (XCD-aware order) ---------------------------------
  const long long bz = blockIdx.y;
  const float *Ag = a.A + bz * a.sA;
  const float *Bg = a.B + bz * a.sB;
  float *Cg = a.C + bz * a.sC;
  // logical tile id -> tile origin, strips of group_m tile-rows
  auto tile_origin = [&](int lid, int &m0, int &n0) {
    const int width = group_m * tiles_n;
    const int grp = lid / width;
    const int first_m = grp * group_m;
    const int gsz = min(tiles_m - first_m, group_m);
    const int within = lid - grp * width;
    m0 = (first_m + within % gsz) * BM;
    n0 = (within / gsz) * BN;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave / T::WT, wt = wave % T::WT;  // K group; wave inside the group
  const int wm = wt / T::WAVES_N, wn = wt % T::WAVES_N;
  const int l32 = lane & 31, half = lane >> 5;
  const int c16 = lane & 15, q4 = lane >> 4;

  // split-K chunks: the last one may be shorter
  const int Kb = a.k_total > 0 ? min(a.K, a.k_total - (int)bz * a.K) : a.K;
  const int nk_tile = (Kb + BK - 1) / BK;
  const int ktail_tile = Kb - (nk_tile - 1) * BK;  // valid k in the tile's last slice, 1..BK

  // Workgroups are handed to the 8 XCDs round-robin by id; logical ids
  // number them so that each XCD receives a contiguous range, so the tiles
  // (or stream-K units) an XCD runs together are neighbours that share A
  // and B panels in its L2.
  const int G = gridDim.x;
  const int xcd = (int)blockIdx.x & 7, per = G >> 3, extra = G & 7;
  const int lid = xcd * per + min(xcd, extra) + ((int)blockIdx.x >> 3);

  // Stream-K arrival bookkeeping.  A workgroup's first segment, when more
  // segments follow, is published without waiting: its arrival at tile
  // pend_t is counted after the next segment's first barrier (by then the
  // partial-tile stores have completed), and if it turns out to be the last
  // arrival, that tile is finished after this workgroup's other segments.
  int pend_t = -1;           // tile of the first segment, arrival pending or counted
  bool pend_sent = false;    // its arrival has been counted
  bool pend_fix = false;     // ... and it was the last one
  bool pend_done = false;    // pend_fix is known
  unsigned pend_before = 0;  // (thread 0) the counter before that arrival
  (void)pend_sent;
  (void)pend_fix;
  (void)pend_done;
  (void)pend_before;
  // segments (workgroups) that share tile t
  auto nseg_of = [&](int t) -> int {
    const long long u0 = (long long)t * nk_tile;
    return (int)((u0 + nk_tile - 1) / sk.ipw - u0 / sk.ipw) + 1;
  };
  (void)nseg_of;
  auto signal_pending = [&]() {
    if (pend_t >= 0 && !pend_sent) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial tile is written
      __syncthreads();
      if (tid == 0)
        pend_before = __hip_atomic_fetch_add(&sk.cnt[pend_t], 1u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
      pend_sent = true;
    }
  };
  (void)signal_pending;

  // One tile (origin m0, n0; tile id t for stream-K) over its K slices
  // [kb, ke).  Stream-K: slot is the partial-tile slot of this segment,
  // last_seg whether it ends the workgroup's units; kb == ke only finishes
  // tile t from the published partial tiles.
  auto run = [&](int m0, int n0, int kb, int ke, int t, int slot, bool last_seg) {
  (void)t;
  (void)slot;
  (void)last_seg;
  const int rows = a.M - m0;  // valid rows of this tile (may exceed BM)
  const int cols = a.N - n0;
  const int nk = ke - kb;                             // slices of this segment
  const int ktail = ke == nk_tile ? ktail_tile : BK;  // valid k in its last slice

  // Source offset (bytes from the slice's base) of the first of this lane's
  // 4 floats per instruction, or kOob when the lane's storage row lies
  // outside the matrix; plus that element's storage column.  On the DMA path
  // the 4 floats are all valid or all invalid (K and the m/n extent are
  // multiples of 4 there), so the column check is folded in as well; the
  // staged path checks each of the 4 floats when it loads them.
  uint32_t offa[OA::NI], offb[OB::NI];
  int cola[OA::NI], colb[OB::NI];
  auto set_offsets = [&](int kvalid) {
#pragma unroll
    for (int q = 0; q < OA::NI; ++q) {
      int row, col;
      OA::src(wave * OA::NI + q, lane, row, col);
      // KC: row = m, col = k.  MC: row = k, col = m.
      const bool row_ok = KCA ? row < rows : row < kvalid;
      const bool col_ok = KCA ? col < kvalid : col < rows;
      offa[q] = (row_ok && (col_ok || !DMA)) ? (uint32_t)(row * a.lda + col) * 4u : kOob;
      cola[q] = col;
    }
#pragma unroll
    for (int q = 0; q < OB::NI; ++q) {
      int row, col;
      OB::src(wave * OB::NI + q, lane, row, col);
      // KC: row = n, col = k.  MC: row = k, col = n.
      const bool row_ok = KCB ? row < cols : row < kvalid;
      const bool col_ok = KCB ? col < kvalid : col < cols;
      offb[q] = (row_ok && (col_ok || !DMA)) ? (uint32_t)(row * a.ldb + col) * 4u : kOob;
      colb[q] = col;
    }
  };

  // Slice bases: the tile origin moved to K slice ks.
  auto base_a = [&](int ks) -> const float * {
    return KCA ? Ag + (size_t)m0 * a.lda + (size_t)(kb + ks) * BK
               : Ag + (size_t)(kb + ks) * BK * a.lda + m0;
  };
  auto base_b = [&](int ks) -> const float * {
    return KCB ? Bg + (size_t)n0 * a.ldb + (size_t)(kb + ks) * BK
               : Bg + (size_t)(kb + ks) * BK * a.ldb + n0;
  };

  // Staged path: registers between the global loads and the LDS writes.
  floatx4 sa[DMA ? 1 : OA::NI], sb[DMA ? 1 : OB::NI];
  (void)sa;
  (void)sb;

  // Start moving slice ks into LDS buffer `buf` (DMA) or into registers.
  auto fetch = [&](float *buf, int ks) {
    const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(base_a(ks));
    const __amdgpu_buffer_rsrc_t rs_b = make_rsrc(base_b(ks));
    if constexpr (DMA) {
#pragma unroll
      for (int q = 0; q < OA::NI; ++q) dma16(rs_a, buf + OA::dst(wave * OA::NI + q), offa[q]);
#pragma unroll
      for (int q = 0; q < OB::NI; ++q)
        dma16(rs_b, buf + OA::FLOATS + OB::dst(wave * OB::NI + q), offb[q]);
    } else {
      (void)buf;
      const int kvalid = ks == nk - 1 ? ktail : BK;
      // a float is loaded when its storage column is inside the matrix
      // (the row check is already in the base offset)
      const int alim = KCA ? kvalid : rows, blim = KCB ? kvalid : cols;
#pragma unroll
      for (int q = 0; q < OA::NI; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t off = cola[q] + e < alim ? offa[q] + 4u * e : kOob;
          sa[q][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_a, off, 0, 0));
        }
#pragma unroll
      for (int q = 0; q < OB::NI; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t off = colb[q] + e < blim ? offb[q] + 4u * e : kOob;
          sb[q][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_b, off, 0, 0));
        }
    }
  };
  // Staged path: write the registers where the DMA would have put them.
  auto commit = [&](float *buf) {
    if constexpr (!DMA) {
#pragma unroll
      for (int q = 0; q < OA::NI; ++q)
        *reinterpret_cast<floatx4 *>(buf + OA::dst(wave * OA::NI + q) + 4 * lane) = sa[q];
#pragma unroll
      for (int q = 0; q < OB::NI; ++q)
        *reinterpret_cast<floatx4 *>(buf + OA::FLOATS + OB::dst(wave * OB::NI + q) + 4 * lane) = sb[q];
    } else {
      (void)buf;
    }
  };

  typedef typename AccOf<T::MF>::type acc_t;
  acc_t acc[T::TM][T::TN];
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j) acc[i][j] = acc_t{};

  // Operand fragments of one group of four MFMA steps: per 32-wide block,
  // this lane's four k values (k = half * BK/2 + 4g + step).
  struct Frag {
    float a[T::TM][4];
    float b[T::TN][4];
  };
  constexpr int MF = T::MF;
  const int lr = MF == 32 ? l32 : c16;
  const int ar = wm * T::WM + lr;  // this lane's row of block 0 along m
  const int br = wn * T::WN + lr;  // ... along n
  const int asw = kc_swizzle<BK>(ar), bsw = kc_swizzle<BK>(br);  // same for every block
  // 16x16x4 blocks: lane quarter q takes k = 16 (q % 2) + 8 (q / 2) + step
  // of the slice's 8 steps, so a KC read of four steps is one chunk and the
  // quarters of an MC read fall in different k-halves (the 32-float gap).
  const int kq = 16 * (q4 & 1) + 8 * (q4 >> 1);
  auto read_frag = [&](const float *buf, int g, Frag &f) {
    const float *As = buf;
    const float *Bs = buf + OA::FLOATS;
    if constexpr (MF == 16) {
      if constexpr (KCA) {
        const float *pa = As + ar * BK + 4 * (((kq >> 2) + g) ^ asw);
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
          const floatx4 v = *reinterpret_cast<const floatx4 *>(pa + i * 16 * BK);
#pragma unroll
          for (int st = 0; st < 4; ++st) f.a[i][st] = v[st];
        }
      } else {
        const float *pa = As + (kq + 4 * g) * BM + (q4 & 1) * 32 + ar;
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int i = 0; i < T::TM; ++i) f.a[i][st] = pa[st * BM + i * 16];
      }
      if constexpr (KCB) {
        const float *pb = Bs + br * BK + 4 * (((kq >> 2) + g) ^ bsw);
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
          const floatx4 v = *reinterpret_cast<const floatx4 *>(pb + j * 16 * BK);
#pragma unroll
          for (int st = 0; st < 4; ++st) f.b[j][st] = v[st];
        }
      } else {
        const float *pb = Bs + (kq + 4 * g) * BN + (q4 & 1) * 32 + br;
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int j = 0; j < T::TN; ++j) f.b[j][st] = pb[st * BN + j * 16];
      }
      return;
    }
    if constexpr (KCA) {
      const float *pa = As + ar * BK + 4 * ((half * (BK / 8) + g) ^ asw);
#pragma unroll
      for (int i = 0; i < T::TM; ++i) {
        const floatx4 v = *reinterpret_cast<const floatx4 *>(pa + i * 32 * BK);
#pragma unroll
        for (int st = 0; st < 4; ++st) f.a[i][st] = v[st];
      }
    } else {
      const float *pa = As + (half * (BK / 2) + 4 * g) * BM + half * 32 + ar;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < T::TM; ++i) f.a[i][st] = pa[st * BM + i * 32];
    }
    if constexpr (KCB) {
      const float *pb = Bs + br * BK + 4 * ((half * (BK / 8) + g) ^ bsw);
#pragma unroll
      for (int j = 0; j < T::TN; ++j) {
        const floatx4 v = *reinterpret_cast<const floatx4 *>(pb + j * 32 * BK);
#pragma unroll
        for (int st = 0; st < 4; ++st) f.b[j][st] = v[st];
      }
    } else {
      const float *pb = Bs + (half * (BK / 2) + 4 * g) * BN + half * 32 + br;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) f.b[j][st] = pb[st * BN + j * 32];
    }
  };
  // The values one 32 x 32 block takes in the four steps of step group g,
  // from the positions read_frag reads: block row i of op(A), block column j
  // of op(B).
  auto read_a_blk = [&](const float *buf, int g, int i, float(&q)[4]) {
    if constexpr (KCA) {
      const float *pa = buf + ar * BK + 4 * ((half * (BK / 8) + g) ^ asw);
      const floatx4 v = *reinterpret_cast<const floatx4 *>(pa + i * 32 * BK);
#pragma unroll
      for (int st = 0; st < 4; ++st) q[st] = v[st];
    } else {
      const float *pa = buf + (half * (BK / 2) + 4 * g) * BM + half * 32 + ar;
#pragma unroll
      for (int st = 0; st < 4; ++st) q[st] = pa[st * BM + i * 32];
    }
  };
  auto read_b_blk = [&](const float *buf, int g, int j, float(&q)[4]) {
    const float *Bs = buf + OA::FLOATS;
    if constexpr (KCB) {
      const float *pb = Bs + br * BK + 4 * ((half * (BK / 8) + g) ^ bsw);
      const floatx4 v = *reinterpret_cast<const floatx4 *>(pb + j * 32 * BK);
#pragma unroll
      for (int st = 0; st < 4; ++st) q[st] = v[st];
    } else {
      const float *pb = Bs + (half * (BK / 2) + 4 * g) * BN + half * 32 + br;
#pragma unroll
      for (int st = 0; st < 4; ++st) q[st] = pb[st * BN + j * 32];
    }
  };
  // Epilogue pieces.  Accumulator register v of lane l holds row
  // 8*(v/4) + 4*(l/32) + v%4, column l%32 of its 32 x 32 block (16 x 16
  // blocks: register v of lane (q, c) holds row 4 q + v, column c).
  auto c_off = [&](int i, int j, int v) -> uint32_t {
    const int row = MF == 32 ? wm * T::WM + i * 32 + 8 * (v / 4) + 4 * half + (v % 4)
                             : wm * T::WM + i * 16 + 4 * q4 + v;
    const int col = wn * T::WN + j * MF + lr;
    return (row < rows && col < cols) ? (uint32_t)(row * a.ldc + col) * 4u : kOob;
  };
  // this lane's bias value per block column (0 without a bias)
  auto load_bias = [&](float(&bj)[T::TN]) {
#pragma unroll
    for (int j = 0; j < T::TN; ++j) bj[j] = 0.0f;
    if (a.bias != nullptr) {
      const __amdgpu_buffer_rsrc_t rs_bias = make_rsrc(a.bias + n0);
#pragma unroll
      for (int j = 0; j < T::TN; ++j) {
        const int col = wn * T::WN + j * MF + lr;
        const uint32_t off = col < cols ? (uint32_t)col * 4u : kOob;
        bj[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_bias, off, 0, 0));
      }
    }
  };

  auto mma = [&](const Frag &f) {
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
          if constexpr (MF == 16)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(f.a[i][st], f.b[j][st], acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[i][st], f.b[j][st], acc[i][j], 0, 0, 0);
  };

  // ---- main loop: one barrier per K slice ---------------------------------
  // The fetch of slice k+1 starts at the top of slice k, into the LDS buffer
  // the last barrier freed (staged path: into registers, written to that
  // buffer just before the barrier).  Fragments are read one group of four
  // MFMA steps ahead; the last group's MFMAs run after the barrier, so they
  // cover the first LDS reads of the next slice.  A scheduling barrier keeps
  // the other groups' MFMAs above the slice barrier: left to itself the
  // compiler sinks most of them below it, which moves the wait for this
  // wave's DMA earlier in the slice (measured 0.3% slower at 4096^3).
  constexpr int NGW = T::NGW;
  const int g0 = kg * NGW;  // this wave's first step group of a slice
  Frag f0, f1;
  auto slice = [&](const float *cur, float *nxt, int kt) {
    const bool more = kt + 1 < nk;
    if (more) {
      if (kt + 2 == nk) set_offsets(ktail);
      fetch(nxt, kt + 1);
    }
#pragma unroll
    for (int g = 0; g < NGW; ++g) {
      Frag &fc = (g & 1) ? f1 : f0;
      Frag &fn = (g & 1) ? f0 : f1;
      if (g + 1 < NGW) {
        read_frag(cur, g0 + g + 1, fn);
        mma(fc);
      } else {
        __builtin_amdgcn_sched_barrier(0);
        if (more) commit(nxt);
        if constexpr (DMA) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMA landed
        __syncthreads();
        if (more) read_frag(nxt, g0, fn);
        mma(fc);
      }
    }
  };

  if (!SK || ke > kb) {
  if constexpr (DMA && T::P > 1) {
    // P slices per barrier.  Stage st is slices [st P, st P + P) in buffers
    // (st % 2) P .. (st % 2) P + P - 1.  The next stage's P fetches start at
    // the top of a stage (past the end of K they are masked: zeros into a
    // free buffer, and those slices then add exact zeros); at the end of the
    // stage every wave waits for its own DMA and one barrier publishes the
    // whole next stage.  Within a stage the last group of a slice reads the
    // first group of the next slice without a barrier (it has landed).
    constexpr int P = T::P;
    auto fetch_slice = [&](int ks) {
      if (ks == nk - 1) set_offsets(ktail);
      else if (ks == nk) set_offsets(0);
      fetch(lds + (ks % (2 * P)) * STAGE, ks);
    };
    const int nst = (nk + P - 1) / P;
    set_offsets(BK);
#pragma unroll
    for (int u = 0; u < P; ++u) fetch_slice(u);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if constexpr (SK) signal_pending();
    read_frag(lds, g0, f0);
    for (int st = 0; st < nst; ++st) {
      float *base = lds + (st & 1) * P * STAGE;
      float *nbase = lds + ((st + 1) & 1) * P * STAGE;
#pragma unroll
      for (int u = 0; u < P; ++u) fetch_slice((st + 1) * P + u);
#pragma unroll
      for (int u = 0; u < P; ++u) {
        const float *cur = base + u * STAGE;
#pragma unroll
        for (int g = 0; g < NGW; ++g) {
          Frag &fc = (g & 1) ? f1 : f0;
          Frag &fn = (g & 1) ? f0 : f1;
          if (g + 1 < NGW) {
            read_frag(cur, g0 + g + 1, fn);
            mma(fc);
          } else if (u + 1 < P) {
            read_frag(cur + STAGE, g0, fn);
            mma(fc);
          } else {
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next stage of this wave landed
            __syncthreads();
            if (st + 1 < nst) read_frag(nbase, g0, fn);
            mma(fc);
          }
        }
      }
    }
  } else {
    set_offsets(nk == 1 ? ktail : BK);
    fetch(lds, 0);
    commit(lds);
    if constexpr (DMA) __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if constexpr (SK) signal_pending();
    read_frag(lds, g0, f0);
    // With one K group and beta = 0, the last slice runs one row of blocks at
    // a time, and each finished row is scaled and stored while the next
    // row's MFMAs run: writing C overlaps the last slice instead of following
    // it.  Every block still takes the slice's steps in the same order.
    constexpr bool ROWS_LAST = T::KS == 1 && !SK && MF == 32;
    const bool rows_last = ROWS_LAST && a.beta == 0.0f;
    const int nreg = rows_last ? nk - 1 : nk;
    for (int kt = 0; kt < nreg; ++kt) {
      const int c = kt & 1;
      slice(lds + c * STAGE, lds + (c ^ 1) * STAGE, kt);
    }
    if constexpr (ROWS_LAST) {
      if (rows_last) {
        const float *cur = lds + ((nk - 1) & 1) * STAGE;
        constexpr int NS = NGW * 4;  // steps of a slice
        float bq[T::TN][NS];
#pragma unroll
        for (int g = 0; g < NGW; ++g)
#pragma unroll
          for (int j = 0; j < T::TN; ++j) {
            float q[4];
            read_b_blk(cur, g0 + g, j, q);
#pragma unroll
            for (int st = 0; st < 4; ++st) bq[j][g * 4 + st] = q[st];
          }
        float aq[2][NS];
        auto read_a_row = [&](int i, float(&r)[NS]) {
#pragma unroll
          for (int g = 0; g < NGW; ++g) {
            float q[4];
            read_a_blk(cur, g0 + g, i, q);
#pragma unroll
            for (int st = 0; st < 4; ++st) r[g * 4 + st] = q[st];
          }
        };
        const __amdgpu_buffer_rsrc_t rs_c = make_rsrc(Cg + (size_t)m0 * a.ldc + n0);
        float bj[T::TN];
        load_bias(bj);
        const bool fused = a.bias != nullptr || a.act != kActNone;
        read_a_row(0, aq[0]);
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
          if (i + 1 < T::TM) read_a_row(i + 1, aq[(i + 1) & 1]);
#pragma unroll
          for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int st = 0; st < NS; ++st)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(aq[i & 1][st], bq[j][st], acc[i][j],
                                                              0, 0, 0);
#pragma unroll
          for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int v = 0; v < T::ACCN; ++v) {
              float out = a.alpha * acc[i][j][v];
              if (fused) out = apply_act(out + bj[j], a.act);
              __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, out), rs_c, c_off(i, j, v),
                                                    0, 0);
            }
        }
        return;
      }
    }
  }
  }  // main loop

  // ---- K groups: groups 1.. park their sums in LDS, group 0 adds them -----
  // The last slice ended with a barrier after every LDS read of the loop, so
  // the buffers are free.  Layout: [group - 1][wave in group][block][v][lane].
  if constexpr (T::KS > 1) {
    constexpr int PER = T::TM * T::TN * T::ACCN * 64;  // floats per wave
    static_assert((T::KS - 1) * T::WT * PER <= 2 * STAGE, "K-group sums fit in the LDS buffers");
    if (kg > 0) {
      float *red = lds + ((kg - 1) * T::WT + wt) * PER + lane;
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
#pragma unroll
          for (int v = 0; v < T::ACCN; ++v) red[((i * T::TN + j) * T::ACCN + v) * 64] = acc[i][j][v];
    }
    __syncthreads();
    if (kg > 0) return;
#pragma unroll
    for (int q = 1; q < T::KS; ++q) {
      const float *red = lds + ((q - 1) * T::WT + wt) * PER + lane;
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
#pragma unroll
          for (int v = 0; v < T::ACCN; ++v) acc[i][j][v] += red[((i * T::TN + j) * T::ACCN + v) * 64];
    }
  }

  // ---- stream-K: a tile that several workgroups share ------------------------
  // Publish the raw partial tile with agent-scope atomic stores (written
  // through the XCD's L2), wait for them, count the arrival; the last
  // workgroup to arrive adds every segment's partial tile in K order (its
  // own included, reloaded like the others) and goes on to the epilogue.  A
  // first segment that more segments follow is counted later (pend_t).  No
  // release/acquire fences (they would write back and invalidate the whole
  // L2): every value that crosses workgroups is an agent-scope atomic.
  if constexpr (SK) {
    static_assert(T::KS == 1, "stream-K tiles have one K group");
    constexpr int PER = T::TM * T::TN * T::ACCN * 64;  // floats per wave
    constexpr int TILE = BM * BN;
    if (kb != 0 || ke != nk_tile) {
      if (ke > kb) {
        float *mine = sk.part + (size_t)slot * TILE + wave * PER + lane;
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
#pragma unroll
          for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int v = 0; v < T::ACCN; ++v)
              __hip_atomic_store(mine + ((i * T::TN + j) * T::ACCN + v) * 64, acc[i][j][v],
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!last_seg) {
          pend_t = t;
          return;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) {
          const unsigned before = __hip_atomic_fetch_add(&sk.cnt[t], 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
          int f = before == (unsigned)(nseg_of(t) - 1) ? 1 : 0;
          if (pend_t >= 0 && pend_before == (unsigned)(nseg_of(pend_t) - 1)) f |= 2;
          sk_last = f;
        }
        __syncthreads();
        const int f = sk_last;
        pend_done = true;
        pend_fix = (f & 2) != 0;
        if (!(f & 1)) return;
        asm volatile("" ::: "memory");
      }
      // Finish tile t: segment js belongs to logical workgroup gfirst + js
      // (its first segment when that workgroup's units start inside the
      // tile, else its last).  R segments' loads are in flight at a time,
      // added into acc strictly in K order.
      const int ipw = sk.ipw;
      const long long u0 = (long long)t * nk_tile;
      const int gfirst = (int)(u0 / ipw);
      const int nseg = nseg_of(t);
      constexpr int R = 2;
      for (int j0 = 0; j0 < nseg; j0 += R) {
        acc_t part[R][T::TM][T::TN];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (j0 + r < nseg) {
            const int g = gfirst + j0 + r;
            const int sl = 2 * g + ((long long)g * ipw >= u0 ? 0 : 1);
            const float *src = sk.part + (size_t)sl * TILE + wave * PER + lane;
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
              for (int j = 0; j < T::TN; ++j)
#pragma unroll
                for (int v = 0; v < T::ACCN; ++v)
                  part[r][i][j][v] = __hip_atomic_load(src + ((i * T::TN + j) * T::ACCN + v) * 64,
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (j0 + r < nseg) {
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
              for (int j = 0; j < T::TN; ++j)
                acc[i][j] = j0 + r == 0 ? part[r][i][j] : acc[i][j] + part[r][i][j];
          }
        }
      }
      if (tid == 0)
        __hip_atomic_store(&sk.cnt[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // ---- epilogue: C = act(alpha * acc + beta * C + bias[col]) ----------------
  // The bias and the activation are the fused elementwise chain of "GPU 基础
  // 原理", section "4.1 算子融合", applied in registers before the only store
  // of C.
  const __amdgpu_buffer_rsrc_t rs_c = make_rsrc(Cg + (size_t)m0 * a.ldc + n0);
  const float alpha = a.alpha, beta = a.beta;
  float bj[T::TN];  // this lane's bias value per block column
  load_bias(bj);
  const bool fused = a.bias != nullptr || a.act != kActNone;
  const int act = a.act;
  auto finish = [&](float out, int j) -> float { return fused ? apply_act(out + bj[j], act) : out; };
  if (beta != 0.0f) {
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
      for (int j = 0; j < T::TN; ++j) {
        float c0[T::ACCN];
#pragma unroll
        for (int v = 0; v < T::ACCN; ++v)
          c0[v] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_c, c_off(i, j, v), 0, 0));
#pragma unroll
        for (int v = 0; v < T::ACCN; ++v) {
          const float out = finish(alpha * acc[i][j][v] + beta * c0[v], j);
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, out), rs_c, c_off(i, j, v), 0, 0);
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
      for (int j = 0; j < T::TN; ++j)
#pragma unroll
        for (int v = 0; v < T::ACCN; ++v) {
          const float out = finish(alpha * acc[i][j][v], j);
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, out), rs_c, c_off(i, j, v), 0, 0);
        }
  }
  };  // run

  if constexpr (!SK) {
    // the logical id is the tile, walked in strips of group_m tile-rows
    int m0, n0;
    tile_origin(lid, m0, n0);
    run(m0, n0, 0, nk_tile, 0, 0, true);
  } else {
    // logical workgroup lid's units, split at tile boundaries into
    // segments; only the first and the last segment can be partial tiles
    const long long total = (long long)tiles_m * tiles_n * nk_tile;
    const long long ub = (long long)lid * sk.ipw;
    const long long ue = min(ub + sk.ipw, total);
    for (long long u = ub; u < ue;) {
      const int t = (int)(u / nk_tile);
      const int kb = (int)(u - (long long)t * nk_tile);
      const int ke = (int)min((long long)nk_tile, kb + (ue - u));
      int m0, n0;
      tile_origin(t, m0, n0);
      run(m0, n0, kb, ke, t, 2 * lid + (u == ub ? 0 : 1), u + (ke - kb) >= ue);
      u += ke - kb;
    }
    if (pend_t >= 0) {
      if (!pend_done) {
        // the last segment was a whole tile: its first barrier counted the
        // pending arrival; thread 0 holds the counter's old value
        if (tid == 0) sk_last = pend_before == (unsigned)(nseg_of(pend_t) - 1) ? 2 : 0;
        __syncthreads();
        pend_fix = (sk_last & 2) != 0;
      }
      if (pend_fix) {
        int m0, n0;
        tile_origin(pend_t, m0, n0);
        run(m0, n0, 0, 0, pend_t, 0, true);
      }
    }
  }
}

// Launch one tile shape for one operand-layout combination.
template <class T, bool TRANS_A, bool TRANS_B>
hipError_t launch(const GemmArgs &a, bool dma, int group_m, hipStream_t s) {
  const int tm = (a.M + T::BM - 1) / T::BM;
  const int tn = (a.N + T::BN - 1) / T::BN;
  const long long G = (long long)tm * tn;
  if (G > 0x7fffffffLL || a.batch > 65535) return hipErrorInvalidConfiguration;
  if (group_m < 1) group_m = 1;
  const dim3 grid((unsigned)G, (unsigned)a.batch);
  const SkArgs none = {0, nullptr, nullptr};
  if (dma)
    hipLaunchKernelGGL((sgemm_kernel<T, TRANS_A, TRANS_B, true>), grid, dim3(T::NT), 0, s, a, tm, tn,
                       group_m, none);
  else
    hipLaunchKernelGGL((sgemm_kernel<T, TRANS_A, TRANS_B, false>), grid, dim3(T::NT), 0, s, a, tm,
                       tn, group_m, none);
  return hipGetLastError();
}

// Stream-K launch of one tile shape: `groups` workgroups of ipw units each
// (the caller's plan: groups x ipw >= tiles x slices), one product.
template <class T, bool TRANS_A, bool TRANS_B>
hipError_t launch_sk(const GemmArgs &a, bool dma, int group_m, int groups, const SkArgs &sk,
                     hipStream_t s) {
  const int tm = (a.M + T::BM - 1) / T::BM;
  const int tn = (a.N + T::BN - 1) / T::BN;
  if (a.batch != 1 || a.k_total != 0 || groups < 1) return hipErrorInvalidValue;
  if (group_m < 1) group_m = 1;
  if (dma)
    hipLaunchKernelGGL((sgemm_kernel<T, TRANS_A, TRANS_B, true, true>), dim3(groups), dim3(T::NT),
                       0, s, a, tm, tn, group_m, sk);
  else
    hipLaunchKernelGGL((sgemm_kernel<T, TRANS_A, TRANS_B, false, true>), dim3(groups), dim3(T::NT),
                       0, s, a, tm, tn, group_m, sk);
  return hipGetLastError();
}

}  // namespace
}  // namespace fp32gemm

// The tile shapes the tuning sweep chooses from, in configuration order:
// (BM, BN, BK, WM, WN, K groups, K slices per barrier of the 128-bit path,
// workgroups per CU of the 128-bit path).  Each fits the gfx950 limits (LDS
// <= 160 KB per workgroup, <= 512 registers per lane); the occupancy column
// comes from the compiler's LDS and register counts.
#define FP32GEMM_TILES(X)             \
  X(256, 256, 32, 128, 64, 1, 1, 1, 32)  \
  X(256, 256, 16, 128, 64, 1, 1, 1, 32)  \
  X(256, 128, 32, 64, 64, 1, 1, 1, 32)   \
  X(128, 256, 32, 64, 64, 1, 1, 1, 32)   \
  X(128, 128, 32, 64, 32, 1, 1, 2, 32)   \
  X(256, 128, 32, 128, 64, 1, 1, 1, 32)  \
  X(256, 128, 16, 128, 64, 1, 1, 1, 32)  \
  X(128, 256, 32, 64, 128, 1, 1, 1, 32)  \
  X(128, 128, 32, 64, 64, 1, 1, 2, 32)   \
  X(128, 128, 16, 64, 64, 1, 1, 3, 32)   \
  X(64, 64, 32, 32, 32, 1, 1, 4, 32)     \
  X(64, 64, 32, 32, 32, 1, 2, 2, 32)     \
  X(64, 64, 32, 32, 32, 1, 4, 1, 32)     \
  X(64, 64, 32, 32, 32, 2, 2, 2, 32)     \
  X(32, 128, 32, 32, 32, 1, 1, 3, 32)    \
  X(64, 64, 32, 32, 32, 1, 1, 4, 16)     \
  X(96, 96, 32, 48, 48, 1, 1, 2, 16)     \
  X(32, 32, 32, 16, 16, 1, 2, 4, 16)     \
  X(32, 32, 32, 16, 16, 1, 4, 2, 16)     \
  X(64, 32, 32, 32, 16, 1, 2, 3, 16)
// The tiles with a stream-K form (one K group, one slice per barrier); the
// occupancy column is the stream-K kernel's own (its fix-up needs more
// registers than the plain kernel: the 128x128 form fits one workgroup per
// CU, the 64x64 form four, held there by its waves-per-SIMD attribute).
// The 256x256 tile is not among them: with the fix-up's partial tiles live
// its 8-wave form needs more than its 256 registers per lane and spills.
#define FP32GEMM_SK_TILES(X)             \
  X(128, 128, 32, 64, 32, 1, 1, 1, 32)   \
  X(64, 64, 32, 32, 32, 1, 1, 4, 32)
