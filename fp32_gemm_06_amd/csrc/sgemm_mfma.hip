// SGEMM C <- alpha A B + beta C on gfx950 with the fp32 matrix cores.
//
// The structure follows the tiling the pages build up step by step, mapped
// onto CDNA4 instead of Ampere:
//  * a workgroup owns a BM x BN tile of C and walks K in slices of BK
//    ("GPU 基础原理", section "4.2 分块": the sum over k regrouped by tiles);
//  * each K slice of A and B is staged through LDS with coalesced 128-bit
//    global loads ("GPU 基础原理", sections "4.3 合并加载" and the float4
//    discussion; "CUDA 矩阵乘法优化", section "7. Kernel 6: 向量化访存优化");
//  * LDS rows are padded so that the fragment reads are free of bank
//    conflicts ("GPU GEMM 优化完全拆解（一）", section "两种解法：Padding 与
//    线性化");
//  * each 64-lane wave owns a WM x WN sub-tile made of 32 x 32 blocks, the
//    CDNA4 counterpart of warp tiling with per-thread register blocks
//    ("CUDA 矩阵乘法优化", sections "6. Kernel 5" and "9. Kernel 10: 线程束级
//    分块"); the per-thread outer product becomes v_mfma_f32_32x32x2_f32,
//    which multiplies fp32 operands and accumulates in fp32;
//  * the next K slice is fetched into registers while the matrix cores work
//    on the current one, with two LDS buffers so that one barrier per slice
//    suffices (the double buffering named as future work in "11. 探索未尽与
//    总结", and the two-barrier rule of "GPU GEMM 优化完全拆解（一）",
//    section "分块的思想");
//  * tiles that overhang M, N or K are handled by zero-filling the operands
//    and masking the stores ("GPU 基础原理", section "最后一个考虑：分块的
//    量化"), using buffer loads whose out-of-range offsets return zero, so
//    interior and edge tiles run the same instruction stream.
//
// K ordering inside a slice.  For v_mfma_f32_32x32x2_f32 lane l supplies
// A[l % 32][k] and B[k][l % 32] with k = l / 32 of the instruction's pair.
// Any bijection between (step, lane half) and the BK values of k gives the
// same sum, so lane half h takes k = h * BK/2 + step.  A lane's A values for
// four consecutive steps are then contiguous in a k-major LDS row and come
// in with one ds_read_b128; B stays n-major (as in global memory) and each
// lane reads one float per step, 32 consecutive floats per lane half.
#include "common.h"

namespace fp32gemm {
namespace {

constexpr int kPadA = 4;   // floats appended to each k-row of the A tile
constexpr int kPadB = 4;   // floats appended to each n-row of the B tile
constexpr int kGapB = 32;  // floats between the two k-halves of the B tile

template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static constexpr int WAVES_N = BN / WN;
  static constexpr int WAVES = (BM / WM) * WAVES_N;
  static constexpr int NT = WAVES * 64;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int LDA_S = BK + kPadA;
  static constexpr int LDB_S = BN + kPadB;
  static constexpr int A_STAGE = BM * LDA_S;
  static constexpr int B_STAGE = BK * LDB_S + kGapB;
  static constexpr int STAGE = A_STAGE + B_STAGE;
  static constexpr int LDS_FLOATS = 2 * STAGE;
  static constexpr int A_VECS = BM * BK / 4;
  static constexpr int B_VECS = BK * BN / 4;
  static constexpr int NA = A_VECS / NT;
  static constexpr int NB = B_VECS / NT;
  static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0, "wave tiling");
  static_assert(BK % 8 == 0, "BK must be a multiple of 8");
  static_assert(A_VECS % NT == 0 && B_VECS % NT == 0, "loader mapping");
};

// B tile LDS offset of row r (a k index inside the slice).
template <class T>
__device__ __forceinline__ int b_row(int r) {
  return r * T::LDB_S + (r >= T::BK / 2 ? kGapB : 0);
}

template <class T, bool VEC>
__global__ void __launch_bounds__(T::NT)
sgemm_mfma(GemmArgs a, int tiles_m, int tiles_n, int group_m) {
  constexpr int BM = T::BM, BN = T::BN, BK = T::BK, NT = T::NT;
  __shared__ __attribute__((aligned(16))) float lds[T::LDS_FLOATS];

  // ---- which C tile: XCD-aware order --------------------------------------
  // Workgroups are handed to the 8 XCDs round-robin by id; renumber them so
  // that each XCD receives a contiguous range of logical ids, then walk the
  // tiles in column strips of group_m tile-rows so that the tiles an XCD
  // runs together share A and B panels in its L2.
  const int G = gridDim.x;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, per = G >> 3, extra = G & 7;
  const int lid = xcd * per + min(xcd, extra) + (bid >> 3);
  const int width = group_m * tiles_n;
  const int grp = lid / width;
  const int first_m = grp * group_m;
  const int gsz = min(tiles_m - first_m, group_m);
  const int within = lid - grp * width;
  const int m0 = (first_m + within % gsz) * BM;
  const int n0 = (within / gsz) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
  const int l32 = lane & 31, half = lane >> 5;

  const int rows = a.M - m0;  // rows of this tile inside C (may exceed BM)
  const int cols = a.N - n0;
  const int nk = (a.K + BK - 1) / BK;
  const int ktail = a.K - (nk - 1) * BK;  // valid k in the last slice, 1..BK

  floatx4 ra[T::NA], rb[T::NB];

  // Fetch K slice kt into registers; kvalid = number of valid k in it.
  auto load_slice = [&](int kt, int kvalid) {
    const __amdgpu_buffer_rsrc_t rs_a =
        make_rsrc(a.A + (size_t)m0 * a.lda + (size_t)kt * BK);
    const __amdgpu_buffer_rsrc_t rs_b =
        make_rsrc(a.B + (size_t)kt * BK * a.ldb + n0);
#pragma unroll
    for (int i = 0; i < T::NA; ++i) {
      const int s = tid + i * NT;
      const int r = s / (BK / 4), c = (s % (BK / 4)) * 4;
      if constexpr (VEC) {
        const bool ok = r < rows && c < kvalid;
        const uint32_t off = ok ? (uint32_t)(r * a.lda + c) * 4u : kOob;
        ra[i] = __builtin_amdgcn_raw_buffer_load_b128(rs_a, off, 0, 0);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = r < rows && c + e < kvalid;
          const uint32_t off = ok ? (uint32_t)(r * a.lda + c + e) * 4u : kOob;
          ra[i][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_a, off, 0, 0));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < T::NB; ++i) {
      const int s = tid + i * NT;
      const int r = s / (BN / 4), c = (s % (BN / 4)) * 4;
      if constexpr (VEC) {
        const bool ok = r < kvalid && c < cols;
        const uint32_t off = ok ? (uint32_t)(r * a.ldb + c) * 4u : kOob;
        rb[i] = __builtin_amdgcn_raw_buffer_load_b128(rs_b, off, 0, 0);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = r < kvalid && c + e < cols;
          const uint32_t off = ok ? (uint32_t)(r * a.ldb + c + e) * 4u : kOob;
          rb[i][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_b, off, 0, 0));
        }
      }
    }
  };

  auto store_a = [&](int buf) {
    float *As = lds + buf * T::STAGE;
#pragma unroll
    for (int i = 0; i < T::NA; ++i) {
      const int s = tid + i * NT;
      const int r = s / (BK / 4), c = (s % (BK / 4)) * 4;
      *reinterpret_cast<floatx4 *>(As + r * T::LDA_S + c) = ra[i];
    }
  };
  auto store_b = [&](int buf) {
    float *Bs = lds + buf * T::STAGE + T::A_STAGE;
#pragma unroll
    for (int i = 0; i < T::NB; ++i) {
      const int s = tid + i * NT;
      const int r = s / (BN / 4), c = (s % (BN / 4)) * 4;
      *reinterpret_cast<floatx4 *>(Bs + b_row<T>(r) + c) = rb[i];
    }
  };

  floatx16 acc[T::TM][T::TN];
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j) acc[i][j] = floatx16{};

  // Operand fragments of one group of four MFMA steps: A as one float4 per
  // 32-row block (four consecutive k of this lane's half), B as one float
  // per step and 32-column block.
  struct Frag {
    floatx4 a[T::TM];
    float b[4][T::TN];
  };
  auto read_frag = [&](int buf, int g, Frag &f) {
    const float *As = lds + buf * T::STAGE;
    const float *Bs = As + T::A_STAGE;
    const float *pa = As + (wm * T::WM + l32) * T::LDA_S + half * (BK / 2) + 4 * g;
    const float *pb = Bs + b_row<T>(half * (BK / 2)) + wn * T::WN + l32 + 4 * g * T::LDB_S;
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
      f.a[i] = *reinterpret_cast<const floatx4 *>(pa + i * 32 * T::LDA_S);
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int j = 0; j < T::TN; ++j) f.b[st][j] = pb[st * T::LDB_S + j * 32];
  };
  auto mma = [&](const Frag &f) {
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[i][st], f.b[st][j], acc[i][j], 0, 0, 0);
  };

  // ---- main loop: one barrier per K slice ---------------------------------
  // Fragments are read one group ahead of the MFMAs that use them.  The last
  // group of a slice is multiplied after the barrier, so its MFMAs cover the
  // latency of the first LDS reads of the next slice.  Slice k+1 is fetched
  // from global memory at the start of slice k and written to the other LDS
  // buffer in two parts while the MFMAs of slice k run (that buffer was last
  // read before the previous barrier), so the waves do not all write LDS at
  // once just before the barrier with the matrix cores idle.
  constexpr int NG = BK / 8;  // groups of four MFMA steps per slice
  static_assert(NG % 2 == 0, "fragment double buffering needs an even group count");
  constexpr int GA = NG >= 4 ? 1 : 0;       // group after which A is stored
  constexpr int GB = NG >= 4 ? 2 : NG - 1;  // group after which B is stored
  Frag f0, f1;
  load_slice(0, nk == 1 ? ktail : BK);
  store_a(0);
  store_b(0);
  __syncthreads();
  read_frag(0, 0, f0);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) load_slice(kt + 1, kt + 2 == nk ? ktail : BK);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      Frag &fc = (g & 1) ? f1 : f0;
      Frag &fn = (g & 1) ? f0 : f1;
      if (g + 1 < NG) {
        read_frag(cur, g + 1, fn);
        mma(fc);
        if (more && g == GA) store_a(cur ^ 1);
        if (more && g == GB) store_b(cur ^ 1);
      } else {
        if (more && GA == NG - 1) store_a(cur ^ 1);
        if (more && GB == NG - 1) store_b(cur ^ 1);
        __syncthreads();
        if (more) read_frag(cur ^ 1, 0, fn);
        mma(fc);
      }
    }
  }

  // ---- epilogue: C = alpha * acc + beta * C ------------------------------
  // Accumulator register v of lane l holds row 8*(v/4) + 4*(l/32) + v%4,
  // column l%32 of its 32 x 32 block.
  const __amdgpu_buffer_rsrc_t rs_c = make_rsrc(a.C + (size_t)m0 * a.ldc + n0);
  const float alpha = a.alpha, beta = a.beta;
  auto c_off = [&](int i, int j, int v) -> uint32_t {
    const int row = wm * T::WM + i * 32 + 8 * (v / 4) + 4 * half + (v % 4);
    const int col = wn * T::WN + j * 32 + l32;
    return (row < rows && col < cols) ? (uint32_t)(row * a.ldc + col) * 4u : kOob;
  };
  if (beta != 0.0f) {
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
      for (int j = 0; j < T::TN; ++j) {
        float c0[16];
#pragma unroll
        for (int v = 0; v < 16; ++v)
          c0[v] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_c, c_off(i, j, v), 0, 0));
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float out = alpha * acc[i][j][v] + beta * c0[v];
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, out), rs_c, c_off(i, j, v), 0, 0);
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
      for (int j = 0; j < T::TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float out = alpha * acc[i][j][v];
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, out), rs_c, c_off(i, j, v), 0, 0);
        }
  }
}

// ---------------------------------------------------------------------------
// 128-bit path: operands go from HBM straight into LDS.
//
// buffer_load_dwordx4 ... lds writes lane l's 16 bytes to LDS at base + 16 l,
// so one wave instruction fills 1 KB of LDS and needs no VGPR staging and no
// ds_write.  The A tile is stored with packed k-rows (BK floats) and its
// float4 chunks XOR-swizzled per row, which keeps the ds_read_b128 fragment
// reads free of bank conflicts without padding; the swizzle is applied on
// the global side by choosing which chunk each lane fetches.  B rows are
// packed with a 32-float gap between the two k-halves (the two lane halves
// of a fragment read then fall in different banks).  The DMA of slice k+1
// goes to the LDS buffer that the last barrier freed; every wave waits for
// its own DMA (vmcnt(0)) before the barrier that publishes the slice.
// ---------------------------------------------------------------------------
template <class T>
struct Dma {
  static constexpr int BM = T::BM, BN = T::BN, BK = T::BK;
  static constexpr int A_ST = BM * BK;        // floats of the A tile
  static constexpr int B_ST = BK * BN + 32;   // floats of the B tile (with the gap)
  static constexpr int STAGE = A_ST + B_ST;
  static constexpr int CPA = BK / 4;          // float4 chunks per A row
  static constexpr int RPA = 64 / CPA;        // A rows per wave instruction
  static constexpr int CPB = BN / 4;          // float4 chunks per B row
  static constexpr int RPB = 64 / CPB;        // B rows per wave instruction
  static constexpr int NIA = BM * BK / 256 / T::WAVES;  // A instructions per wave
  static constexpr int NIB = BK * BN / 256 / T::WAVES;  // B instructions per wave
  static_assert(BK == 16 || BK == 32, "swizzle defined for BK 16 and 32");
  static_assert(BN >= 64 && BN <= 256 && 64 % CPB == 0, "B rows per instruction");
  static_assert(BM * BK % (256 * T::WAVES) == 0 && BK * BN % (256 * T::WAVES) == 0,
                "whole DMA instructions per wave");
  static_assert((BK / 2) % RPB == 0, "a B instruction stays inside one k-half");
};

// Chunk swizzle of A row r (verified conflict-free for 8-lane/32-bank and
// 16-lane/64-bank ds_read_b128 service).
template <int BK>
__device__ __forceinline__ int a_swizzle(int r) {
  if constexpr (BK == 32) return (r & 7) ^ ((r >> 3) & 1);
  else return ((r >> 1) ^ (r >> 3)) & 3;
}

// One 16-byte-per-lane DMA from a buffer into LDS at dst + 16 * lane.  The
// body exists only in the device pass (the host pass cannot form an LDS
// address-space pointer, and the kernels' host stubs must still be emitted).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, float *dst, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) void lds_void_t;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)dst, 16, off, 0, 0, 0);
#else
  (void)rs; (void)dst; (void)off;
#endif
}

template <class T>
__global__ void __launch_bounds__(T::NT)
sgemm_mfma_dma(GemmArgs a, int tiles_m, int tiles_n, int group_m) {
  using D = Dma<T>;
  constexpr int BM = T::BM, BN = T::BN, BK = T::BK;
  __shared__ __attribute__((aligned(16))) float lds[2 * D::STAGE];

  // tile coordinates: same XCD-aware order as the staged kernel
  const int G = gridDim.x;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, per = G >> 3, extra = G & 7;
  const int lid = xcd * per + min(xcd, extra) + (bid >> 3);
  const int width = group_m * tiles_n;
  const int grp = lid / width;
  const int first_m = grp * group_m;
  const int gsz = min(tiles_m - first_m, group_m);
  const int within = lid - grp * width;
  const int m0 = (first_m + within % gsz) * BM;
  const int n0 = (within / gsz) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
  const int l32 = lane & 31, half = lane >> 5;

  const int rows = a.M - m0;
  const int cols = a.N - n0;
  const int nk = (a.K + BK - 1) / BK;
  const int ktail = a.K - (nk - 1) * BK;

  // This lane's source offsets (bytes from the slice's base) per DMA
  // instruction; kvalid masks the k range of the slice.
  uint32_t offa[D::NIA], offb[D::NIB];
  auto set_offsets = [&](int kvalid) {
#pragma unroll
    for (int q = 0; q < D::NIA; ++q) {
      const int r = (wave * D::NIA + q) * D::RPA + lane / D::CPA;
      const int k = 4 * ((lane % D::CPA) ^ a_swizzle<BK>(r));
      offa[q] = (r < rows && k < kvalid) ? (uint32_t)(r * a.lda + k) * 4u : kOob;
    }
#pragma unroll
    for (int q = 0; q < D::NIB; ++q) {
      const int k = (wave * D::NIB + q) * D::RPB + lane / D::CPB;
      const int c = (lane % D::CPB) * 4;
      offb[q] = (k < kvalid && c < cols) ? (uint32_t)(k * a.ldb + c) * 4u : kOob;
    }
  };
  auto dma_slice = [&](float *buf, int kt) {
    const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(a.A + (size_t)m0 * a.lda + (size_t)kt * BK);
    const __amdgpu_buffer_rsrc_t rs_b = make_rsrc(a.B + (size_t)kt * BK * a.ldb + n0);
#pragma unroll
    for (int q = 0; q < D::NIA; ++q)
      dma16(rs_a, buf + (wave * D::NIA + q) * 256, offa[q]);
#pragma unroll
    for (int q = 0; q < D::NIB; ++q) {
      const int rb = (wave * D::NIB + q) * D::RPB;
      dma16(rs_b, buf + D::A_ST + rb * BN + (rb >= BK / 2 ? 32 : 0), offb[q]);
    }
  };

  floatx16 acc[T::TM][T::TN];
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j) acc[i][j] = floatx16{};

  struct Frag {
    floatx4 a[T::TM];
    float b[4][T::TN];
  };
  const int ar = wm * T::WM + l32;                // this lane's A row in block 0
  const int asw = a_swizzle<BK>(ar);              // same for every 32-row block
  auto read_frag = [&](const float *buf, int g, Frag &f) {
    const int chunk = (half * (BK / 8) + g) ^ asw;
    const float *pa = buf + ar * BK + 4 * chunk;
    const float *pb = buf + D::A_ST + (half * (BK / 2) + 4 * g) * BN + half * 32 + wn * T::WN + l32;
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
      f.a[i] = *reinterpret_cast<const floatx4 *>(pa + i * 32 * BK);
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int j = 0; j < T::TN; ++j) f.b[st][j] = pb[st * BN + j * 32];
  };
  auto mma = [&](const Frag &f) {
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[i][st], f.b[st][j], acc[i][j], 0, 0, 0);
  };

  constexpr int NG = BK / 8;
  static_assert(NG % 2 == 0, "fragment double buffering needs an even group count");
  Frag f0, f1;
  // One K slice: the DMA of slice kt+1 into `nxt` starts first; fragments are
  // read one group ahead; the last group is multiplied after the barrier.
  auto slice = [&](const float *cur, float *nxt, int kt) {
    const bool more = kt + 1 < nk;
    if (more) {
      if (kt + 2 == nk) set_offsets(ktail);
      dma_slice(nxt, kt + 1);
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      Frag &fc = (g & 1) ? f1 : f0;
      Frag &fn = (g & 1) ? f0 : f1;
      if (g + 1 < NG) {
        read_frag(cur, g + 1, fn);
        mma(fc);
      } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMA has landed
        __syncthreads();
        if (more) read_frag(nxt, 0, fn);
        mma(fc);
      }
    }
  };

  set_offsets(nk == 1 ? ktail : BK);
  dma_slice(lds, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  read_frag(lds, 0, f0);
  for (int kt = 0; kt < nk; ++kt) {
    const int c = kt & 1;
    slice(lds + c * D::STAGE, lds + (c ^ 1) * D::STAGE, kt);
  }

  // epilogue (same as the staged kernel)
  const __amdgpu_buffer_rsrc_t rs_c = make_rsrc(a.C + (size_t)m0 * a.ldc + n0);
  const float alpha = a.alpha, beta = a.beta;
  auto c_off = [&](int i, int j, int v) -> uint32_t {
    const int row = wm * T::WM + i * 32 + 8 * (v / 4) + 4 * half + (v % 4);
    const int col = wn * T::WN + j * 32 + l32;
    return (row < rows && col < cols) ? (uint32_t)(row * a.ldc + col) * 4u : kOob;
  };
  if (beta != 0.0f) {
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
      for (int j = 0; j < T::TN; ++j) {
        float c0[16];
#pragma unroll
        for (int v = 0; v < 16; ++v)
          c0[v] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_c, c_off(i, j, v), 0, 0));
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float out = alpha * acc[i][j][v] + beta * c0[v];
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, out), rs_c, c_off(i, j, v), 0, 0);
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
      for (int j = 0; j < T::TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float out = alpha * acc[i][j][v];
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, out), rs_c, c_off(i, j, v), 0, 0);
        }
  }
}

template <class T>
hipError_t launch(const GemmArgs &a, bool vec4, int group_m, hipStream_t s) {
  const int tm = (a.M + T::BM - 1) / T::BM;
  const int tn = (a.N + T::BN - 1) / T::BN;
  const long long G = (long long)tm * tn;
  if (G > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (group_m < 1) group_m = 1;
  if (vec4)
    hipLaunchKernelGGL((sgemm_mfma_dma<T>), dim3((unsigned)G), dim3(T::NT), 0, s, a, tm, tn, group_m);
  else
    hipLaunchKernelGGL((sgemm_mfma<T, false>), dim3((unsigned)G), dim3(T::NT), 0, s, a, tm, tn, group_m);
  return hipGetLastError();
}

// OCC: workgroups per CU of the 128-bit kernel, from its LDS size (160 KB per
// CU) and register count (512 per SIMD lane, waves spread over 4 SIMDs), as
// reported by the compiler for gfx950.
#define FP32GEMM_CFG(BM, BN, BK, WM, WN, OCC)                                             \
  {#BM "x" #BN "x" #BK "_w" #WM "x" #WN, BM, BN, BK, WM, WN, Tile<BM, BN, BK, WM, WN>::NT, \
   (int)(2 * Dma<Tile<BM, BN, BK, WM, WN>>::STAGE * sizeof(float)), OCC,                   \
   &launch<Tile<BM, BN, BK, WM, WN>>}

}  // namespace

// The tile shapes the tuning sweep chooses from.  Each one fits the gfx950
// limits: LDS <= 160 KB per workgroup, at most 512 registers per lane.
const GemmConfig *gemm_configs(int *count) {
  static const GemmConfig table[] = {
      FP32GEMM_CFG(256, 256, 32, 128, 64, 1),  // 131 KB LDS
      FP32GEMM_CFG(256, 256, 16, 128, 64, 1),  // 192 VGPRs x 2 waves/SIMD per workgroup
      FP32GEMM_CFG(256, 128, 32, 64, 64, 1),   // 99 KB LDS
      FP32GEMM_CFG(128, 256, 32, 64, 64, 1),   // 99 KB LDS
      FP32GEMM_CFG(128, 128, 32, 64, 32, 2),   // 66 KB LDS
      FP32GEMM_CFG(256, 128, 32, 128, 64, 1),  // 99 KB LDS
      FP32GEMM_CFG(256, 128, 16, 128, 64, 1),  // 292 VGPRs: one wave per SIMD
      FP32GEMM_CFG(128, 256, 32, 64, 128, 1),  // 99 KB LDS
      FP32GEMM_CFG(128, 128, 32, 64, 64, 2),   // 66 KB LDS
      FP32GEMM_CFG(128, 128, 16, 64, 64, 3),   // 33 KB LDS, 164 VGPRs: 3 waves/SIMD
      FP32GEMM_CFG(64, 64, 32, 32, 32, 4),     // 33 KB LDS
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

}  // namespace fp32gemm
