// Skinny product Y[M x N] <- alpha X[M x K] W[K x N] + beta Y for 9 <= M <= 128:
// several decode sequences at once against a weight matrix.
//
// Like M <= 8 ("GPU GEMM 优化完全拆解（一）", section "LLM 推理本质上是 GEMM 的
// 串联": the decode GEMMs stream W once from HBM), the time is set by the
// weight read until M reaches about a hundred, but from M ~ 16 on the vector
// ALUs of the column-stripe GEMV (4 M FMAs per 16 bytes of W) fall behind
// that stream, and the tiled kernel has too few tiles (64 for M <= 64 at
// N = 4096) to keep the memory system busy.  This kernel keeps the GEMV's
// memory pattern and does the arithmetic on the matrix cores:
//
//  * a workgroup owns a stripe of 16 NB columns of W (NB = 1, 2, 4; the
//    library picks the width whose grid needs the fewest rounds of 256)
//    over the whole of K, and its 8 waves split each pass of ROWS rows of K;
//    with 16-column stripes the two of a 128-byte line run on one XCD;
//  * W values go straight from buffer loads into the B operand of
//    v_mfma_f32_16x16x4_f32 (lane l holds B[k = l / 16][n = l % 16]).  The
//    sum over a pass is the same under any assignment of its k to (step,
//    lane quarter); step g of lane quarter q takes k = 16 (g / 4) + 4 q +
//    g % 4 of the wave's part of the pass, so four consecutive steps of a
//    lane are four consecutive k and the four quarters cover 16 consecutive k;
//  * W stored K x N: a wave instruction reads four 64-byte row segments;
//    stored N x K (TB): lane (q, c) reads stored rows n0 + 16 e + c along k
//    (column block e), and a wave instruction reads 64 contiguous bytes of
//    each of 16 consecutive rows;
//  * X is staged per pass in LDS as [m][k] rows with a stride of ROWS + 8
//    floats; one ds_read_b128 holds the A operand of four consecutive steps.
//    With one row block (and 16-byte aligned rows) a wave can instead load
//    its own part of X straight into registers, which needs no LDS and no
//    barrier between passes (see XR below).
//    With a stride of ROWS + 4 the counters showed about two bank-conflict
//    cycles per LDS instruction, with ROWS + 8 one in seventeen (ROWS + 16
//    and + 20 as many as + 4); the time did not change;
//  * M up to 16 MB rows, MB blocks of 16 sharing each W value; W runs D
//    passes deep in registers and X one pass ahead (two LDS buffers or two
//    register sets),
//    with the same branch-free masking as the GEMV: rows of X past M and
//    rows of W past K (or N) read zeros through an out-of-range buffer offset;
//  * the waves' partial sums are added in LDS in wave order: the result does
//    not depend on timing.
#include "common.h"

namespace fp32gemm {
namespace {

constexpr int kSkWaves = 8;
constexpr int kSkThreads = kSkWaves * 64;

constexpr int pow2_floor(int v) {
  int p = 1;
  while (2 * p <= v) p *= 2;
  return p;
}

template <int E> struct Vec { typedef float type __attribute__((ext_vector_type(E))); };
template <> struct Vec<1> { typedef float type; };

// One raw buffer load of E floats (E = 1, 2, 4) at voffset + soffset bytes.
template <int E>
__device__ __forceinline__ typename Vec<E>::type load_vec(__amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                                         int soff) {
  if constexpr (E == 4)
    return __builtin_bit_cast(typename Vec<4>::type,
                              __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0));
  else if constexpr (E == 2)
    return __builtin_bit_cast(typename Vec<2>::type,
                              __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0));
  else
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0));
}

template <int E>
__device__ __forceinline__ float elem(const typename Vec<E>::type &v, int e) {
  if constexpr (E == 1)
    return v;
  else
    return v[e];
}

// MB: blocks of 16 rows of X (M <= 16 MB).  NB: column blocks of 16 per
// workgroup; lane (q, c) loads NB consecutive columns n0 + NB c .. + NB - 1
// of a row of W, and column block e of the MFMA takes element e, so its
// column c stands for n0 + NB c + e.  TA: op(A) = A^T (X stored K x M).
// XV: float4 loads of X (op(A) = A, 16-byte aligned rows, K % 4 == 0).
// TB: op(B) = B^T (W stored N x K, a linear layer's weight): lane (q, c)
// reads stored rows n0 + 16 e + c along k, WV floats at a time (4 when the
// rows are 16-byte aligned and K % 4 == 0), each float one MFMA step; column
// c of block e is then stripe column 16 e + c.
template <int MB, int NB, bool TA, bool XV, bool TB = false, int WV = 1>
__global__ void __launch_bounds__(kSkThreads)
skinny_kernel(GemmArgs a) {
  constexpr int MR = 16 * MB;               // row capacity of X
  constexpr int CW = 16 * NB;               // columns of W per workgroup
  // Rows of K per pass: the power of two at or below 1024 / (MB NB), halved
  // when MB NB <= 2, where a shorter pass gets W and X moving sooner (4096^2:
  // M = 32, W stored N x K, 26.2 -> 24.1 us; M = 16, W stored K x N, 22.6 ->
  // 21.5; with more blocks half the rows made M = 64 slower), and at least
  // 128, which keeps four MFMA steps per wave and pass.
  constexpr int ROWS_FIT = pow2_floor((MB * NB <= 2 ? 512 : 1024) / (MB * NB));
  constexpr int ROWS = ROWS_FIT < 128 ? 128 : ROWS_FIT;
  constexpr int RW = ROWS / kSkWaves;       // rows per wave per pass
  constexpr int G = RW / 4;                 // MFMA steps per wave per pass (rows per lane quarter)
  constexpr int SK = ROWS + 8;              // LDS row stride of the X chunk, in floats
  // accumulator sets: with few independent blocks, consecutive steps
  // alternate between sets so that no MFMA waits on the one before it
  constexpr int NA = MB * NB >= 4 ? 1 : 4 / (MB * NB);
  // X straight into registers (op(A) = A, float4 loads): each wave multiplies
  // only its own RW rows of K of a pass, so its X values need no sharing
  // through LDS and the passes need no barrier.  Taken for one row block over
  // W stored N x K (4096^2: M = 9 20.0 -> 17.3 us, M = 16 19.9 -> 19.1) and
  // on 64-column stripes over W stored K x N (N = 11008, M = 9: 41.8 -> 38.8);
  // with more blocks the scattered 16-byte X loads cost more than the staging
  // saves (M = 64: 33.8 -> 38.8 us), and on narrower stripes over W stored
  // K x N it was mixed (M = 16 at 4096^2: 21.4 -> 22.6; at 8192^2 27.3 ->
  // 28.4).
  constexpr bool XR = !TA && XV && MB == 1 && (TB || NB == 4);
  constexpr int XBUF = XR ? 0 : 2 * MR * SK, RED = kSkWaves * MR * CW;
  static_assert(G % 4 == 0, "A fragments are read four steps at a time");
  static_assert(!TA || kSkThreads % MR == 0,
                "op(A) = A^T stages whole columns of X per thread group");
  static_assert(!TB || G % WV == 0, "stored-transposed W: whole vectors per pass");
  static_assert((XBUF > RED ? XBUF : RED) * 4 <= 160 * 1024, "fits in LDS");
  __shared__ __attribute__((aligned(16))) float xs[XBUF > RED ? XBUF : RED];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, c = lane & 15;

  // (batch entry, stripe) from the linear workgroup id; with 16-column
  // stripes the two of a 128-byte line run on one XCD (id % 8)
  const int GX = gridDim.x;
  const long long L = (long long)blockIdx.y * GX + blockIdx.x;
  const long long T = (long long)gridDim.y * GX;
  const long long w = L < (T & ~15LL) ? 2 * (8 * ((L >> 3) >> 1) + (L & 7)) + ((L >> 3) & 1) : L;
  const long long bz = w / GX;
  const int cb = (int)(w - bz * GX);
  a.A += bz * a.sA;
  a.B += bz * a.sB;
  a.C += bz * a.sC;
  const int n0 = cb * CW;
  // NB > 1: N % NB == 0, so a lane's NB columns are all inside N or all past it
  const bool col_ok = n0 + NB * c < a.N;  // K x N layout
  const int K = a.K;

  // W at k = 16 (g / 4) + 4 q + g % 4 of the wave's part of the pass (the
  // wave's first row is the buffer base): 4 q in the per-lane offset, the
  // rest in the scalar offset.  Stored transposed: stored row n0 + 16 e + c
  // for column block e, WV consecutive k per load.
  constexpr int WL = TB ? G / WV * NB : G;  // W loads per wave per pass
  typedef typename Vec<TB ? WV : NB>::type wload_t;
  // stripe column of element (block e, lane column c) of the MFMA output
  auto col_of = [](int e, int cc) { return TB ? 16 * e + cc : NB * cc + e; };
  auto kstep = [](int g) { return 16 * (g / 4) + g % 4; };  // k of step g, lane quarter 0
  // Per-lane offsets.  The masks combine their conditions with "&": a
  // short-circuit "col_ok && k < K" let LLVM branch around duplicated loads,
  // each branch with a vmcnt(0) wait.  Stored N x K, the offset of column
  // block e is already kOob for stored rows past N (measured faster there);
  // stored K x N, the column test stays in each load's mask (folding it into
  // the offset cost 11% at N = 11008, M = 32).
  const uint32_t w_off = TB ? ((uint32_t)c * (uint32_t)a.ldb + (uint32_t)(4 * q)) * 4u
                            : ((uint32_t)(4 * q) * (uint32_t)a.ldb + (uint32_t)(NB * c)) * 4u;
  uint32_t w_lane[NB];
#pragma unroll
  for (int e = 0; e < NB; ++e) w_lane[e] = n0 + 16 * e + c < a.N ? w_off : kOob;
  auto load_w = [&](wload_t (&wv)[WL], int k0) {
    const int r0 = k0 + wave * RW;
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(TB ? a.B + (size_t)n0 * a.ldb + r0 : a.B + (size_t)r0 * a.ldb + n0);
#pragma unroll
    for (int l = 0; l < WL; ++l) {
      if constexpr (TB) {
        // load l: column block e = l / (WL / NB), steps (l % (WL / NB)) WV ..
        // + WV - 1, so a row's chunks are requested back to back.
        // WV == 4: K % 4 == 0 and kk + 4 q is a multiple of 4, so the four k
        // are all inside K or all past it
        const int e = l / (WL / NB), kk = kstep(l % (WL / NB) * WV);
        wv[l] = load_vec<WV>(rw, r0 + 4 * q + kk < K ? w_lane[e] : kOob,
                             (16 * e * a.ldb + kk) * 4);
      } else {
        // load l: step l, the lane's NB columns
        const int kk = kstep(l);
        wv[l] = load_vec<NB>(rw, (col_ok & (r0 + 4 * q + kk < K)) ? w_off : kOob,
                             kk * a.ldb * 4);
      }
    }
  };
  // the B operand of step g, column block e
  auto b_of = [&](const wload_t (&wv)[WL], int g, int e) -> float {
    if constexpr (TB)
      return elem<WV>(wv[e * (WL / NB) + g / WV], g % WV);
    else
      return elem<NB>(wv[g], e);
  };

  // X of the pass at k0: MR rows of ROWS values, consecutive threads along k
  // (X stored M x K) or along m (stored K x M) so the reads are coalesced.
  // Load j of a thread covers element (m_l + m_j, k_l + k_j): a per-lane part
  // and a part that is the same for every lane.
  static_assert(!(TA && XV), "float4 X loads only for op(A) = A");
  constexpr int XE = XV ? 4 : 1;                     // floats per load
  constexpr int P = kSkThreads * XE;                 // floats per load round
  constexpr int XP = MR * ROWS / P;                  // loads per thread
  static_assert(MR * ROWS % P == 0, "X loads divide evenly");
  typedef typename Vec<XE>::type xvec_t;
  int m_l, k_l;
  if constexpr (TA) {
    m_l = tid % MR;
    k_l = tid / MR;
  } else if constexpr (P % ROWS == 0) {
    m_l = tid * XE / ROWS;
    k_l = tid * XE % ROWS;
  } else {
    m_l = 0;
    k_l = tid * XE;
  }
  auto x_part = [&](int j, int &m_j, int &k_j) {
    if constexpr (TA) {
      m_j = 0;
      k_j = j * (kSkThreads / MR);
    } else if constexpr (P % ROWS == 0) {
      m_j = j * (P / ROWS);
      k_j = 0;
    } else {
      m_j = j / (ROWS / P);
      k_j = (j % (ROWS / P)) * P;
    }
  };
  const uint32_t x_lane = (TA ? (uint32_t)k_l * (uint32_t)a.lda + (uint32_t)m_l
                               : (uint32_t)m_l * (uint32_t)a.lda + (uint32_t)k_l) * 4u;
  auto load_x = [&](xvec_t (&xv)[XP], int k0) {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(TA ? a.A + (size_t)k0 * a.lda : a.A + k0);
#pragma unroll
    for (int j = 0; j < XP; ++j) {
      int m_j, k_j;
      x_part(j, m_j, k_j);
      // XV: K % 4 == 0, so a float4 is all inside K or all past it
      const bool ok = (m_l + m_j < a.M) & (k0 + k_l + k_j < K);  // no short circuit
      const int so = (TA ? k_j * a.lda + m_j : m_j * a.lda + k_j) * 4;
      xv[j] = load_vec<XE>(rx, ok ? x_lane : kOob, so);
    }
  };
  auto store_x = [&](const xvec_t (&xv)[XP], int buf) {
    float *base = &xs[buf * MR * SK + m_l * SK + k_l];
#pragma unroll
    for (int j = 0; j < XP; ++j) {
      int m_j, k_j;
      x_part(j, m_j, k_j);
      *reinterpret_cast<xvec_t *>(base + m_j * SK + k_j) = xv[j];
    }
  };

  floatx4 acc[NA][MB][NB];
#pragma unroll
  for (int s = 0; s < NA; ++s)
#pragma unroll
    for (int j = 0; j < MB; ++j)
#pragma unroll
      for (int e = 0; e < NB; ++e) acc[s][j][e] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  // X in registers: lane (q, c) loads X[16 j + c][k0 + wave RW + 16 t + 4 q
  // .. + 3] for block j and step group t, the A operand of four steps.
  typedef floatx4 xq_t[MB][G / 4 > 0 ? G / 4 : 1];
  const uint32_t xq_lane = ((uint32_t)c * (uint32_t)a.lda + (uint32_t)(4 * q)) * 4u;
  auto load_xq = [&](xq_t &xv, int k0) {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.A + k0 + wave * RW);
#pragma unroll
    for (int j = 0; j < MB; ++j)
#pragma unroll
      for (int t = 0; t < G / 4; ++t) {
        // K % 4 == 0 here, so a float4 is all inside K or all past it
        const bool ok = (c + 16 * j < a.M) & (k0 + wave * RW + 16 * t + 4 * q < K);
        xv[j][t] = load_vec<4>(rx, ok ? xq_lane : kOob, (16 * j * a.lda + 16 * t) * 4);
      }
  };

  // step g = 4 t + s of this lane: A = X[16 j + c][wave RW + 16 t + 4 q + s],
  // B = element e of the W value of step g
  auto compute = [&](const wload_t (&wv)[WL], int buf, const xq_t &xv) {
    const float *xb = &xs[XR ? 0 : buf * MR * SK + c * SK + wave * RW + 4 * q];
#pragma unroll
    for (int t = 0; t < G / 4; ++t) {
      floatx4 av[MB];
#pragma unroll
      for (int j = 0; j < MB; ++j)
        av[j] = XR ? xv[j][t] : *reinterpret_cast<const floatx4 *>(xb + 16 * j * SK + 16 * t);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int e = 0; e < NB; ++e)
#pragma unroll
          for (int j = 0; j < MB; ++j) {
            floatx4 &d = acc[(4 * t + s) % NA][j][e];
            d = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j][s], b_of(wv, 4 * t + s, e), d, 0, 0, 0);
          }
    }
  };

  // W runs D passes deep (D register sets), X one pass ahead through the two
  // LDS buffers.  A pass is ROWS rows, fewer as MB grows, and deeper sets
  // keep more bytes in flight: 4096^2, M = 128 went 63.9 -> 58.0 us (stored
  // N x K) and 63.8 -> 59.6 (stored K x N).  vmcnt retires loads in issue
  // order, so the wait for a pass's staged X also waits for every older W
  // load; stored K x N with MB = 2 a pass has 4 NB times as many W loads as
  // stored N x K, and depth 4 there only added waits (M = 32: 24.8 -> 27.0
  // us).  A wave keeps at most 63 loads in flight, which bounds D.
  constexpr int D = MB == 1 || (MB == 2 && !TB) ? 2 : MB <= 4 ? 4 : 8;
  static_assert(D % 2 == 0, "pass parity selects the X buffer");
  wload_t wr[D][WL];
  if constexpr (XR) {
    // X one pass ahead in two register sets, W D passes deep; no barrier
    xq_t xq[2];
    load_xq(xq[0], 0);
#pragma unroll
    for (int p = 0; p + 1 < D; ++p) load_w(wr[p], p * ROWS);
    for (int k0 = 0; k0 < K; k0 += D * ROWS) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const int kp = k0 + u * ROWS;
        load_xq(xq[(u + 1) % 2], kp + ROWS);
        load_w(wr[(u + D - 1) % D], kp + (D - 1) * ROWS);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (D > 2) {
          if (kp < K) compute(wr[u], 0, xq[u % 2]);
        } else {
          compute(wr[u], 0, xq[u % 2]);  // at most one pass past K, on zeros
        }
      }
    }
  } else {
    xvec_t xr[XP];
    xq_t none;
    load_x(xr, 0);
#pragma unroll
    for (int p = 0; p + 1 < D; ++p) load_w(wr[p], p * ROWS);
    store_x(xr, 0);
    __syncthreads();
    // The scheduling barriers keep each prefetch ahead of the compute that
    // waits on an earlier pass.  Passes run in groups of D; a pass that starts
    // past K (only in the last group) skips its multiply, its loads read zeros.
    for (int k0 = 0; k0 < K; k0 += D * ROWS) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const int kp = k0 + u * ROWS;
        load_x(xr, kp + ROWS);
        load_w(wr[(u + D - 1) % D], kp + (D - 1) * ROWS);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (D > 2) {
          if (kp < K) compute(wr[u], u % 2, none);
        } else {
          compute(wr[u], u % 2, none);  // at most one pass past K, on zeros
        }
        store_x(xr, (u + 1) % 2);
        __syncthreads();
      }
    }
  }

  // Partial sums: accumulator sets in order, then the waves in wave order
  // through LDS (the X buffers are free: the loop ended on a barrier).
  // Output layout of v_mfma_f32_16x16x4_f32: lane (q, c), element r holds
  // D[4 q + r][c]; column c of block e is stripe column col_of(e, c).
  float *red = xs;  // [wave][MR][CW]
#pragma unroll
  for (int j = 0; j < MB; ++j)
#pragma unroll
    for (int e = 0; e < NB; ++e) {
      floatx4 v = acc[0][j][e];
#pragma unroll
      for (int s = 1; s < NA; ++s) v += acc[s][j][e];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        red[(wave * MR + 16 * j + 4 * q + r) * CW + col_of(e, c)] = v[r];
    }
  __syncthreads();
  const float alpha = a.alpha, beta = a.beta;
  for (int o = tid; o < MR * CW; o += kSkThreads) {
    const int m = o / CW, cc = o % CW;
    if (m >= a.M || n0 + cc >= a.N) continue;
    float s = red[o];
#pragma unroll
    for (int w2 = 1; w2 < kSkWaves; ++w2) s += red[w2 * MR * CW + o];
    float *y = a.C + (size_t)m * a.ldc + n0 + cc;
    float out = alpha * s;
    if (beta != 0.0f) out += beta * *y;
    if (a.bias) out += a.bias[n0 + cc];
    *y = apply_act(out, a.act);
  }
}

template <int MB, int NB, bool TB = false, int WV = 1>
hipError_t launch_mb(const GemmArgs &a, int transA, bool xv, hipStream_t s) {
  const long long blocks = ((long long)a.N + 16 * NB - 1) / (16 * NB);
  if (blocks > 0x7fffffffLL || a.batch > 65535) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks, (unsigned)a.batch), block(kSkThreads);
  if (transA) {
    // 3, 5, 6 or 7 row blocks run op(A) = A only (their X staging for A^T
    // would not divide evenly between the threads)
    if constexpr (kSkThreads % (16 * MB) == 0)
      hipLaunchKernelGGL((skinny_kernel<MB, NB, true, false, TB, WV>), grid, block, 0, s, a);
    else
      return hipErrorInvalidValue;
  } else if (xv)
    hipLaunchKernelGGL((skinny_kernel<MB, NB, false, true, TB, WV>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((skinny_kernel<MB, NB, false, false, TB, WV>), grid, block, 0, s, a);
  return hipGetLastError();
}

// W stored N x K: float4 loads along k when its rows are 16-byte aligned.
template <int MB, int NB>
hipError_t launch_mb_tb(const GemmArgs &a, int transA, bool xv, hipStream_t s) {
  const bool wv4 = (uintptr_t)a.B % 16 == 0 && a.ldb % 4 == 0 && a.K % 4 == 0 &&
                   (a.batch == 1 || a.sB % 4 == 0);
  return wv4 ? launch_mb<MB, NB, true, 4>(a, transA, xv, s)
             : launch_mb<MB, NB, true, 1>(a, transA, xv, s);
}

// NB column blocks of 16 per workgroup; M <= 16 MB with MB * NB <= 16.
template <int NB>
hipError_t launch_nb(const GemmArgs &a, int transA, hipStream_t s) {
  if (a.M < 1 || a.M > 256 / NB || (transA && a.lda > (1 << 17))) return hipErrorInvalidValue;
  // NB > 1: W rows read NB floats at a time (B 4 NB-byte aligned, N and ldb
  // multiples of NB); otherwise the 16-column kernel runs
  if (NB > 1 && ((uintptr_t)a.B % (4 * NB) != 0 || a.N % NB != 0 || a.ldb % NB != 0 ||
                 (a.batch > 1 && a.sB % NB != 0)))
    return launch_nb<1>(a, transA, s);
  // float4 loads of X need 16-byte aligned rows and whole float4s inside K
  const bool xv = !transA && (uintptr_t)a.A % 16 == 0 && a.lda % 4 == 0 && a.K % 4 == 0 &&
                  (a.batch == 1 || a.sA % 4 == 0);
  if (a.M <= 16) return launch_mb<1, NB>(a, transA, xv, s);
  if constexpr (NB <= 4) {
    if (a.M <= 32) return launch_mb<2, NB>(a, transA, xv, s);
    if (a.M <= 48 && !transA) return launch_mb<3, NB>(a, transA, xv, s);
    if (a.M <= 64) return launch_mb<4, NB>(a, transA, xv, s);
  }
  if constexpr (NB <= 2) {
    if (a.M <= 80 && !transA) return launch_mb<5, NB>(a, transA, xv, s);
    if (a.M <= 96 && !transA) return launch_mb<6, NB>(a, transA, xv, s);
    if (a.M <= 112 && !transA) return launch_mb<7, NB>(a, transA, xv, s);
    return launch_mb<8, NB>(a, transA, xv, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool skinny_supported(const GemmArgs &a, int transA) {
  // op(A) = A^T: the offsets of a pass (ROWS <= 1024 rows of lda floats)
  // stay within 31 bits up to lda = 2^17
  return a.M >= 1 && a.M <= kSkinnyMaxRows && (!transA || a.lda <= (1 << 17));
}

hipError_t launch_skinny16(const GemmArgs &a, int transA, hipStream_t s) {
  return launch_nb<1>(a, transA, s);
}

// W stored N x K, 16 NB stored rows per workgroup (M <= 16 MB, MB NB <= 16).
template <int NB>
hipError_t launch_tb_nb(const GemmArgs &a, int transA, hipStream_t s) {
  if (a.M < 1 || a.M > 256 / NB || (transA && a.lda > (1 << 17))) return hipErrorInvalidValue;
  const bool xv = !transA && (uintptr_t)a.A % 16 == 0 && a.lda % 4 == 0 && a.K % 4 == 0 &&
                  (a.batch == 1 || a.sA % 4 == 0);
  if (a.M <= 16) return launch_mb_tb<1, NB>(a, transA, xv, s);
  if constexpr (NB <= 4) {
    if (a.M <= 32) return launch_mb_tb<2, NB>(a, transA, xv, s);
    if (a.M <= 48 && !transA) return launch_mb_tb<3, NB>(a, transA, xv, s);
    if (a.M <= 64) return launch_mb_tb<4, NB>(a, transA, xv, s);
  }
  if constexpr (NB <= 2) {
    if (a.M <= 80 && !transA) return launch_mb_tb<5, NB>(a, transA, xv, s);
    if (a.M <= 96 && !transA) return launch_mb_tb<6, NB>(a, transA, xv, s);
    if (a.M <= 112 && !transA) return launch_mb_tb<7, NB>(a, transA, xv, s);
    return launch_mb_tb<8, NB>(a, transA, xv, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_skinny_tb(const GemmArgs &a, int transA, hipStream_t s) {
  if (!skinny_supported(a, transA)) return hipErrorInvalidValue;
  const int nb = skinny_stripe_blocks(a.M, a.N, a.batch, true);
  if (nb == 4) return launch_tb_nb<4>(a, transA, s);
  if (nb == 2) return launch_tb_nb<2>(a, transA, s);
  return launch_tb_nb<1>(a, transA, s);
}
hipError_t launch_skinny32(const GemmArgs &a, int transA, hipStream_t s) {
  return launch_nb<2>(a, transA, s);
}
hipError_t launch_skinny64(const GemmArgs &a, int transA, hipStream_t s) {
  return launch_nb<4>(a, transA, s);
}

}  // namespace fp32gemm
