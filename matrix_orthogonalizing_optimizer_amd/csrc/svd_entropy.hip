// SVD-entropy diagnostic of weight matrices (gfx950).
//
// "Muon is Scalable for LLM Training", section 3.4 (singular-value spectrum
// dynamics): the SVD entropy of a matrix with singular values sigma_1..n is
// the entropy of p_i = sigma_i^2 / sum_j sigma_j^2 divided by log n;
// appendix F plots the singular values, largest first, over the largest.
//
// sigma_i^2 are the eigenvalues of the Gram matrix S = X X^T of the matrix
// oriented short side first (X [m, n], m = min(rows, cols)).  After reading
// the input everything is fp64:
//   1. svd_gram_kernel: S (block-lower 128 x 128 tiles, diagonal tiles
//      full): exact products of the fp32/bf16 inputs, fp64 sums;
//   2. Householder reduction of S to a symmetric tridiagonal T with the same
//      eigenvalues.  Step k reflects with H_k = I - v_k v_k^T (|v_k|^2 = 2,
//      support k+1 .. m-1): with p = B v_k (B the trailing block),
//      w_k = p - (v_k^T p / 2) v_k, H B H = B - v_k w_k^T - w_k v_k^T.
//      The rank-2 updates are deferred over panels of 16 steps and applied
//      together (svd_trd_panel_kernel): each step only reads the stored
//      block-lower trailing tiles once (svd_trd_pass_kernel, products with
//      v_k) and corrects for the panel's pending updates in
//      svd_trd_col_kernel (one workgroup per matrix), which also builds the
//      next reflector from the updated column;
//   3. svd_eig_kernel: eigenvalues of T by bisection on Sturm counts (the
//      number of negative pivots of T - x I), one lane per eigenvalue, so
//      they come out in ascending order;
//   4. svd_out_kernel: sigma_i^2 = max(lambda_i, 0), the entropy, and the
//      singular values largest first.
// Sums are taken in a fixed order: results do not depend on the batching.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>

#include "svd_internal.h"

namespace mo {
namespace {

constexpr int kT = kSvdTile;

__device__ __forceinline__ double to_f64(float x) { return static_cast<double>(x); }
__device__ __forceinline__ double to_f64(uint16_t x) {
  return static_cast<double>(__uint_as_float(static_cast<uint32_t>(x) << 16));
}

// Lower-triangular tile t -> (ti, tj), ti >= tj, row-major over the triangle.
__device__ __forceinline__ void tri_tile(int t, int& ti, int& tj) {
  int i = static_cast<int>((sqrtf(8.0f * static_cast<float>(t) + 1.0f) - 1.0f) * 0.5f);
  while (i * (i + 1) / 2 > t) --i;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

// Lane l's value of a double, as a wave-uniform value.
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(u), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(u >> 32), l);
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// Sum over the workgroup in a fixed order; every thread gets the same value.
// `sh` holds NT / 64 doubles.
template <int NT>
__device__ double block_sum(double x, double* sh) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < NT / 64; ++i) t += sh[i];
  return t;
}
template <int NT, bool kMax>
__device__ double block_ext(double x, double* sh) {
  for (int o = 32; o > 0; o >>= 1) {
    const double y = __shfl_xor(x, o);
    x = kMax ? fmax(x, y) : fmin(x, y);
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
  __syncthreads();
  double t = sh[0];
  for (int i = 1; i < NT / 64; ++i) t = kMax ? fmax(t, sh[i]) : fmin(t, sh[i]);
  return t;
}

// ------------------------------------------------------------------ 1. Gram
// One 128 x 128 block-lower tile of S per workgroup (blockIdx.y: matrix of
// the launch), fp64 FMA on the vector ALU: thread (ty, tx) of a 16 x 16 grid
// owns rows ty + 16 a and columns tx + 16 b (a, b < 8), so its LDS reads are
// either shared by 16 lanes or 16 consecutive doubles.  (On this chip fp64
// FMA on the vector ALU outruns fp64 MFMA: about 68 against 49 TFLOP/s
// measured.)  K is staged through LDS 32 columns at a time as fp64
// [k][row], rows padded to 129 so the transposed stores spread over the
// banks; the next chunk's global loads are issued into registers before the
// current chunk's products.  A diagonal tile computes its whole 128 x 128
// block, which covers the diagonal 64 x 64 tiles in full.
constexpr int kGT = 128;                  // output tile edge
constexpr int kGK = 32;                   // K per LDS stage
constexpr int kGLd = kGT + 1;             // LDS row stride (doubles)

// The thread's share of one operand chunk: rows row0 .. row0 + 127 of X,
// K columns k0 .. k0 + 31, 16 elements per thread.
template <typename T>
struct GramChunk {
  T v[16];
};

template <typename T>
__device__ __forceinline__ void gram_fetch(const T* __restrict__ w, const SvdGramArgs& p, int row0, int k0,
                                           GramChunk<T>& f) {
  const int tid = threadIdx.x;
  if (!p.trans) {
    // X = W [m, n]: 32 lanes along k (contiguous), 8 rows per pass
    const int kk = tid & 31, rr = tid >> 5;
    const int k = k0 + kk;
    const int kc = min(k, p.n - 1);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = row0 + rr + 8 * e;
      const T x = w[static_cast<int64_t>(min(row, p.m - 1)) * p.ld + kc];   // clamped: always valid
      f.v[e] = (row < p.m && k < p.n) ? x : T(0);
    }
  } else {
    // X = W^T, W [n, m]: lanes along the row index of X (contiguous in W)
    const int rr = tid & 127, kk = tid >> 7;
    const int row = row0 + rr;
    const int rc = min(row, p.m - 1);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int k = k0 + kk + 2 * e;
      const T x = w[static_cast<int64_t>(min(k, p.n - 1)) * p.ld + rc];       // clamped: always valid
      f.v[e] = (row < p.m && k < p.n) ? x : T(0);
    }
  }
}

template <typename T>
__device__ __forceinline__ void gram_store(const SvdGramArgs& p, const GramChunk<T>& f, double* xs) {
  const int tid = threadIdx.x;
  if (!p.trans) {
    const int kk = tid & 31, rr = tid >> 5;
#pragma unroll
    for (int e = 0; e < 16; ++e) xs[kk * kGLd + rr + 8 * e] = to_f64(f.v[e]);
  } else {
    const int rr = tid & 127, kk = tid >> 7;
#pragma unroll
    for (int e = 0; e < 16; ++e) xs[(kk + 2 * e) * kGLd + rr] = to_f64(f.v[e]);
  }
}

template <typename T>
__global__ __launch_bounds__(256, 2) void svd_gram_kernel(SvdGramArgs p) {
  __shared__ double xa[kGK * kGLd], xb[kGK * kGLd];
  int ti, tj;
  tri_tile(blockIdx.x, ti, tj);
  const T* __restrict__ w = static_cast<const T*>(p.src[blockIdx.y]);
  double* __restrict__ s = p.dst[blockIdx.y];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  double acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0;
  GramChunk<T> fa, fb;
  gram_fetch(w, p, ti * kGT, 0, fa);
  gram_fetch(w, p, tj * kGT, 0, fb);
  for (int k0 = 0; k0 < p.n; k0 += kGK) {
    gram_store(p, fa, xa);
    gram_store(p, fb, xb);
    __syncthreads();
    if (k0 + kGK < p.n) {
      gram_fetch(w, p, ti * kGT, k0 + kGK, fa);
      gram_fetch(w, p, tj * kGT, k0 + kGK, fb);
    }
    for (int k = 0; k < kGK; ++k) {
      double a[8], b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        a[i] = xa[k * kGLd + ty + 16 * i];
        b[i] = xb[k * kGLd + tx + 16 * i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = ti * kGT + ty + 16 * i;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = tj * kGT + tx + 16 * j;
      if (row < p.m && col < p.m) s[static_cast<int64_t>(row) * p.m + col] = acc[i][j];
    }
  }
}

// ------------------------------------------------- 2. Householder reduction
// Step k (k = 0 .. m - 3) reflects rows and columns k+1 .. m-1 with
// H_k = I - v_k v_k^T.  With B the current trailing block and p = B v_k,
// w_k = p - (v_k . p / 2) v_k and H B H = B - v_k w_k^T - w_k v_k^T.
// The rank-2 updates are deferred over a panel of up to kSvdPanel steps
// that starts at step k0: the stored matrix A is the matrix before step k0
// (on rows and columns >= k0 + 1), and the matrix before step k is
//   A - sum_t (v_t w_t^T + w_t v_t^T)   over the panel's steps t < k.
// Per step, with j = k + 1 (launch order col(-1), pass(0), col(0), [panel],
// pass(1), col(1), ...):
//   col(k):   [k >= 0] p_k = (sum of the slots of pass(k))
//                            - sum_t (v_t (w_t . v_k) + w_t (v_t . v_k)),
//             the dots summed from pass(k)'s per-block partials;
//             w_k = p_k - (v_k . p_k / 2) v_k, recorded in the panel.
//             Column j after step k: c_i = a_ij - sum over the panel and
//             step k of (v_t,i w_t,j + w_t,i v_t,j), i >= j; d_j = c_j.
//             j <= m - 3: v_j from x = c_{j+1..m-1} (the reflector mapping x
//             to (alpha, 0, ..), alpha = -sign(x_0) |x|), e_j = alpha
//             (v_j = 0, e_j = x_0 when x already has that form).
//             j = m - 2: e_j = c_{m-1}; d_{m-1} from a_{m-1,m-1} the same way.
//   panel:    once step k fills the panel (and more steps follow):
//             A -= sum_t (v_t w_t^T + w_t v_t^T) on rows and columns >= k + 2;
//             the next panel starts at step k + 1.
//   pass(j):  [j <= m - 3] partial sums of A v_j over rows and columns
//             >= j + 1 (read only), one slot per 64-wide tile: the tile (I, J),
//             I >= J, stores its row sums in slot J of rows I and, off the
//             diagonal, its column sums (the mirrored upper tile) in slot I of
//             rows J.  Its diagonal tiles also form the dots of the panel's
//             w_t and v_t with v_j over their rows (per row block).
// Column j keeps its old value in memory once read: it is never read again.
constexpr int kColThreads = 1024;
constexpr int kColPer = kSvdMaxM / kColThreads;
constexpr int kColWaves = kColThreads / 64;
constexpr int kP = kSvdPanel;

__global__ __launch_bounds__(kColThreads) void svd_trd_col_kernel(SvdTrdArgs p, int k, int k0) {
  __shared__ double red[kColWaves];
  __shared__ double dots[1][2 * kP];
  __shared__ double bc[3 + 2 * kP];       // w_k,j, v_k,j, x_0, then v_t,j and w_t,j of the panel
  const int b = blockIdx.x, tid = threadIdx.x, m = p.m, j = k + 1;
  const int np = k >= 0 ? k - k0 : 0;     // panel steps before step k
  const double* __restrict__ a = p.a + static_cast<int64_t>(b) * m * m;
  const double* __restrict__ vk = p.v + (static_cast<int64_t>(k & 1) * p.batch + b) * m;
  double* __restrict__ vj = p.v + (static_cast<int64_t>((k + 1) & 1) * p.batch + b) * m;
  const double* __restrict__ part = p.part + static_cast<int64_t>(b) * p.nb * m;
  double* __restrict__ pv = p.pv + static_cast<int64_t>(b) * kP * m;
  double* __restrict__ pw = p.pw + static_cast<int64_t>(b) * kP * m;
  double* __restrict__ d = p.d + static_cast<int64_t>(b) * m;
  double* __restrict__ e = p.e + static_cast<int64_t>(b) * m;

  double wv[kColPer], vkv[kColPer], c[kColPer];
  double wj = 0.0, vkj = 0.0;
  if (k >= 0) {
    // panel dots alpha_t = w_t . v_k, beta_t = v_t . v_k: sums of the
    // per-row-block partials of pass(k), in block order
    const int s0 = (k + 1) / kT;          // first slot / row block pass(k) wrote
    const double* __restrict__ pdot = p.pdot + static_cast<int64_t>(b) * p.nb * 2 * kP;
    if (tid < 2 * kP) {
      double a4[4] = {0.0, 0.0, 0.0, 0.0};
      if ((tid < kP ? tid : tid - kP) < np) {
        int sl = s0;
        for (; sl + 4 <= p.nb; sl += 4) {
#pragma unroll
          for (int u = 0; u < 4; ++u) a4[u] += pdot[(sl + u) * 2 * kP + tid];
        }
        for (int u = 0; sl < p.nb; ++sl, ++u) a4[u] += pdot[sl * 2 * kP + tid];
      }
      dots[0][tid] = (a4[0] + a4[1]) + (a4[2] + a4[3]);
    }
#pragma unroll
    for (int q = 0; q < kColPer; ++q) {
      const int i = tid + q * kColThreads;
      vkv[q] = (i < m && i >= k + 1) ? vk[i] : 0.0;
    }
    __syncthreads();
    double dot = 0.0;
#pragma unroll
    for (int q = 0; q < kColPer; ++q) {
      const int i = tid + q * kColThreads;
      wv[q] = 0.0;
      if (i < m && i >= k + 1) {
        // four independent partial sums (loads in flight together), combined
        // in a fixed order
        double s4[4] = {0.0, 0.0, 0.0, 0.0};
        int sl = s0;
        for (; sl + 4 <= p.nb; sl += 4) {
#pragma unroll
          for (int u = 0; u < 4; ++u) s4[u] += part[static_cast<int64_t>(sl + u) * m + i];
        }
        for (int u = 0; sl < p.nb; ++sl, ++u) s4[u] += part[static_cast<int64_t>(sl) * m + i];
        double s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
#pragma unroll
        for (int t = 0; t < kP; ++t)
          if (t < np)
            s -= pv[static_cast<int64_t>(t) * m + i] * dots[0][t] + pw[static_cast<int64_t>(t) * m + i] * dots[0][kP + t];
        wv[q] = s;
        dot = fma(vkv[q], s, dot);
      }
    }
    const double half = 0.5 * block_sum<kColThreads>(dot, red);
#pragma unroll
    for (int q = 0; q < kColPer; ++q) {
      const int i = tid + q * kColThreads;
      if (i < m) {
        const double wi = i >= k + 1 ? wv[q] - half * vkv[q] : 0.0;
        pv[static_cast<int64_t>(np) * m + i] = vkv[q];
        pw[static_cast<int64_t>(np) * m + i] = wi;
        wv[q] = wi;
        if (i == j) {
          bc[0] = wi;
          bc[1] = vkv[q];
        }
      }
    }
    __syncthreads();
    wj = bc[0];
    vkj = bc[1];
  } else {
#pragma unroll
    for (int q = 0; q < kColPer; ++q) wv[q] = vkv[q] = 0.0;
  }
  // row j of the earlier panel steps (written by earlier launches)
  if (tid < np) {
    bc[3 + tid] = pv[static_cast<int64_t>(tid) * m + j];
    bc[3 + kP + tid] = pw[static_cast<int64_t>(tid) * m + j];
  }
  __syncthreads();
  // column j after step k
#pragma unroll
  for (int q = 0; q < kColPer; ++q) {
    const int i = tid + q * kColThreads;
    c[q] = 0.0;
    if (i < m && i >= j) {
      double x = a[static_cast<int64_t>(i) * m + j];
      double dl = 0.0;
      const bool last = j == m - 2 && i == m - 1;
      if (last) dl = a[static_cast<int64_t>(i) * m + i];
#pragma unroll
      for (int t = 0; t < kP; ++t)
        if (t < np) {
          const double vti = pv[static_cast<int64_t>(t) * m + i], wti = pw[static_cast<int64_t>(t) * m + i];
          x -= vti * bc[3 + kP + t] + wti * bc[3 + t];
          if (last) dl -= 2.0 * vti * wti;
        }
      if (k >= 0) {
        x -= vkv[q] * wj + wv[q] * vkj;
        if (last) dl -= 2.0 * vkv[q] * wv[q];
      }
      c[q] = x;
      if (i == j) d[j] = x;
      if (last) {
        e[j] = x;
        d[i] = dl;
      }
    }
  }
  if (j > m - 3) return;                  // no reflector left (uniform)

  double ss = 0.0;
#pragma unroll
  for (int q = 0; q < kColPer; ++q) {
    const int i = tid + q * kColThreads;
    if (i < m && i >= j + 2) ss = fma(c[q], c[q], ss);
    if (i == j + 1) bc[2] = c[q];
  }
  const double sigma = block_sum<kColThreads>(ss, red);   // (its barriers publish bc[2])
  const double x0 = bc[2];
  double scale = 0.0, u0 = 0.0, alpha = x0;
  if (sigma > 0.0) {
    const double mu = sqrt(fma(x0, x0, sigma));
    alpha = x0 >= 0.0 ? -mu : mu;
    u0 = x0 - alpha;                      // |u0| = |x0| + mu: no cancellation
    scale = sqrt(2.0 / fma(u0, u0, sigma));
  }
#pragma unroll
  for (int q = 0; q < kColPer; ++q) {
    const int i = tid + q * kColThreads;
    if (i < m) vj[i] = i == j + 1 ? u0 * scale : (i >= j + 2 ? c[q] * scale : 0.0);
  }
  if (tid == 0) e[j] = alpha;
}

// Tile (I, J) of the block-lower trailing region [r0, m)^2 for blockIdx.x;
// a lane owns column J * 64 + (lane) and rows rbase .. rbase + 15 of it.
struct TrdTile {
  int I, J, col, colc, rbase, tc, tr;
  bool cok;
};
__device__ __forceinline__ TrdTile trd_tile(int m, int r0) {
  TrdTile t;
  int ti, tj;
  tri_tile(blockIdx.x, ti, tj);
  t.I = r0 / kT + ti;
  t.J = r0 / kT + tj;
  t.tc = threadIdx.x & 63;
  t.tr = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  t.col = t.J * kT + t.tc;
  t.colc = min(t.col, m - 1);
  t.cok = t.col < m && t.col >= r0;
  t.rbase = t.I * kT + t.tr * 16;
  return t;
}

// pass(j): partial sums of A v_j.  Loads go to clamped (always valid)
// addresses, all 16 issued before any use, and positions outside the
// trailing block are masked afterwards, so no load sits in a lane-divergent
// branch.  The wave's 16 entries of v_j (rows) come in with one load by
// lanes 0-15 and are broadcast by lane.
__global__ __launch_bounds__(256) void svd_trd_pass_kernel(SvdTrdArgs p, int j, int np) {
  __shared__ double red[kT][kT + 1];
  __shared__ double colp[4][kT];
  const int m = p.m, r0 = j + 1;
  const TrdTile g = trd_tile(m, r0);
  const int b = blockIdx.y;
  const double* __restrict__ a = p.a + static_cast<int64_t>(b) * m * m;
  const double* __restrict__ vn = p.v + (static_cast<int64_t>(j & 1) * p.batch + b) * m;
  double* __restrict__ part = p.part + static_cast<int64_t>(b) * p.nb * m;

  double x[16];
#pragma unroll
  // non-temporal: a step streams the whole trailing block, which is far
  // larger than the caches, and keeping it would evict the slots the
  // column kernel reads next
  for (int q = 0; q < 16; ++q)
    x[q] = __builtin_nontemporal_load(&a[static_cast<int64_t>(min(g.rbase + q, m - 1)) * m + g.colc]);
  const double vnc = vn[g.colc];
  const double rv = g.tc < 16 ? vn[min(g.rbase + g.tc, m - 1)] : 0.0;
  double cp = 0.0;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int row = g.rbase + q;
    const double y = (g.cok && row < m && row >= r0) ? x[q] : 0.0;
    cp = fma(y, readlane_f64(rv, q), cp);
    red[g.tr * 16 + q][g.tc] = y * vnc;
  }
  colp[g.tr][g.tc] = cp;
  __syncthreads();
  {
    // row sums: four lanes per row, 16 columns each, then combined in the
    // same order on every lane
    const int rl = threadIdx.x >> 2, qd = threadIdx.x & 3;
    double s = 0.0;
#pragma unroll
    for (int t = 0; t < 16; ++t) s += red[rl][qd * 16 + t];
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    const int row = g.I * kT + rl;
    if (qd == 0 && row < m) part[static_cast<int64_t>(g.J) * m + row] = s;
  }
  if (g.I != g.J && threadIdx.x < kT) {
    const int c2 = g.J * kT + threadIdx.x;
    if (c2 < m)
      part[static_cast<int64_t>(g.I) * m + c2] =
          (colp[0][threadIdx.x] + colp[1][threadIdx.x]) + (colp[2][threadIdx.x] + colp[3][threadIdx.x]);
  }
  if (g.I == g.J) {
    // panel dots over this row block: lane = row, wave tr takes t = tr, tr + 4, ..
    const int row = g.I * kT + g.tc;
    const bool rok = row < m && row >= r0;
    const double vr = rok ? vn[row] : 0.0;
    const double* __restrict__ pv = p.pv + static_cast<int64_t>(b) * kP * m;
    const double* __restrict__ pw = p.pw + static_cast<int64_t>(b) * kP * m;
    double* __restrict__ pdot = p.pdot + (static_cast<int64_t>(b) * p.nb + g.I) * 2 * kP;
    for (int t = g.tr; t < np; t += 4) {
      double sa = 0.0, sb = 0.0;
      if (rok) {
        sa = pw[static_cast<int64_t>(t) * m + row] * vr;
        sb = pv[static_cast<int64_t>(t) * m + row] * vr;
      }
      for (int o = 32; o > 0; o >>= 1) {
        sa += __shfl_xor(sa, o);
        sb += __shfl_xor(sb, o);
      }
      if (g.tc == 0) {
        pdot[t] = sa;
        pdot[kP + t] = sb;
      }
    }
  }
}

// panel: A -= sum_t (v_t w_t^T + w_t v_t^T) over the kSvdPanel steps of the
// full panel, on the block-lower region [r0, m)^2.  The tile's rows of v_t
// and w_t are staged in LDS (read as broadcasts); the lane's column of them
// stays in registers.
__global__ __launch_bounds__(256) void svd_trd_panel_kernel(SvdTrdArgs p, int r0) {
  __shared__ double rpv[kP][kT], rpw[kP][kT];
  const int m = p.m;
  const TrdTile g = trd_tile(m, r0);
  const int b = blockIdx.y;
  double* __restrict__ a = p.a + static_cast<int64_t>(b) * m * m;
  const double* __restrict__ pv = p.pv + static_cast<int64_t>(b) * kP * m;
  const double* __restrict__ pw = p.pw + static_cast<int64_t>(b) * kP * m;

  double x[16];
#pragma unroll
  for (int q = 0; q < 16; ++q)   // non-temporal, as in the pass kernel
    x[q] = __builtin_nontemporal_load(&a[static_cast<int64_t>(min(g.rbase + q, m - 1)) * m + g.colc]);
  double cv[kP], cw[kP];
#pragma unroll
  for (int t = 0; t < kP; ++t) {
    cv[t] = pv[static_cast<int64_t>(t) * m + g.colc];
    cw[t] = pw[static_cast<int64_t>(t) * m + g.colc];
  }
  for (int f = threadIdx.x; f < kP * kT; f += 256) {
    const int t = f / kT, rl = f % kT;
    const int row = min(g.I * kT + rl, m - 1);
    rpv[t][rl] = pv[static_cast<int64_t>(t) * m + row];
    rpw[t][rl] = pw[static_cast<int64_t>(t) * m + row];
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int row = g.rbase + q, rl = g.tr * 16 + q;
    double u = 0.0;
#pragma unroll
    for (int t = 0; t < kP; ++t) u = fma(rpv[t][rl], cw[t], fma(rpw[t][rl], cv[t], u));
    if (g.cok && row < m && row >= r0) a[static_cast<int64_t>(row) * m + g.col] = x[q] - u;
  }
}

// ------------------------------------------------------- 3. eigenvalues
// Sturm count: the number of eigenvalues of T below x equals the number of
// negative pivots of the LDL^T factorisation of T - x I (Sylvester's law of
// inertia).  A pivot smaller than `pivmin` in magnitude is replaced by
// -pivmin so that the recurrence never divides by zero.  e^2 / q is formed
// as e^2 times a reciprocal refined by two Newton steps from the hardware
// estimate (within about an ulp: the count is that of T with e^2 perturbed
// by about an ulp), half the instructions of an IEEE division.
__device__ __forceinline__ double recip_nr(double q) {
  double r = __builtin_amdgcn_rcp(q);
  double e = fma(-q, r, 1.0);
  r = fma(e, r, r);
  e = fma(-q, r, 1.0);
  return fma(e, r, r);
}

constexpr int kEigThreads = 256;

__global__ __launch_bounds__(kEigThreads) void svd_eig_kernel(SvdEigArgs p) {
  extern __shared__ double eig_lds[];     // d and e^2: 16 m bytes
  __shared__ double red[kEigThreads / 64];
  const int b = blockIdx.y, m = p.m, tid = threadIdx.x;
  double* sd = eig_lds;
  double* se2 = eig_lds + m;
  const double* __restrict__ d = p.d + static_cast<int64_t>(b) * m;
  const double* __restrict__ e = p.e + static_cast<int64_t>(b) * m;
  double lo = DBL_MAX, hi = -DBL_MAX, emax = 0.0;
  for (int i = tid; i < m; i += kEigThreads) {
    const double di = d[i];
    const double el = i > 0 ? fabs(e[i - 1]) : 0.0;
    const double er = i < m - 1 ? fabs(e[i]) : 0.0;
    sd[i] = di;
    se2[i] = er * er;
    lo = fmin(lo, di - el - er);          // Gershgorin discs
    hi = fmax(hi, di + el + er);
    emax = fmax(emax, er);
  }
  lo = block_ext<kEigThreads, false>(lo, red);
  hi = block_ext<kEigThreads, true>(hi, red);
  emax = block_ext<kEigThreads, true>(emax, red);
  const double tnorm = fmax(fabs(lo), fabs(hi));
  const double pivmin = DBL_MIN * fmax(1.0, emax * emax);
  const double atol = DBL_EPSILON * tnorm;
  // widen so that the counts at the ends are exactly 0 and m
  lo -= 2.0 * DBL_EPSILON * tnorm * m + 2.0 * pivmin;
  hi += 2.0 * DBL_EPSILON * tnorm * m + 2.0 * pivmin;

  const int kk = blockIdx.x * kEigThreads + tid;
  if (kk >= m) return;                    // no barrier follows
  for (int it = 0; it < 128; ++it) {
    if (hi - lo <= atol + 2.0 * DBL_EPSILON * fmax(fabs(lo), fabs(hi))) break;
    const double x = 0.5 * (lo + hi);
    int cnt = 0;
    double q = sd[0] - x;
    if (fabs(q) < pivmin) q = -pivmin;
    cnt += q < 0.0;
    for (int i = 1; i < m; ++i) {
      q = (sd[i] - x) - se2[i - 1] * recip_nr(q);
      if (fabs(q) < pivmin) q = -pivmin;
      cnt += q < 0.0;
    }
    if (cnt <= kk) lo = x;
    else hi = x;
  }
  p.lam[static_cast<int64_t>(b) * m + kk] = 0.5 * (lo + hi);
}

// ------------------------------------------------- 4. entropy, sigma
constexpr int kOutThreads = 256;

__global__ __launch_bounds__(kOutThreads) void svd_out_kernel(SvdOutArgs p) {
  __shared__ double red[kOutThreads / 64];
  const int q = blockIdx.x, b = p.first + q, m = p.m, tid = threadIdx.x;
  const double* __restrict__ lam = p.lam + static_cast<int64_t>(b) * m;
  double tot = 0.0;
  for (int i = tid; i < m; i += kOutThreads) tot += fmax(lam[i], 0.0);
  tot = block_sum<kOutThreads>(tot, red);
  double h = 0.0;
  if (tot > 0.0) {
    for (int i = tid; i < m; i += kOutThreads) {
      const double pi = fmax(lam[i], 0.0) / tot;
      if (pi > 0.0) h -= pi * log(pi);
    }
  }
  h = block_sum<kOutThreads>(h, red);
  if (tid == 0) p.entropy[p.out_index[q]] = (m > 1 && tot > 0.0) ? h / log(static_cast<double>(m)) : 0.0;
  if (p.sigma) {
    double* s = p.sigma + p.sigma_off[q];
    for (int i = tid; i < m; i += kOutThreads) s[m - 1 - i] = sqrt(fmax(lam[i], 0.0));
  }
}

}  // namespace

hipError_t launch_svd_gram(int dt, const SvdGramArgs& a, int count, hipStream_t s) {
  const int nt = (a.m + kGT - 1) / kGT;
  const dim3 grid(nt * (nt + 1) / 2, count);
  if (dt == MO_F32) hipLaunchKernelGGL(svd_gram_kernel<float>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(svd_gram_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_svd_trd_col(const SvdTrdArgs& a, int k, int k0, hipStream_t s) {
  hipLaunchKernelGGL(svd_trd_col_kernel, dim3(a.batch), dim3(kColThreads), 0, s, a, k, k0);
  return hipGetLastError();
}

hipError_t launch_svd_trd_pass(const SvdTrdArgs& a, int j, int np, hipStream_t s) {
  const int t = a.nb - (j + 1) / kT;
  hipLaunchKernelGGL(svd_trd_pass_kernel, dim3(t * (t + 1) / 2, a.batch), dim3(256), 0, s, a, j, np);
  return hipGetLastError();
}

hipError_t launch_svd_trd_panel(const SvdTrdArgs& a, int r0, hipStream_t s) {
  const int t = a.nb - r0 / kT;
  hipLaunchKernelGGL(svd_trd_panel_kernel, dim3(t * (t + 1) / 2, a.batch), dim3(256), 0, s, a, r0);
  return hipGetLastError();
}

hipError_t launch_svd_eig(const SvdEigArgs& a, int batch, hipStream_t s) {
  // dynamic LDS above 64 KiB (m > 4096) needs the kernel's limit raised
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(svd_eig_kernel),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     2 * kSvdMaxM * static_cast<int>(sizeof(double)));
  if (attr != hipSuccess) return attr;
  const size_t lds = 2 * static_cast<size_t>(a.m) * sizeof(double);
  hipLaunchKernelGGL(svd_eig_kernel, dim3((a.m + kEigThreads - 1) / kEigThreads, batch), dim3(kEigThreads), lds, s,
                     a);
  return hipGetLastError();
}

hipError_t launch_svd_out(const SvdOutArgs& a, int count, hipStream_t s) {
  hipLaunchKernelGGL(svd_out_kernel, dim3(count), dim3(kOutThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mo
