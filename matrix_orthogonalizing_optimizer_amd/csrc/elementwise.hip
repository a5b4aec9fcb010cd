// HBM-bound kernels of the Muon step and of the AdamW side path (gfx950).
//
//  * prep:  momentum M <- mu M + G (section 2.1, Eq. 1), the Nesterov input
//           N = mu M + G (paragraph after Eq. 1), per-tile fp32 partial sums
//           of N^2 for the Frobenius norm (text before Eq. 2), and N written
//           once, in the Newton-Schulz dtype, as the oriented blocked iterate
//           X_0 (transposed through LDS for tall parameters) -- one pass over
//           G and M.
//  * norm:  per-matrix fp64 combine of the partials -> r = 1/(||N||_F + eps).
//           X_0 = r N is never materialised: r is applied in the epilogues of
//           the first Gram and Update products.
//  * apply_x0: W <- W - lr (0.2 sqrt(max(A,B)) X_0 + wd W) when N = 0
//           iterations are requested (section 2.2, Eq. 4).
//  * rms:   per-matrix fp64 combine of squared-update partials ->
//           sqrt(mean(X_N^2)) (section 2.3, Algorithm 1's return value).
//  * adamw: AdamW with bias correction and decoupled decay for non-matrix
//           parameters (section 2.2).
// Reductions are deterministic: fixed-shape trees, no float atomics.
#include "mo_internal.h"
#include "mo_layout.h"

namespace mo {

__device__ __forceinline__ float bf2f(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Load 4 consecutive elements [off, off + nvalid) of a fp32 or bf16 array;
// missing ones read as 0.  `vec` = the 4 are in range and 4-aligned.
// kNT: the data is touched once per step, so the vector accesses carry the
// non-temporal hint (streamed past the caches instead of filling them).
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

template <bool kNT = false>
__device__ __forceinline__ void load4(const void* base, int dt, int64_t off, int nvalid,
                                      bool vec, float v[4]) {
  if (dt == F32) {
    const float* p = static_cast<const float*>(base) + off;
    if (vec) {
      f32x4v q;
      if constexpr (kNT) q = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
      else q = *reinterpret_cast<const f32x4v*>(p);
      v[0] = q[0]; v[1] = q[1]; v[2] = q[2]; v[3] = q[3];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = j < nvalid ? p[j] : 0.0f;
    }
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(base) + off;
    if (vec) {
      u32x2v q;
      if constexpr (kNT) q = __builtin_nontemporal_load(reinterpret_cast<const u32x2v*>(p));
      else q = *reinterpret_cast<const u32x2v*>(p);
      v[0] = bf2f(q[0] & 0xffffu); v[1] = bf2f(q[0] >> 16);
      v[2] = bf2f(q[1] & 0xffffu); v[3] = bf2f(q[1] >> 16);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = j < nvalid ? bf2f(p[j]) : 0.0f;
    }
  }
}

template <bool kNT = false>
__device__ __forceinline__ void store4(void* base, int dt, int64_t off, int nvalid,
                                       bool vec, const float v[4]) {
  if (dt == F32) {
    float* p = static_cast<float*>(base) + off;
    if (vec) {
      const f32x4v q = {v[0], v[1], v[2], v[3]};
      if constexpr (kNT) __builtin_nontemporal_store(q, reinterpret_cast<f32x4v*>(p));
      else *reinterpret_cast<f32x4v*>(p) = q;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j < nvalid) p[j] = v[j];
    }
  } else {
    uint16_t* p = static_cast<uint16_t*>(base) + off;
    if (vec) {
      const u32x2v q = {static_cast<uint32_t>(f2bf(v[0])) | (static_cast<uint32_t>(f2bf(v[1])) << 16),
                        static_cast<uint32_t>(f2bf(v[2])) | (static_cast<uint32_t>(f2bf(v[3])) << 16)};
      if constexpr (kNT) __builtin_nontemporal_store(q, reinterpret_cast<u32x2v*>(p));
      else *reinterpret_cast<u32x2v*>(p) = q;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j < nvalid) p[j] = f2bf(v[j]);
    }
  }
}

// Round a value to the storage dtype (what a later load would return).
__device__ __forceinline__ float round_to(int dt, float v) {
  return dt == F32 ? v : bf2f(f2bf(v));
}

__device__ __forceinline__ float block_sum_256(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// kW = 8 consecutive elements of one row: 16 bytes of bf16, or two
// 16-byte halves of fp32 (each half one vector access when aligned).
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

template <int kW, bool kNT>
__device__ __forceinline__ void loadw(const void* base, int dt, int64_t off, int nvalid, bool vecw,
                                      bool vec4, float v[kW]) {
  if (kW == 8 && dt == BF16 && vecw) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + off;
    u32x4v q;
    if constexpr (kNT) q = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
    else q = *reinterpret_cast<const u32x4v*>(p);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      v[2 * h] = bf2f(q[h] & 0xffffu);
      v[2 * h + 1] = bf2f(q[h] >> 16);
    }
    return;
  }
#pragma unroll
  for (int h = 0; h < kW / 4; ++h) {
    const int nv = max(0, min(4, nvalid - 4 * h));
    load4<kNT>(base, dt, off + 4 * h, nv, vec4 && nv == 4, v + 4 * h);
  }
}

template <int kW, bool kNT>
__device__ __forceinline__ void storew(void* base, int dt, int64_t off, int nvalid, bool vecw,
                                       bool vec4, const float v[kW]) {
  if (kW == 8 && dt == BF16 && vecw) {
    uint16_t* p = static_cast<uint16_t*>(base) + off;
    u32x4v q;
#pragma unroll
    for (int h = 0; h < 4; ++h)
      q[h] = static_cast<uint32_t>(f2bf(v[2 * h])) | (static_cast<uint32_t>(f2bf(v[2 * h + 1])) << 16);
    if constexpr (kNT) __builtin_nontemporal_store(q, reinterpret_cast<u32x4v*>(p));
    else *reinterpret_cast<u32x4v*>(p) = q;
    return;
  }
#pragma unroll
  for (int h = 0; h < kW / 4; ++h) {
    const int nv = max(0, min(4, nvalid - 4 * h));
    store4<kNT>(base, dt, off + 4 * h, nv, vec4 && nv == 4, v + 4 * h);
  }
}

// kW consecutive elements of X (oriented row xr, columns xc ..) in the
// blocked layout: a 16-byte chunk holds 8 bf16 or 4 fp32 consecutive
// columns, so a bf16 group of 8 is one store and an fp32 group one store
// per 4 (chunks are permuted within a row).  Non-temporal like the other
// streams: X of a whole step is far larger than the caches, so the first
// Gram reads it from HBM either way.
template <int kW>
__device__ __forceinline__ void store_x(char* x, int ns_dt, const Blocked& Lx, int xr, int xc,
                                        const float v[kW]) {
  if (kW == 8 && ns_dt == BF16) {
    storew<kW, true>(x, ns_dt, blk_off(Lx, xr, xc), kW, true, true, v);
  } else {
#pragma unroll
    for (int h = 0; h < kW / 4; ++h) store4<true>(x, ns_dt, blk_off(Lx, xr, xc + 4 * h), 4, true, v + 4 * h);
  }
}

// One 64x64 tile of the padded natural domain [A_pad, B_pad] per block.
// Thread layout: 64 / kW threads x kW columns across a row, 256 / (64 / kW)
// rows per pass.  The Newton-Schulz input is written once, in the oriented
// layout [m_pad, n_pad]: straight through for a wide parameter, transposed
// through an LDS tile for a tall one (its columns are the rows of X).
// kW = 8 serves bf16 gradients: 16-byte accesses for the bf16 arrays, and
// every load of the thread's rows issued before any arithmetic or store
// (the momentum stores may alias later rows' loads, so the compiler would
// not hoist them by itself).  kW = 4 serves fp32 gradients, whose 16-byte
// loads run as fast row by row.
template <int kW>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs p) {
  constexpr int kTX = 64 / kW;           // threads across a row
  constexpr int kRows = 256 / kTX;       // rows per pass
  constexpr int kPasses = 64 / kRows;
  constexpr bool kAhead = kW == 8;
  __shared__ float tile[64][65];
  __shared__ float red[4];
  const int b = blockIdx.x / p.tiles_per_mat;
  const int t = blockIdx.x - b * p.tiles_per_mat;
  const MatDesc md = p.desc[b];
  const bool ori = md.oriented != 0;
  const int A = ori ? p.n : p.m, B = ori ? p.m : p.n;
  const int B_pad = ori ? p.m_pad : p.n_pad;
  const int tiles_b = B_pad >> 6;
  const int ta = t / tiles_b, tb = t - ta * tiles_b;
  const int tx = threadIdx.x % kTX, ty = threadIdx.x / kTX;
  const int esz = p.ns_dt == F32 ? 4 : 2;
  char* x = static_cast<char*>(p.x) + b * p.x_stride * esz;
  const Blocked Lx = blocked(p.tile, p.n_pad, esz);      // X: [m_pad, n_pad]
  const bool vec4 = (B & 3) == 0;
  const bool vecw = (B % kW) == 0;
  float sq = 0.0f;

  const int c = tb * 64 + tx * kW;
  const int nvalid = max(0, min(kW, B - c));
  const bool full = vecw && nvalid == kW;
  float g[kPasses][kW], m[kPasses][kW];
  if constexpr (kAhead) {
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
      const int r = ta * 64 + ty + pass * kRows;
      if (r < A && nvalid > 0) {
        const int64_t off = static_cast<int64_t>(r) * B + c;
        loadw<kW, true>(md.grad, p.grad_dt, off, nvalid, full, vec4, g[pass]);
        if (p.has_mom) loadw<kW, true>(md.mom, p.mom_dt, off, nvalid, full, vec4, m[pass]);
      }
    }
  }
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int rl = ty + pass * kRows;
    const int r = ta * 64 + rl;
    float n4[kW];
#pragma unroll
    for (int j = 0; j < kW; ++j) n4[j] = 0.0f;
    if (r < A && nvalid > 0) {
      const int64_t off = static_cast<int64_t>(r) * B + c;
      if constexpr (!kAhead) {
        loadw<kW, true>(md.grad, p.grad_dt, off, nvalid, full, vec4, g[pass]);
        if (p.has_mom) loadw<kW, true>(md.mom, p.mom_dt, off, nvalid, full, vec4, m[pass]);
      }
      if (p.has_mom) {
#pragma unroll
        for (int j = 0; j < kW; ++j) {
          const float mn = p.mu * m[pass][j] + g[pass][j];
          m[pass][j] = mn;
          n4[j] = p.nesterov ? p.mu * mn + g[pass][j] : mn;
        }
        storew<kW, true>(md.mom, p.mom_dt, off, nvalid, full, vec4, m[pass]);
      } else {
#pragma unroll
        for (int j = 0; j < kW; ++j) n4[j] = g[pass][j];
      }
#pragma unroll
      for (int j = 0; j < kW; ++j) {
        if (j >= nvalid) n4[j] = 0.0f;
        sq += n4[j] * n4[j];
      }
    }
    if (!ori) {
      // padding written as zeros
      store_x<kW>(x, p.ns_dt, Lx, r, c, n4);
    } else {
#pragma unroll
      for (int j = 0; j < kW; ++j) tile[rl][tx * kW + j] = n4[j];
    }
  }
  if (ori) {
    __syncthreads();
    // rows of X are columns of the tile
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
      const int cl = ty + pass * kRows;
      float v[kW];
#pragma unroll
      for (int j = 0; j < kW; ++j) v[j] = tile[tx * kW + j][cl];
      store_x<kW>(x, p.ns_dt, Lx, tb * 64 + cl, ta * 64 + tx * kW, v);
    }
  }
  const float s = block_sum_256(sq, red);
  if (threadIdx.x == 0) p.norm_part[static_cast<int64_t>(b) * p.tiles_per_mat + t] = s;
}

// One wave per matrix: fp64 sum of its partials.
__global__ __launch_bounds__(64) void norm_kernel(NormArgs p) {
  const int b = blockIdx.x;
  const float* part = p.part + static_cast<int64_t>(b) * p.tiles;
  double s = 0.0;
  for (int i = threadIdx.x; i < p.tiles; i += 64) s += static_cast<double>(part[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (threadIdx.x == 0) p.rscale[b] = static_cast<float>(1.0 / (sqrt(s) + static_cast<double>(p.eps)));
}

// X_N = X_0 = r N.  One 64x64 tile of the true natural domain per block.
__global__ __launch_bounds__(256) void apply_x0_kernel(ApplyX0Args p) {
  __shared__ float red[4];
  const int b = blockIdx.x / p.tiles_per_mat;
  const int t = blockIdx.x - b * p.tiles_per_mat;
  const MatDesc md = p.desc[b];
  const int A = md.oriented ? p.n : p.m, B = md.oriented ? p.m : p.n;
  const int tiles_b = (B + 63) >> 6;
  const int ta = t / tiles_b, tb = t - ta * tiles_b;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int esz = p.ns_dt == F32 ? 4 : 2;
  // N in the oriented layout X [m_pad, n_pad] (transposed for a tall parameter)
  const char* base = static_cast<const char*>(p.x) + b * p.x_stride * esz;
  const Blocked Lx = blocked(p.tile, p.n_pad, esz);
  const float r0 = p.rscale[b];
  const float lrwd = p.lrwd;
  const float stp = p.step_dev ? p.step_dev[b] : p.step;
  const int c = tb * 64 + tx * 4;
  const int nvalid = max(0, min(4, B - c));
  const bool vec = ((B & 3) == 0) && nvalid == 4;
  float sq = 0.0f;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int r = ta * 64 + ty + pass * 16;
    if (r >= A || nvalid == 0) continue;
    float x[4];
    if (!md.oriented) {
      load4(base, p.ns_dt, blk_off(Lx, r, c), 4, true, x);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v[4];
        load4(base, p.ns_dt, blk_off(Lx, c + j, r), 1, false, v);
        x[j] = v[0];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = j < nvalid ? r0 * x[j] : 0.0f;
      sq += x[j] * x[j];
    }
    const int64_t off = static_cast<int64_t>(r) * B + c;
    if (p.out) {
      store4(static_cast<char*>(p.out) + b * p.s_out * esz, p.ns_dt, off, nvalid, vec, x);
    } else {
      float w[4];
      load4(md.param, F32, off, nvalid, vec, w);
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = w[j] - (lrwd * w[j] + stp * x[j]);
      store4(md.param, F32, off, nvalid, vec, w);
    }
  }
  if (p.rms_part) {
    const float s = block_sum_256(sq, red);
    if (threadIdx.x == 0) p.rms_part[static_cast<int64_t>(b) * p.tiles_per_mat + t] = s;
  }
}

__global__ __launch_bounds__(64) void rms_kernel(RmsArgs p) {
  const int b = blockIdx.x;
  const float* part = p.part + static_cast<int64_t>(b) * p.tiles;
  double s = 0.0;
  for (int i = threadIdx.x; i < p.tiles; i += 64) s += static_cast<double>(part[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (threadIdx.x == 0) {
    if (p.rscale) {
      const double r = static_cast<double>(p.rscale[b]);
      s *= r * r;
    }
    const double rms = sqrt(s * p.inv_count);
    if (p.update_rms) p.update_rms[p.desc[b].out_index] = static_cast<float>(rms);
    if (p.step) p.step[b] = rms > 0.0 ? static_cast<float>(static_cast<double>(p.lr_scale) / rms) : 0.0f;
  }
}

// AdamW: each block covers kAdamElemsPerBlock consecutive elements of one
// tensor, 8 per thread as two groups of 4.
__global__ __launch_bounds__(256) void adamw_kernel(AdamArgs p) {
  int k = 0;
  while (k + 1 < p.count && p.t[k + 1].block0 <= blockIdx.x) ++k;
  const AdamTensor T = p.t[k];
  const int64_t base = (static_cast<int64_t>(blockIdx.x) - T.block0) * kAdamElemsPerBlock;
  const float ob1 = p.one_m_beta1, ob2 = p.one_m_beta2, lrwd = p.lr * p.wd;
  // kParts groups of 4 elements per thread: every load is issued before any
  // arithmetic or store (the stores may alias the next group's loads, so the
  // compiler would not hoist them by itself)
  constexpr int kParts = kAdamElemsPerBlock / 1024;
  float g[kParts][4], w[kParts][4], m[kParts][4], v[kParts][4];
  int nv[kParts];
#pragma unroll
  for (int h = 0; h < kParts; ++h) {
    const int64_t off = base + h * 1024 + threadIdx.x * 4;
    nv[h] = static_cast<int>(max<int64_t>(0, min<int64_t>(4, T.n - off)));
    if (nv[h] == 0) continue;
    const bool vec = nv[h] == 4;
    load4<true>(T.g, p.grad_dt, off, nv[h], vec, g[h]);
    load4<true>(T.p, F32, off, nv[h], vec, w[h]);
    load4<true>(T.m, F32, off, nv[h], vec, m[h]);
    load4<true>(T.v, F32, off, nv[h], vec, v[h]);
  }
#pragma unroll
  for (int h = 0; h < kParts; ++h) {
    if (nv[h] == 0) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m[h][j] = p.beta1 * m[h][j] + ob1 * g[h][j];
      v[h][j] = p.beta2 * v[h][j] + ob2 * g[h][j] * g[h][j];
      const float upd = (m[h][j] * p.bc1) / (sqrtf(v[h][j]) * p.bc2_rsqrt + p.eps);
      w[h][j] = w[h][j] - (p.lr * upd + lrwd * w[h][j]);
    }
    const int64_t off = base + h * 1024 + threadIdx.x * 4;
    const bool vec = nv[h] == 4;
    store4<true>(T.p, F32, off, nv[h], vec, w[h]);
    store4<true>(T.m, F32, off, nv[h], vec, m[h]);
    store4<true>(T.v, F32, off, nv[h], vec, v[h]);
  }
}

// Descriptor upload carried in the kernel arguments: the runtime copies the
// arguments when the launch is enqueued, so the host neither stages the
// table in pinned memory nor waits for an earlier upload to finish, and the
// launch can be captured into a graph like any other.
__global__ __launch_bounds__(kDescPerCopy) void desc_copy_kernel(DescCopyArgs a) {
  const int i = threadIdx.x;
  if (i < a.count) a.dst[i] = a.d[i];
}

hipError_t launch_desc_copy(const MatDesc* src, int64_t count, MatDesc* dst, hipStream_t s) {
  for (int64_t i0 = 0; i0 < count; i0 += kDescPerCopy) {
    DescCopyArgs a;
    a.count = static_cast<int>(count - i0 < kDescPerCopy ? count - i0 : kDescPerCopy);
    a.dst = dst + i0;
    for (int k = 0; k < a.count; ++k) a.d[k] = src[i0 + k];
    hipLaunchKernelGGL(desc_copy_kernel, dim3(1), dim3(kDescPerCopy), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_prep(const PrepArgs& a, int chunk, hipStream_t s) {
  if (a.grad_dt == BF16) hipLaunchKernelGGL(prep_kernel<8>, dim3(a.tiles_per_mat * chunk), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(prep_kernel<4>, dim3(a.tiles_per_mat * chunk), dim3(256), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_norm(const NormArgs& a, int chunk, hipStream_t s) {
  hipLaunchKernelGGL(norm_kernel, dim3(chunk), dim3(64), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_apply_x0(const ApplyX0Args& a, int chunk, hipStream_t s) {
  hipLaunchKernelGGL(apply_x0_kernel, dim3(a.tiles_per_mat * chunk), dim3(256), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_rms(const RmsArgs& a, int chunk, hipStream_t s) {
  hipLaunchKernelGGL(rms_kernel, dim3(chunk), dim3(64), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_adamw(const AdamArgs& a, int64_t blocks, hipStream_t s) {
  hipLaunchKernelGGL(adamw_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mo
