// Newton-Schulz GEMMs on CDNA4 matrix cores (gfx950).
//
// Eq. 2 of "Muon is Scalable for LLM Training" (section 2.1) is evaluated as
// three products per iteration, all of the form C = A * B^T with both
// operands K-contiguous (row-major [rows, K]):
//   Gram    S = X X^T          A = B = X (row-major [m, n])      symmetric
//   Poly    P = b S + c S S^T  A = B = S (S is exactly symmetric) symmetric
//   Update  X' = a X + P X     A = P, B = X^T (row-major [n, m])
// Keeping every iterate in both layouts (the Update epilogue writes X' and
// X'^T) makes all three the same NT kernel.  The symmetric products compute
// only lower-triangle tiles and write each tile twice (itself and its
// mirror), so S and P are exactly symmetric.
//
// Kernel shape: 256 threads = 4 waves in a 2x2 grid, square block tile of
// TILE x TILE, K-steps of 128 bytes per row (64 bf16 / 32 fp32), operands
// staged through LDS (double-buffered, 16-byte chunks XOR-swizzled by row),
// wave tiles of (TILE/2)^2 built from 32x32 MFMA blocks:
//   bf16: v_mfma_f32_32x32x16_bf16 (fp32 accumulate)
//   fp32: v_mfma_f32_32x32x2_f32
// All sizes are padded by the host to tile multiples (the padding is zero
// and stays zero through the iteration), so the main loop has no bounds
// checks; only the apply/store epilogues check against the true sizes.
#include <utility>

#include "mo_internal.h"

namespace mo {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // one 16-byte chunk

__device__ __forceinline__ float bf2f(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {          // bf16 storage
  static constexpr int kVec = 8;             // elements per 16-byte chunk
  __device__ static float ld(const uint16_t* p) { return bf2f(*p); }
  __device__ static void st(uint16_t* p, float v) { *p = f2bf(v); }
  __device__ static f32x16_t mma(u32x4 a, u32x4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ static float ld(const float* p) { return *p; }
  __device__ static void st(float* p, float v) { *p = v; }
  // The four fp32 of a lane's chunk feed four K=2 MFMAs; A and B use the
  // same component order, so the contraction covers all 8 K values.
  __device__ static f32x16_t mma(u32x4 a, u32x4 b, f32x16_t c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[0]), __uint_as_float(b[0]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[1]), __uint_as_float(b[1]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[2]), __uint_as_float(b[2]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[3]), __uint_as_float(b[3]), c, 0, 0, 0);
    return c;
  }
};

// Consecutive workgroup ids are dispatched round-robin over the 8 XCDs.
// Renumber so that each XCD owns one contiguous range of logical tiles and
// neighbouring tiles (which share operand panels) meet in the same L2.
__device__ __forceinline__ int xcd_remap(int wg, int total) {
  const int xcd = wg & 7, idx = wg >> 3;
  const int q = total >> 3, r = total & 7;
  return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

constexpr int kGroupM = 8;   // tile rows per swizzle group (non-symmetric)

// Calls f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>): the
// indices are constants from the start, so small per-thread arrays indexed
// by them are split into registers before any loop pass runs.
template <typename F, int... I>
__device__ __forceinline__ void unroll_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_impl(f, std::make_integer_sequence<int, N>{});
}

template <typename T, int TILE, int EPI>
__global__ __launch_bounds__(256) void ns_gemm_kernel(GemmArgs p) {
  using E = Elem<T>;
  constexpr bool kSym = (EPI == EPI_GRAM || EPI == EPI_POLY);
  constexpr int BK = 128 / sizeof(T);        // K elements per K-step
  constexpr int WT = TILE / 2;               // wave tile edge
  constexpr int FM = WT / 32;                // 32x32 blocks per wave edge
  constexpr int CH = TILE * 8 / 256;         // 16-byte chunks per thread per operand
  __shared__ u32x4 smem[2][2 * TILE * 8];

  const int tid = threadIdx.x;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int b = lid / p.tiles_per_mat;
  const int t = lid - b * p.tiles_per_mat;
  int ti, tj;
  if (kSym) {
    // lower-triangle enumeration: t = ti (ti + 1) / 2 + tj, tj <= ti
    int r = static_cast<int>((sqrtf(8.0f * t + 1.0f) - 1.0f) * 0.5f);
    while (r * (r + 1) / 2 > t) --r;
    while ((r + 1) * (r + 2) / 2 <= t) ++r;
    ti = r;
    tj = t - r * (r + 1) / 2;
  } else {
    const int per_group = kGroupM * p.tiles_n;
    const int g = t / per_group;
    const int first = g * kGroupM;
    const int gm = min(p.tiles_m - first, kGroupM);
    const int w = t - g * per_group;
    ti = first + w % gm;
    tj = w / gm;
  }

  const T* __restrict__ Ag = static_cast<const T*>(p.A) + b * p.sA + static_cast<int64_t>(ti) * TILE * p.lda;
  const T* __restrict__ Bg = static_cast<const T*>(p.B) + b * p.sB + static_cast<int64_t>(tj) * TILE * p.ldb;

  // Global -> register staging, one K-step ahead.  Thread tid moves the
  // 16-byte chunks tid + 256 i (row = chunk / 8, column chunk = chunk % 8);
  // rows advance by 32 per i, so the per-i offsets are constants.
  u32x4 ra[CH], rb[CH];
  const int srow = tid >> 3, sch = tid & 7;
  const T* __restrict__ Ab = Ag + srow * p.lda + sch * E::kVec;
  const T* __restrict__ Bb = Bg + srow * p.ldb + sch * E::kVec;
  const int lda32 = 32 * p.lda, ldb32 = 32 * p.ldb;
  const int soff0 = srow * 8 + (sch ^ (srow & 7));   // (srow + 32 i) & 7 == srow & 7
  auto gload = [&](int k0) {
    unroll<CH>([&](auto i) {
      ra[i] = *reinterpret_cast<const u32x4*>(Ab + i * lda32 + k0);
      rb[i] = *reinterpret_cast<const u32x4*>(Bb + i * ldb32 + k0);
    });
  };
  auto sstore = [&](int buf) {
    unroll<CH>([&](auto i) {
      smem[buf][soff0 + i * 256] = ra[i];
      smem[buf][TILE * 8 + soff0 + i * 256] = rb[i];
    });
  };

  const int lane = tid & 63, wave = tid >> 6;
  const int wr = (wave >> 1) * WT, wc = (wave & 1) * WT;
  const int l32 = lane & 31, lh = lane >> 5;

  f32x16_t acc[FM][FM];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // MFMA work of one K-step from LDS buffer `buf`.
  auto compute = [&](int buf) {
    const u32x4* sA = smem[buf];
    const u32x4* sB = smem[buf] + TILE * 8;
    unroll<4>([&](auto ks) {
      const int chunk = (ks * 2 + lh) ^ (l32 & 7);
      u32x4 fa[FM], fb[FM];
      unroll<FM>([&](auto f) {
        fa[f] = sA[(wr + f * 32 + l32) * 8 + chunk];
        fb[f] = sB[(wc + f * 32 + l32) * 8 + chunk];
      });
      unroll<FM>([&](auto i) {
        unroll<FM>([&](auto j) { acc[i][j] = E::mma(fa[i], fb[j], acc[i][j]); });
      });
    });
  };

  // Double-buffered main loop; the last K-step is peeled so that the loop
  // body has no branches and the staging registers stay in registers.
  const int nk = p.K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt + 1 < nk; ++kt) {
    gload((kt + 1) * BK);
    compute(kt & 1);
    sstore((kt + 1) & 1);
    __syncthreads();
  }
  compute((nk - 1) & 1);

  // ---------------------------------------------------------------- epilogue
  // 32x32 accumulator layout: lane (l32, lh), register r holds
  // row 8*(r/4) + 4*lh + (r%4), column l32 of the block.
  float s = 1.0f;
  if (p.rscale) {
    s = p.rscale[b];
    if (EPI == EPI_GRAM) s = s * s;
  }
  const int row0 = ti * TILE + wr, col0 = tj * TILE + wc;
  T* __restrict__ C = static_cast<T*>(p.C) + b * p.sC;
  const T* __restrict__ D = static_cast<const T*>(p.D) + (p.D ? b * p.sD : 0);
  constexpr bool kUsesD = (EPI != EPI_GRAM);

  // Visit every accumulator element with compile-time register indices.
  // For each 32x32 block the 16 epilogue operands D[gi][gj] are loaded
  // first, so their loads are in flight together.
  auto for_each_acc = [&](auto&& fn) {
    unroll<FM>([&](auto i) {
      unroll<FM>([&](auto j) {
        float dv[16];
        const int gj = col0 + j * 32 + l32;
        unroll<16>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          const int gi = row0 + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          dv[r] = kUsesD ? E::ld(D + static_cast<int64_t>(gi) * p.ldd + gj) : 0.0f;
        });
        unroll<16>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          const int gi = row0 + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          fn(gi, gj, acc[i][j][r], dv[r]);
        });
      });
    });
  };

  if constexpr (EPI == EPI_GRAM || EPI == EPI_POLY) {
    const bool diag = (ti == tj);
    for_each_acc([&](int gi, int gj, float v, float d) {
      if (diag && gi < gj) return;
      if (EPI == EPI_GRAM) v = s * v;
      else v = p.alpha * v + p.beta * d;
      E::st(C + static_cast<int64_t>(gi) * p.ldc + gj, v);
      if (gi != gj) E::st(C + static_cast<int64_t>(gj) * p.ldc + gi, v);
    });
  } else if constexpr (EPI == EPI_UPDATE) {
    T* __restrict__ Ct = static_cast<T*>(p.Ct) + b * p.sCt;
    for_each_acc([&](int gi, int gj, float a, float d) {
      const float v = s * (p.alpha * a + p.beta * d);
      E::st(C + static_cast<int64_t>(gi) * p.ldc + gj, v);
      E::st(Ct + static_cast<int64_t>(gj) * p.ldct + gi, v);
    });
  } else {
    // EPI_APPLY / EPI_STORE: x = s (acc + a X); write at the parameter's
    // natural position (transposed back when the matrix was oriented).
    const MatDesc md = p.desc[b];
    const int64_t ldw = md.oriented ? p.m_true : p.n_true;
    const float lrwd = p.lrwd;
    float sq = 0.0f;
    float* __restrict__ W = md.param;
    T* __restrict__ O = EPI == EPI_STORE ? static_cast<T*>(p.out) + b * p.s_out : nullptr;
    unroll<FM>([&](auto i) {
      unroll<FM>([&](auto j) {
        const int gj = col0 + j * 32 + l32;
        float dv[16], wv[16];
        int64_t off[16];
        bool ok[16];
        // all loads of the block first (operand X and, for apply, W)
        unroll<16>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          const int gi = row0 + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          ok[r] = gi < p.m_true && gj < p.n_true;
          off[r] = md.oriented ? static_cast<int64_t>(gj) * ldw + gi : static_cast<int64_t>(gi) * ldw + gj;
          dv[r] = E::ld(D + static_cast<int64_t>(gi) * p.ldd + gj);
          wv[r] = (EPI == EPI_APPLY && ok[r]) ? W[off[r]] : 0.0f;
        });
        unroll<16>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          if (!ok[r]) return;
          const float x = s * (p.alpha * acc[i][j][r] + p.beta * dv[r]);
          sq += x * x;
          if constexpr (EPI == EPI_APPLY) W[off[r]] = wv[r] - (lrwd * wv[r] + p.step * x);
          else E::st(O + off[r], x);
        });
      });
    });
    if (p.rms_part) {
      // block reduction of the squared update (deterministic, no atomics)
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 64);
      __syncthreads();                      // all waves are done with the LDS tiles
      float* red = reinterpret_cast<float*>(smem[0]);
      if (lane == 0) red[wave] = sq;
      __syncthreads();
      if (tid == 0)
        p.rms_part[static_cast<int64_t>(b) * p.tiles_per_mat + t] =
            (red[0] + red[1]) + (red[2] + red[3]);
    }
  }
}

int tile_size(TileCfg t) { return t == TILE_256 ? 256 : (t == TILE_128 ? 128 : 64); }

template <typename T, int TILE>
static hipError_t launch_t(Epi epi, const GemmArgs& a, hipStream_t s) {
  const int grid = a.tiles_per_mat * a.batch;
  switch (epi) {
    case EPI_GRAM:   hipLaunchKernelGGL((ns_gemm_kernel<T, TILE, EPI_GRAM>), dim3(grid), dim3(256), 0, s, a); break;
    case EPI_POLY:   hipLaunchKernelGGL((ns_gemm_kernel<T, TILE, EPI_POLY>), dim3(grid), dim3(256), 0, s, a); break;
    case EPI_UPDATE: hipLaunchKernelGGL((ns_gemm_kernel<T, TILE, EPI_UPDATE>), dim3(grid), dim3(256), 0, s, a); break;
    case EPI_APPLY:  hipLaunchKernelGGL((ns_gemm_kernel<T, TILE, EPI_APPLY>), dim3(grid), dim3(256), 0, s, a); break;
    case EPI_STORE:  hipLaunchKernelGGL((ns_gemm_kernel<T, TILE, EPI_STORE>), dim3(grid), dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int ns_dt, TileCfg cfg, Epi epi, const GemmArgs& a, hipStream_t s) {
  if (ns_dt == BF16) {
    switch (cfg) {
      case TILE_256: return launch_t<uint16_t, 256>(epi, a, s);
      case TILE_128: return launch_t<uint16_t, 128>(epi, a, s);
      case TILE_64:  return launch_t<uint16_t, 64>(epi, a, s);
    }
  } else {
    switch (cfg) {
      case TILE_256: return hipErrorInvalidValue;   // fp32 tiles stop at 128
      case TILE_128: return launch_t<float, 128>(epi, a, s);
      case TILE_64:  return launch_t<float, 64>(epi, a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace mo
