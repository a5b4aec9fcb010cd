// Newton-Schulz GEMMs on CDNA4 matrix cores (gfx950).
//
// Eq. 2 of "Muon is Scalable for LLM Training" (section 2.1) is evaluated as
// three products per iteration, all of the form C = A * B^T with both
// operands K-contiguous (row-major [rows, K]):
//   Gram    S = X X^T                  A = B = X ([m, n])             symmetric
//   Poly    P' = a I + b S + c S S^T   A = B = S (exactly symmetric)  symmetric
//   Update  X' = P' X                  A = P', B = X^T ([n, m])
// (a X + b S X + c S^2 X = (a I + b S + c S^2) X: the linear term rides in
// P', whose diagonal is near 1 on converged directions.)
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
//
// Operands live in the blocked layout of mo_layout.h: one K-stage of one
// row panel is a contiguous block that direct-to-LDS loads copy verbatim,
// and an output tile is a contiguous range, so the Gram, polynomial and
// update epilogues assemble the tile (and its mirror or transpose) in LDS
// and stream it out with coalesced 16-byte stores.
#include <utility>

#include "mo_internal.h"
#include "mo_layout.h"

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
  __device__ static float cvt(uint16_t h) { return bf2f(h); }
  __device__ static uint16_t pack(float v) { return f2bf(v); }
  // four consecutive elements (8-byte aligned) in one store
  __device__ static void store4(uint16_t* p, float a, float b, float c, float d) {
    uint2 q;
    q.x = static_cast<uint32_t>(f2bf(a)) | (static_cast<uint32_t>(f2bf(b)) << 16);
    q.y = static_cast<uint32_t>(f2bf(c)) | (static_cast<uint32_t>(f2bf(d)) << 16);
    *reinterpret_cast<uint2*>(p) = q;
  }
  __device__ static f32x16_t mma(u32x4 a, u32x4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ static float ld(const float* p) { return *p; }
  __device__ static void st(float* p, float v) { *p = v; }
  __device__ static float cvt(float v) { return v; }
  __device__ static float pack(float v) { return v; }
  __device__ static void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
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

constexpr int kGroupM = 8;   // tile rows per group of the tile order

// Tile order of a full tiles_m x tiles_n grid: groups of kGroupM tile rows,
// column-major inside a group, so that consecutive tiles (which run at the
// same time on one XCD) share few A and B panels.
__device__ __forceinline__ void grouped_tile(int t, int tiles_m, int tiles_n, int& ti, int& tj) {
  const int per_group = kGroupM * tiles_n;
  const int g = t / per_group;
  const int first = g * kGroupM;
  const int gm = min(tiles_m - first, kGroupM);
  const int w = t - g * per_group;
  ti = first + w % gm;
  tj = w / gm;
}

// The same order restricted to the lower triangle (tj <= ti) of a square
// grid: a group of rows [r0, r0 + gm) first runs its full columns
// tj < r0 column-major, then its own triangle.
__device__ __forceinline__ void sym_tile(int t, int tiles_m, int& ti, int& tj) {
  int r0 = 0, gm = 0;
  for (;;) {
    gm = min(tiles_m - r0, kGroupM);
    const int n = gm * r0 + gm * (gm + 1) / 2;
    if (t < n) break;
    t -= n;
    r0 += gm;
  }
  if (t < gm * r0) {
    ti = r0 + t % gm;
    tj = t / gm;
    return;
  }
  t -= gm * r0;
  int c = 0;
  while (t >= gm - c) {
    t -= gm - c;
    ++c;
  }
  tj = r0 + c;
  ti = r0 + c + t;
}

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

// s_waitcnt immediate (gfx9 encoding) that waits until at most `vm`
// vector-memory loads of this wave are outstanding; LDS and export
// counters are left unconstrained.
constexpr int waitcnt_vm(int vm) { return (vm & 15) | (((vm >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);   // lgkmcnt(0) only

#define MO_LDS(ptr) ((__attribute__((address_space(3))) void*)(ptr))

template <typename T, int TILE, int EPI>
__global__ __launch_bounds__(256) void ns_gemm_kernel(GemmArgs p) {
  using E = Elem<T>;
  constexpr bool kSym = (EPI == EPI_GRAM || EPI == EPI_POLY);
  constexpr int kRowBytes = 64;                   // bytes of a tile row per stage
  constexpr int BK = kRowBytes / sizeof(T);       // K elements per stage
  constexpr int CPR = kRowBytes / 16;             // 16-byte chunks per row (4)
  constexpr int NST = 4;                          // LDS stages (3 in flight)
  constexpr int WT = TILE / 2;                    // wave tile edge
  constexpr int FM = WT / 32;                     // 32x32 blocks per wave edge
  constexpr int OPS = TILE * CPR;                 // chunks of one operand per stage
  constexpr int STAGE = 2 * OPS;                  // chunks per stage (A then B)
  constexpr int RPI = 64 / CPR;                   // rows per wave-wide load (16)
  constexpr int INST = TILE / RPI / 4;            // loads per wave per operand per stage
  constexpr int DPW = 2 * INST;                   // loads per wave per stage
  __shared__ u32x4 smem[NST * STAGE];

  const int tid = threadIdx.x;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int b = lid / p.tiles_per_mat;
  const int t = lid - b * p.tiles_per_mat;
  int ti, tj;
  if (kSym) sym_tile(t, p.tiles_m, ti, tj);
  else grouped_tile(t, p.tiles_m, p.tiles_n, ti, tj);

  // row panels ti of A and tj of B: nk stages of TILE x BK each
  const int nk = p.K / BK;
  const int64_t stage_elems = static_cast<int64_t>(TILE) * BK;
  const T* __restrict__ Ag = static_cast<const T*>(p.A) + b * p.sA + static_cast<int64_t>(ti) * nk * stage_elems;
  const T* __restrict__ Bg = static_cast<const T*>(p.B) + b * p.sB + static_cast<int64_t>(tj) * nk * stage_elems;

  const int lane = tid & 63, wave = tid >> 6;
  const int wr = (wave >> 1) * WT, wc = (wave & 1) * WT;
  const int l32 = lane & 31, lh = lane >> 5;

  // Direct-to-LDS loads.  A stage of a panel is one contiguous block that
  // is already in the LDS order (64-byte rows, permuted chunks); a
  // wave-wide global_load_lds_dwordx4 copies 1 KiB of it (lane l moves the
  // 16 bytes at +16 l), and this wave's loads i cover 1 KiB pieces
  // wave*INST + i of the operand's block.
  const int goff = (wave * INST) * 64 * E::kVec + lane * E::kVec;
  // load q of this wave's DPW loads of stage kt into LDS buffer buf: even q
  // are pieces of A, odd q the matching pieces of B
  auto dma1 = [&](int buf, int kt, auto q) {
    constexpr int i = decltype(q)::value / 2;
    u32x4* st = smem + buf * STAGE + (q % 2 ? OPS : 0);
    const T* src = (q % 2 ? Bg : Ag) + static_cast<int64_t>(kt) * stage_elems + goff + i * 64 * E::kVec;
    __builtin_amdgcn_global_load_lds(static_cast<void*>(const_cast<T*>(src)), MO_LDS(st + (wave * INST + i) * 64), 16, 0, 0);
  };
  auto dma = [&](int buf, int kt) { unroll<DPW>([&](auto q) { dma1(buf, kt, q); }); };

  f32x16_t acc[FM][FM];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // A stage is two substeps of two 16-byte chunks per row.  Fragments of a
  // substep are read from LDS (set 0 / set 1 registers) while the MFMAs of
  // the other substep run.
  const int rsw = (l32 >> 2) & 3;               // slot swizzle of the rows this lane reads
  u32x4 fa[2][FM], fb[2][FM];
  // fragment read q of substep ks into register set `set`: even q read A
  // fragments, odd q B fragments
  auto frag1 = [&](int buf, auto ks, auto set, auto q) {
    constexpr int f = decltype(q)::value / 2;
    const u32x4* sA = smem + buf * STAGE;
    const int slot = (ks * 2 + lh) ^ rsw;
    if constexpr (decltype(q)::value % 2 == 0) fa[set][f] = sA[(wr + f * 32 + l32) * CPR + slot];
    else fb[set][f] = sA[OPS + (wc + f * 32 + l32) * CPR + slot];
  };
  constexpr int kGroups = FM * FM;              // MFMA groups (E::mma) per substep
  constexpr int kReads = 2 * FM;                // fragment reads per substep
  // The MFMAs of one substep, each followed by its share of other work:
  // fragment reads rd(q) front-loaded (their results are needed by the
  // next substep), loads ld(q) spread evenly.  A scheduling fence after
  // every group keeps this order, so memory instructions never queue up
  // in front of an MFMA.
  auto pipelined = [&](auto set, auto nld, auto&& rd, auto&& ld) {
    constexpr int kLd = std::decay_t<decltype(nld)>::value;
    unroll<kGroups>([&](auto g) {
      constexpr int G = decltype(g)::value;
      acc[G / FM][G % FM] = E::mma(fa[set][G / FM], fb[set][G % FM], acc[G / FM][G % FM]);
      constexpr int r0 = kReads <= kGroups ? G : G * kReads / kGroups;
      constexpr int r1 = kReads <= kGroups ? (G < kReads ? G + 1 : G) : (G + 1) * kReads / kGroups;
      unroll<r1 - r0>([&](auto k) { rd(std::integral_constant<int, r0 + decltype(k)::value>{}); });
      constexpr int l0 = G * kLd / kGroups, l1 = (G + 1) * kLd / kGroups;
      unroll<l1 - l0>([&](auto k) { ld(std::integral_constant<int, l0 + decltype(k)::value>{}); });
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto barrier = [&]() {                        // no memory fence: it would drain the loads
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using L0 = std::integral_constant<int, 0>;
  using LD = std::integral_constant<int, DPW>;
  auto no_ld = [](auto) {};

  // Main loop.  Stage kt lives in LDS buffer kt % NST.  Every iteration
  // issues exactly one stage of loads (stage kt + NST, or -- past the end
  // -- the last stage again into the buffer that has just been consumed),
  // so the number of loads in flight is the same at every barrier and the
  // loop body has no branch.  Before the barrier a wave waits until stage
  // kt + 1 of its own loads has landed (two later stages may still be in
  // flight) and its own LDS reads are done; after the barrier every wave's
  // part of stage kt + 1 is visible and buffer kt % NST (fully read) may be
  // refilled.  The barrier carries no memory fence: a fence would wait for
  // every outstanding load.
  for (int s = 0; s < NST; ++s) dma(s, min(s, nk - 1));
  __builtin_amdgcn_s_waitcnt(waitcnt_vm((NST - 1) * DPW));
  barrier();
  unroll<kReads>([&](auto q) { frag1(0, S0{}, S0{}, q); });
  __builtin_amdgcn_sched_barrier(0);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt % NST;
    pipelined(S0{}, L0{}, [&](auto q) { frag1(cur, S1{}, S1{}, q); }, no_ld);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((NST - 2) * DPW));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    barrier();
    const int nxt = (kt + 1) % NST;
    const int kl = min(kt + NST, nk - 1);
    pipelined(S1{}, LD{}, [&](auto q) { frag1(nxt, S0{}, S0{}, q); },
              [&](auto q) { dma1(cur, kl, q); });
  }
  // every load has landed and every wave is done with the staged tiles
  // before LDS is reused
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  barrier();

  // ---------------------------------------------------------------- epilogue
  // 32x32 accumulator layout: lane (l32, lh), register r holds
  // row 8*(r/4) + 4*lh + (r%4), column l32 of the block.
  float s = 1.0f;
  if (p.rscale) {
    s = p.rscale[b];
    if (EPI == EPI_GRAM) s = s * s;
  }
  const int row0 = ti * TILE + wr, col0 = tj * TILE + wc;
  const Blocked Lc = blocked(TILE, p.N, sizeof(T));       // C and D: [M, N]
  T* __restrict__ C = static_cast<T*>(p.C) + b * p.sC;
  const T* __restrict__ D = static_cast<const T*>(p.D) + (p.D ? b * p.sD : 0);

  // Tile-local position (rr, cc) inside an LDS copy of one output tile,
  // which has the blocked layout of the tile's contiguous global range:
  // TILE / BK stages of TILE rows x BK elements, chunks permuted per row.
  auto loff = [&](int rr, int cc) {
    const int st = cc / BK, c2 = cc - st * BK, ch = c2 / E::kVec;
    return (st * TILE + rr) * BK + ((ch ^ ((rr >> 2) & 3)) * E::kVec) + (c2 - ch * E::kVec);
  };
  // Visit every accumulator element with compile-time register indices,
  // passing tile-local coordinates; the visitor returns the element's new
  // value.
  auto for_each_acc = [&](auto&& fn) {
    unroll<FM>([&](auto i) {
      unroll<FM>([&](auto j) {
        unroll<16>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          const int rr = wr + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          const int cc = wc + j * 32 + l32;
          acc[i][j][r] = fn(rr, cc, acc[i][j][r]);
        });
      });
    });
  };
  T* const lt = reinterpret_cast<T*>(smem);                // TILE * TILE elements fit
  constexpr int kTileChunks = TILE * TILE * static_cast<int>(sizeof(T)) / 16;
  // LDS tile -> contiguous global range, 16 bytes per thread and step
  auto copy_out = [&](T* dst) {
    u32x4* g = reinterpret_cast<u32x4*>(dst);
    for (int c = tid; c < kTileChunks; c += 256) g[c] = smem[c];
  };

  if constexpr (EPI == EPI_GRAM || EPI == EPI_POLY || EPI == EPI_UPDATE) {
    if constexpr (EPI == EPI_POLY) {
      // the operand tile S[ti, tj] (same blocked layout as C) into LDS
      const u32x4* dsrc = reinterpret_cast<const u32x4*>(D + blk_tile(Lc, ti, tj));
      for (int c = tid; c < kTileChunks; c += 256) {
        const int wave_base = c - lane;                  // uniform across the wave
        __builtin_amdgcn_global_load_lds(dsrc + c, MO_LDS(smem + wave_base), 16, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      barrier();
    }
    const bool diag = kSym && (ti == tj);
    // finished values: back into the accumulators (for the transposed pass)
    // and into LDS at their own position; on diagonal tiles only the lower
    // triangle is kept, written to both positions, so S and P' stay
    // exactly symmetric
    for_each_acc([&](int rr, int cc, float a) {
      float v;
      if constexpr (EPI == EPI_POLY)
        v = p.alpha * a + p.beta * E::cvt(lt[loff(rr, cc)]) + (diag && rr == cc ? p.gamma : 0.0f);
      else if constexpr (EPI == EPI_GRAM)
        v = s * a;
      else
        v = s * a;
      if (!(diag && rr < cc)) {
        lt[loff(rr, cc)] = E::pack(v);
        if (diag && rr != cc) lt[loff(cc, rr)] = E::pack(v);
      }
      return v;
    });
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    barrier();
    copy_out(C + blk_tile(Lc, ti, tj));
    if (!diag) {
      // the mirror tile (symmetric products) or the transposed copy
      // (update): four consecutive rows of a lane are four consecutive
      // columns of the transposed tile, written as one LDS store
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      barrier();
      unroll<FM>([&](auto i) {
        unroll<FM>([&](auto j) {
          unroll<4>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            const int rr0 = wr + i * 32 + 8 * q + 4 * lh;
            const int cc = wc + j * 32 + l32;
            E::store4(lt + loff(cc, rr0), acc[i][j][4 * q], acc[i][j][4 * q + 1],
                      acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          });
        });
      });
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      barrier();
      if constexpr (EPI == EPI_UPDATE) {
        const Blocked Lt = blocked(TILE, p.M, sizeof(T));  // Ct: [N, M]
        copy_out(static_cast<T*>(p.Ct) + b * p.sCt + blk_tile(Lt, tj, ti));
      } else {
        copy_out(C + blk_tile(Lc, tj, ti));
      }
    }
  } else {
    // EPI_APPLY / EPI_STORE: x = s acc; write at the parameter's natural
    // position (transposed back when the matrix was oriented).
    const MatDesc md = p.desc[b];
    const int64_t ldw = md.oriented ? p.m_true : p.n_true;
    const float lrwd = p.lrwd;
    float sq = 0.0f;
    float* __restrict__ W = md.param;
    T* __restrict__ O = EPI == EPI_STORE ? static_cast<T*>(p.out) + b * p.s_out : nullptr;
    unroll<FM>([&](auto i) {
      unroll<FM>([&](auto j) {
        const int gj = col0 + j * 32 + l32;
        float wv[16];
        int64_t off[16];
        bool ok[16];
        // all loads of the block first (for apply: W)
        unroll<16>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          const int gi = row0 + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          ok[r] = gi < p.m_true && gj < p.n_true;
          off[r] = md.oriented ? static_cast<int64_t>(gj) * ldw + gi : static_cast<int64_t>(gi) * ldw + gj;
          wv[r] = (EPI == EPI_APPLY && ok[r]) ? W[off[r]] : 0.0f;
        });
        unroll<16>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          if (!ok[r]) return;
          const float x = s * acc[i][j][r];
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
      float* red = reinterpret_cast<float*>(smem);
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
