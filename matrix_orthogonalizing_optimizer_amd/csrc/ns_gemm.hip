// Newton-Schulz GEMMs on CDNA4 matrix cores (gfx950).
//
// Eq. 2 of "Muon is Scalable for LLM Training" (section 2.1) is evaluated as
// three products per iteration:
//   Gram    S = X X^T                  A = B = X ([m, n], row panels)  symmetric
//   Poly    P' = a I + b S + c S S^T   A = B = S (exactly symmetric)   symmetric
//   Update  X' = P' X                  A = P', B = X read K-major
// (a X + b S X + c S^2 X = (a I + b S + c S^2) X: the linear term rides in
// P', whose diagonal is near 1 on converged directions.)  The last update
// of a step is fused with the parameter update (apply) or with the output
// store.  The symmetric products compute only lower-triangle tiles and
// write each tile twice (itself and its mirror), so S and P are exactly
// symmetric.
//
// Kernel shape: NW = 4 or 8 waves in a 2 x (NW / 2) grid over a square
// TILE x TILE output tile; wave tiles of 32x32 MFMA blocks
//   bf16: v_mfma_f32_32x32x16_bf16 (fp32 accumulate)
//   fp32: v_mfma_f32_32x32x2_f32
// K-steps of 64 bytes per row (32 bf16 / 16 fp32), operands copied straight
// from global memory into a ring of LDS stages by direct-to-LDS loads, and
// fragments read from LDS (transposing reads for the K-major operand) one
// substep ahead of the MFMAs that use them.  With 8 waves two share each
// SIMD, so one wave's memory waits are covered by the other's MFMAs.
// All sizes are padded by the host to tile multiples (the padding is zero
// and stays zero through the iteration), so the main loop has no bounds
// checks; only the apply/store epilogues check against the true sizes.
//
// Operands live in the blocked layout of mo_layout.h: one K-stage of one
// row panel is a contiguous block that direct-to-LDS loads copy verbatim,
// and an output tile is a contiguous range, so the Gram, polynomial and
// update epilogues assemble the tile (and its mirror) in LDS and stream it
// out with coalesced 16-byte stores.
#include <utility>

#include "mo_internal.h"
#include "mo_layout.h"
#include "ns_common.h"

namespace mo {

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

// Super-block tile order for large matrices (tile counts multiples of 16).
// The 256 tiles that run at once over the whole chip (8 XCDs x 32 CUs) form
// one 16 x 16 block of tiles of one matrix; XCD x takes the 8 x 4 sub-block
// at rows 8 (x % 2), columns 4 (x / 2).  The chip then streams 16 row and 16
// column panels at a time instead of 12 per XCD, so what one XCD misses in
// its L2 another has usually just brought into the chip-wide cache.
// w: this XCD's tile index within the matrix; nsc: column super-blocks.
__device__ __forceinline__ void super_gen(int w, int x, int nsc, int& ti, int& tj) {
  const int sg = w >> 5, r = w & 31;
  const int sr = sg / nsc, sc = sg - sr * nsc;
  ti = sr * 16 + (x & 1) * 8 + (r & 7);
  tj = sc * 16 + (x >> 1) * 4 + (r >> 3);
}
// Diagonal super-blocks of the symmetric products: the 136 lower tiles of a
// 16 x 16 block split into 8 compact regions of 17 tiles, one per XCD.  In
// 4 x 4 groups of tiles the block has six full squares and four triangles
// of 10: XCDs 0-5 take one square each plus one tile of a triangle on the
// same panel groups, XCDs 6 and 7 take the rest of two triangles each.
// Each region touches 8 distinct panels of the (single) operand matrix.
// Entries are 16 * row + column within the block.
__constant__ unsigned char kDiagTiles[8][17] = {
    {64, 80, 96, 112, 65, 81, 97, 113, 66, 82, 98, 114, 67, 83, 99, 115, 51},
    {132, 148, 164, 180, 133, 149, 165, 181, 134, 150, 166, 182, 135, 151, 167, 183, 119},
    {196, 212, 228, 244, 197, 213, 229, 245, 198, 214, 230, 246, 199, 215, 231, 247, 118},
    {128, 144, 160, 176, 129, 145, 161, 177, 130, 146, 162, 178, 131, 147, 163, 179, 187},
    {200, 216, 232, 248, 201, 217, 233, 249, 202, 218, 234, 250, 203, 219, 235, 251, 186},
    {192, 208, 224, 240, 193, 209, 225, 241, 194, 210, 226, 242, 195, 211, 227, 243, 255},
    {0, 16, 17, 32, 33, 34, 48, 49, 50, 68, 84, 85, 100, 101, 102, 116, 117},
    {136, 152, 153, 168, 169, 170, 184, 185, 204, 220, 221, 236, 237, 238, 252, 253, 254}};

// Lower triangle of a square grid: super-blocks (sr, sc <= sr) in order;
// an off-diagonal block gives each XCD its 8 x 4 sub-block (32 tiles), a
// diagonal block (136 tiles) gives each XCD its region of kDiagTiles (17
// tiles).  (Giving XCD x the lower parts of rows x and 15 - x instead
// touches all 16 panels per XCD: Gram 2.5% and the whole large-matrix step
// 0.8% slower.)
__device__ __forceinline__ void super_sym(int w, int x, int& ti, int& tj) {
  int sr = 0;
  while (w >= 32 * sr + 17) {                    // tiles of super-row sr for one XCD
    w -= 32 * sr + 17;
    ++sr;
  }
  const int sc = w >> 5;
  if (sc < sr) {
    const int r = w & 31;
    ti = sr * 16 + (x & 1) * 8 + (r & 7);
    tj = sc * 16 + (x >> 1) * 4 + (r >> 3);
  } else {
    const int e = kDiagTiles[x][w - 32 * sr];
    ti = sr * 16 + (e >> 4);
    tj = sr * 16 + (e & 15);
  }
}


template <typename T, int TILE, int EPI, int NW>
__global__ __launch_bounds__(64 * NW) void ns_gemm_kernel(GemmArgs p) {
  using E = Elem<T>;
  constexpr bool kSym = (EPI == EPI_GRAM || EPI == EPI_POLY);
  // Products with X as the second factor (X' = P' X) read B = X in its own
  // row-major blocked layout, i.e. K-major: stage kt is rows [32 kt, 32 kt
  // + 32) of X restricted to this tile's columns, and fragments are taken
  // with transposing LDS reads.  The MFMA operands are swapped for them so
  // that each lane ends up with four consecutive columns of one row of the
  // result (one 8- or 16-byte store).
  constexpr bool kNN = (EPI == EPI_UPDATE || EPI == EPI_APPLY || EPI == EPI_STORE);
  constexpr int kRowBytes = 64;                   // bytes of a tile row per stage
  constexpr int BK = kRowBytes / sizeof(T);       // K elements per stage
  constexpr int CPR = kRowBytes / 16;             // 16-byte chunks per row (4)
  // NW waves in a 2 x (NW / 2) grid; with 8 waves two share each SIMD and
  // cover each other's waits, and three LDS stages (two in flight) suffice.
  constexpr int NT = 64 * NW;                     // threads
  constexpr int NST = NW == 8 ? 3 : 4;            // LDS stages
  constexpr int WM = TILE / 2;                    // wave tile rows
  constexpr int WN = TILE / (NW / 2);             // wave tile columns
  constexpr int FMM = WM / 32, FMN = WN / 32;     // 32x32 blocks per wave tile
  constexpr int OPS = TILE * CPR;                 // chunks of one operand per stage
  constexpr int STAGE = 2 * OPS;                  // chunks per stage (A then B)
  constexpr int INST = OPS / 64 / NW;             // 1 KiB loads per wave per operand per stage
  constexpr int DPW = 2 * INST;                   // loads per wave per stage
  static_assert(INST >= 1 && OPS % (64 * NW) == 0, "stage split over the waves");
  // The apply/store epilogue stages the fp32 update through LDS in passes
  // of kPR tile rows, as [kPR][TILE + 4] (parameter rows = tile rows) or
  // [TILE][kPR + 4] (oriented parameters: parameter rows = tile columns).
  constexpr bool kApply = (EPI == EPI_APPLY || EPI == EPI_STORE);
  constexpr int kPR = TILE == 256 ? 128 : TILE;
  constexpr int kApplyFloats = TILE * (kPR + 4) > kPR * (TILE + 4) ? TILE * (kPR + 4) : kPR * (TILE + 4);
  // LDS: the main loop's stages, and what the epilogue stages -- the whole
  // output tile (Gram, polynomial, update) or one apply pass
  constexpr int kEpiChunks = kApply ? kApplyFloats / 4 : TILE * TILE * static_cast<int>(sizeof(T)) / 16;
  constexpr int kSmemChunks = kEpiChunks > NST * STAGE ? kEpiChunks : NST * STAGE;
  static_assert(kSmemChunks * 16 <= 160 * 1024, "LDS per workgroup");
  __shared__ u32x4 smem[kSmemChunks];

  const int tid = threadIdx.x;
  // Workgroup ids are dispatched round-robin over the 8 XCDs: this XCD's
  // k-th workgroup takes the k-th tile of the XCD's share, walking the
  // groups from group (xcd mod nbins) on; each group's share is a
  // contiguous eighth of its tiles.
  const int xcd = blockIdx.x & 7;
  int k = blockIdx.x >> 3, bi = -1, lid = 0;
  for (int jj = 0; jj < p.nbins; ++jj) {
    const int bj = p.rotate ? (xcd + jj) % p.nbins : jj;
    const int total = p.bin[bj].tiles_per_mat * p.bin[bj].batch;
    const int q = total >> 3, r = total & 7;
    const int cnt = q + (xcd < r ? 1 : 0);
    if (k < cnt) {
      bi = bj;
      lid = xcd * q + min(xcd, r) + k;
      break;
    }
    k -= cnt;
  }
  if (bi < 0) return;                           // this XCD has no more tiles
  const GemmBin& g = p.bin[bi];
  int b, t, ti, tj;
  if (g.super_order) {
    // tiles_per_mat is a multiple of 8: every XCD runs tiles_per_mat / 8
    // tiles of each matrix, matrices in order
    const int per = g.tiles_per_mat >> 3;
    b = k / per;
    const int w = k - b * per;
    if (kSym) {
      super_sym(w, xcd, ti, tj);
      t = ti * (ti + 1) / 2 + tj;
    } else {
      super_gen(w, xcd, g.tiles_n >> 4, ti, tj);
      t = ti * g.tiles_n + tj;
    }
  } else {
    b = lid / g.tiles_per_mat;
    t = lid - b * g.tiles_per_mat;
    if (kSym) sym_tile(t, g.tiles_m, ti, tj);
    else grouped_tile(t, g.tiles_m, g.tiles_n, ti, tj);
  }

  // row panels ti of A and tj of B: nk stages of TILE x BK each, of which
  // the first nkl are visited (the rest multiply zero padding)
  const int nk = g.K / BK;
  const int nkl = g.k_loop;
  const int64_t stage_elems = static_cast<int64_t>(TILE) * BK;
  const T* __restrict__ Ag = static_cast<const T*>(g.A) + b * g.sA + static_cast<int64_t>(ti) * nk * stage_elems;
  const T* __restrict__ Bg = kNN ? static_cast<const T*>(g.B) + b * g.sB
                                  : static_cast<const T*>(g.B) + b * g.sB + static_cast<int64_t>(tj) * nk * stage_elems;
  // K-major B: X is blocked [K / TILE panels][N / BK column stages][TILE][BK];
  // the 32 (bf16) or 16 (fp32) rows of stage kt in column stage c form one
  // contiguous block of BK rows x 64 bytes
  constexpr int kSPT = TILE / BK;                 // column stages per tile
  constexpr int kBlkBytes = BK * 64;              // bytes of one such block
  static_assert((kSPT & (kSPT - 1)) == 0, "stages per tile: a power of two");
  // elements between consecutive 128/256-row panels of X (N / BK blocks of
  // TILE x BK each)
  const int64_t panel_elems = static_cast<int64_t>(g.N / BK) * TILE * BK;
  auto b_koff = [&](int kt) -> int64_t {          // elements: stage kt's row block (kt >= 0)
    const uint32_t uk = static_cast<uint32_t>(kt);
    return static_cast<int64_t>(uk / kSPT) * panel_elems + static_cast<int64_t>((uk % kSPT) * BK * BK);
  };

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const int wr = (wave / (NW / 2)) * WM, wc = (wave % (NW / 2)) * WN;
  const int l32 = lane & 31, lh = lane >> 5;

  // Direct-to-LDS loads.  A stage of a panel is one contiguous block that
  // is already in the LDS order (64-byte rows, permuted chunks); a
  // wave-wide global_load_lds_dwordx4 copies 1 KiB of it (lane l moves the
  // 16 bytes at +16 l), and this wave's loads i cover 1 KiB pieces
  // wave*INST + i of the operand's block.
  // The address of a load is a wave-uniform base (scalar registers) plus
  // this lane's 16 l, so the main loop does no per-lane address arithmetic.
  const uint32_t lane16 = static_cast<uint32_t>(lane * 16);
  // load q of this wave's DPW loads of stage kt into LDS buffer buf: even q
  // are pieces of A, odd q the matching pieces of B
  auto dma1 = [&](int buf, int kt, auto q) {
    constexpr int i = decltype(q)::value / 2;
    constexpr bool isB = decltype(q)::value % 2;
    u32x4* st = smem + buf * STAGE + (isB ? OPS : 0);
    const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_addr(st + (wave * INST + i) * 64));
    if constexpr (kNN && isB) {
      // piece wave*INST + i: 1 KiB of column stage (piece / (kBlkBytes / 1 KiB))
      const int piece = wave * INST + i;
      const int c = piece * 1024 / kBlkBytes, within = piece * 1024 - c * kBlkBytes;
      const char* base = reinterpret_cast<const char*>(
          Bg + b_koff(kt) + static_cast<int64_t>(tj * kSPT + c) * TILE * BK) + within;
      lds_dma16(base, lane16, lds);
    } else {
      const char* base = reinterpret_cast<const char*>((isB ? Bg : Ag) + static_cast<int64_t>(kt) * stage_elems) +
                         (wave * INST + i) * 1024;
      lds_dma16(base, lane16, lds);
    }
  };
  auto dma = [&](int buf, int kt) { unroll<DPW>([&](auto q) { dma1(buf, kt, q); }); };

  f32x16_t acc[FMM][FMN];
#pragma unroll
  for (int i = 0; i < FMM; ++i)
#pragma unroll
    for (int j = 0; j < FMN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // A stage is two substeps of two 16-byte chunks per row.  Fragments of a
  // substep are read from LDS (set 0 / set 1 registers) while the MFMAs of
  // the other substep run.
  const int rsw = (l32 >> 2) & 3;               // slot swizzle of the rows this lane reads
  u32x4 fa[2][FMM], fb[2][FMN];
  // B fragment of column block f from a K-major stage ([kSPT][BK rows][BK],
  // chunks permuted per row): this lane's column n = wc + 32 f + l32 and its
  // K values of substep ks.
  //   bf16: two ds_read_b64_tr_b16, four K each.  Within each 16-lane group
  //   lane i points at row k0 + i / 4, columns n0 + 4 (i % 4) .. + 3, and the
  //   read returns to lane i the four rows k0 .. k0 + 3 of column n0 + i.
  //   fp32: the four K values of the lane's chunk one by one.
  auto frag_kmajor = [&](const T* sB, auto ks, auto f) -> u32x4 {
    constexpr int F = decltype(f)::value, KS = decltype(ks)::value;
    auto at = [&](int k, int n) {                 // element offset of (k, n) in the stage
      const int c = n / BK, c2 = n - c * BK, ch = c2 / E::kVec;
      return c * BK * BK + k * BK + ((ch ^ ((k >> 2) & 3)) * E::kVec) + (c2 - ch * E::kVec);
    };
    u32x4 r;
    if constexpr (sizeof(T) == 2) {
      const int gi = lane & 15;
      const int n = wc + 32 * F + (l32 & 16) + 4 * (gi & 3);
      unroll<2>([&](auto h) {
        const int k = KS * 16 + 8 * lh + 4 * decltype(h)::value + (gi >> 2);
        const v4s16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s16_t*)(sB + at(k, n)));
        const uint2 u = __builtin_bit_cast(uint2, v);
        r[2 * decltype(h)::value] = u.x;
        r[2 * decltype(h)::value + 1] = u.y;
      });
    } else {
      const int n = wc + 32 * F + l32;
      unroll<4>([&](auto t) {
        const int k = (KS * 2 + lh) * 4 + decltype(t)::value;
        r[decltype(t)::value] = __float_as_uint(reinterpret_cast<const float*>(sB)[at(k, n)]);
      });
    }
    return r;
  };
  // fragment read q of substep ks into register set `set`: A and B
  // fragments alternate (A0 B0 A1 B1 ...), the surplus of the longer side
  // last, so the first MFMAs of the next substep have their operands early
  constexpr int kPair = FMM < FMN ? FMM : FMN;
  auto frag1 = [&](int buf, auto ks, auto set, auto q) {
    constexpr int Q = decltype(q)::value;
    constexpr bool isA = Q < 2 * kPair ? (Q % 2 == 0) : (FMM > FMN);
    constexpr int f = Q < 2 * kPair ? Q / 2 : Q - kPair;
    const u32x4* sA = smem + buf * STAGE;
    const int slot = (ks * 2 + lh) ^ rsw;
    if constexpr (isA) {
      fa[set][f] = sA[(wr + f * 32 + l32) * CPR + slot];
    } else if constexpr (!kNN) {
      fb[set][f] = sA[OPS + (wc + f * 32 + l32) * CPR + slot];
    } else {
      fb[set][f] = frag_kmajor(reinterpret_cast<const T*>(sA + OPS), ks, std::integral_constant<int, f>{});
    }
  };
  constexpr int kGroups = FMM * FMN;            // MFMA groups (E::mma) per substep
  constexpr int kReads = FMM + FMN;             // fragment reads per substep
  // The MFMAs of one substep, each followed by its share of other work:
  // fragment reads rd(q) front-loaded (their results are needed by the
  // next substep), loads ld(q) spread evenly.  A scheduling fence after
  // every group keeps this order, so memory instructions never queue up
  // in front of an MFMA.
  auto pipelined = [&](auto set, auto nld, auto&& rd, auto&& ld) {
    constexpr int kLd = std::decay_t<decltype(nld)>::value;
    unroll<kGroups>([&](auto g) {
      constexpr int G = decltype(g)::value;
      constexpr int I = G / FMN, J = G % FMN;
      if constexpr (kNN)
        acc[I][J] = E::mma(fb[set][J], fa[set][I], acc[I][J]);
      else
        acc[I][J] = E::mma(fa[set][I], fb[set][J], acc[I][J]);
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

  // Polynomial product, bf16: the epilogue's b S term is taken from the B
  // operand while it streams through.  The tile's S[rows ti, cols tj] equals
  // S[cols tj, rows ti] (S is exactly symmetric), and that block is the B
  // panel (rows tj) at the K-stages of tile ti's columns: the stage of
  // accumulator row block i is kSPT ti + wr / 32 + i.  In the B fragment of
  // column block j a lane (l32, lh) holds S[row wc + 32 j + l32 of panel tj]
  // at K offsets 16 ks + 8 lh + 0..7; accumulator registers 4 q + e need the
  // K offsets 8 q + 4 lh + e: for q = 2 ks + lh the lane's own elements
  // 4 lh .. 4 lh + 3, for the other q the same elements of lane l ^ 32.
  // They are added as (b / c) S, so that the epilogue's c acc gives
  // c S S + b S.  This is the 8-wave bf16 kernel's only path (the host runs
  // c = 0 with 4 waves); the others read S in the epilogue.
  constexpr bool kCapture = (EPI == EPI_POLY) && sizeof(T) == 2 && NW == 8;
  constexpr bool cap = kCapture;
  const float bc = cap ? p.beta / p.alpha : 0.0f;
  const int cap_kt = kCapture ? (TILE / BK) * ti + wr / BK : 0;
  // adds (b / c) S for accumulator row block I from register set `set`
  // (substep ks of the stage cap_kt + I)
  auto capture = [&](auto i, auto set, auto ks) {
    constexpr int I = decltype(i)::value, KS = decltype(ks)::value;
    unroll<FMN>([&](auto j) {
      constexpr int J = decltype(j)::value;
      const u32x4 f = fb[set][J];
      const uint32_t own0 = lh ? f[2] : f[0], own1 = lh ? f[3] : f[1];
      const uint32_t oth0 = lane_xor32(lh ? f[0] : f[2]), oth1 = lane_xor32(lh ? f[1] : f[3]);
      const uint32_t a0 = lh ? oth0 : own0, a1 = lh ? oth1 : own1;   // q = 2 ks
      const uint32_t b0 = lh ? own0 : oth0, b1 = lh ? own1 : oth1;   // q = 2 ks + 1
      constexpr int R = 8 * KS;
      acc[I][J][R + 0] += bc * __uint_as_float(a0 << 16);
      acc[I][J][R + 1] += bc * __uint_as_float(a0 & 0xffff0000u);
      acc[I][J][R + 2] += bc * __uint_as_float(a1 << 16);
      acc[I][J][R + 3] += bc * __uint_as_float(a1 & 0xffff0000u);
      acc[I][J][R + 4] += bc * __uint_as_float(b0 << 16);
      acc[I][J][R + 5] += bc * __uint_as_float(b0 & 0xffff0000u);
      acc[I][J][R + 6] += bc * __uint_as_float(b1 << 16);
      acc[I][J][R + 7] += bc * __uint_as_float(b1 & 0xffff0000u);
    });
  };

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
  for (int s = 0; s < NST; ++s) dma(s, min(s, nkl - 1));
  __builtin_amdgcn_s_waitcnt(waitcnt_vm((NST - 1) * DPW));
  barrier();
  unroll<kReads>([&](auto q) { frag1(0, S0{}, S0{}, q); });
  __builtin_amdgcn_sched_barrier(0);
  // one stage: substep 0, wait + barrier, substep 1 with the next stage's
  // loads; capI >= 0 adds the captured b S of row block capI (see above)
  // `cb` is the stage's buffer, kt % NST: a compile-time constant in the
  // loop unrolled by NST, so the LDS addresses of the fragment reads are too
  auto iteration = [&](int kt, auto capi, auto cb) __attribute__((always_inline)) {
    constexpr int CI = decltype(capi)::value;
    const int cur = cb;
    pipelined(S0{}, L0{}, [&](auto q) { frag1(cur, S1{}, S1{}, q); }, no_ld);
    if constexpr (CI >= 0) capture(capi, S0{}, S0{});
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((NST - 2) * DPW));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    barrier();
    const int nxt = cur + 1 == NST ? 0 : cur + 1;
    const int kl = min(kt + NST, nkl - 1);
    pipelined(S1{}, LD{}, [&](auto q) { frag1(nxt, S0{}, S0{}, q); },
              [&](auto q) { dma1(cur, kl, q); });
    if constexpr (CI >= 0) capture(capi, S1{}, S1{});
  };
  using NoCap = std::integral_constant<int, -1>;
  // stages [k0, k1): single stages up to a multiple of NST, then blocks of
  // NST with compile-time buffers, then the rest.  (The 4-wave 256 tile has
  // no registers to spare for the unrolled body.)
  constexpr bool kUnroll = !(TILE == 256 && NW == 4);
  auto run_range = [&](int k0, int k1) __attribute__((always_inline)) {
    int kt = k0;
    if constexpr (kUnroll) {
      for (; kt < k1 && kt % NST != 0; ++kt) iteration(kt, NoCap{}, kt % NST);
      for (; kt + NST <= k1; kt += NST)
        unroll<NST>([&](auto u) {
          iteration(kt + decltype(u)::value, NoCap{}, std::integral_constant<int, decltype(u)::value>{});
        });
    }
    for (; kt < k1; ++kt) iteration(kt, NoCap{}, kt % NST);
  };
  if constexpr (!cap) {
    run_range(0, nkl);
  } else {
    // the FMM capture stages unrolled, so every accumulator index is a
    // compile-time constant
    // With K trimmed to the true m, capture stages at or past nkl hold
    // only S's zero padding and are skipped; every wave still runs exactly
    // nkl iterations (one barrier each), so the barriers stay matched.
    run_range(0, min(cap_kt, nkl));
    unroll<FMM>([&](auto i) {
      const int kt = cap_kt + decltype(i)::value;
      if (kt < nkl) iteration(kt, i, kt % NST);
    });
    run_range(cap_kt + FMM, nkl);
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
  if (p.use_rscale) {
    s = g.rscale[b];
    if (EPI == EPI_GRAM) s = s * s;
  }
  const Blocked Lc = blocked(TILE, g.N, sizeof(T));       // C and D: [M, N]
  T* __restrict__ C = static_cast<T*>(g.C) + b * g.sC;
  const T* __restrict__ D = static_cast<const T*>(g.D) + (g.D ? b * g.sD : 0);

  // Tile-local position (rr, cc) inside an LDS copy of one output tile,
  // which has the blocked layout of the tile's contiguous global range:
  // TILE / BK stages of TILE rows x BK elements, chunks permuted per row.
  auto loff = [&](int rr, int cc) {
    const int st = cc / BK, c2 = cc - st * BK, ch = c2 / E::kVec;
    return (st * TILE + rr) * BK + ((ch ^ ((rr >> 2) & 3)) * E::kVec) + (c2 - ch * E::kVec);
  };
  T* const lt = reinterpret_cast<T*>(smem);                // TILE * TILE elements fit
  static_assert(kApply || kSmemChunks * 16 >= TILE * TILE * static_cast<int>(sizeof(T)), "tile staging");
  constexpr int kTileChunks = TILE * TILE * static_cast<int>(sizeof(T)) / 16;
  // LDS tile -> contiguous global range: 16 bytes per thread and step, eight
  // steps' loads in flight before their stores.  The stores are
  // non-temporal: the next product reads the output after every tile of
  // this one is written, and a whole output is larger than the caches, so
  // keeping it would only evict operand panels other tiles still read.
  auto copy_out = [&](T* dst) {
    u32x4* g = reinterpret_cast<u32x4*>(dst);
    constexpr int kIter = kTileChunks / NT;
    constexpr int kB = kIter < 8 ? kIter : 8;
#pragma unroll
    for (int c0 = 0; c0 < kIter; c0 += kB) {
      u32x4 v[kB];
      unroll<kB>([&](auto k) { v[decltype(k)::value] = smem[tid + (c0 + decltype(k)::value) * NT]; });
      unroll<kB>([&](auto k) { __builtin_nontemporal_store(v[decltype(k)::value], &g[tid + (c0 + decltype(k)::value) * NT]); });
    }
  };

  if constexpr (EPI == EPI_UPDATE) {
    // X' = s acc.  The swapped MFMA operands leave in register r of block
    // (i, j) the element at row wr + 32 i + l32, column wc + 32 j + 8 q + 4 lh
    // + e of the tile (q = r / 4, e = r % 4): four consecutive columns, one
    // store into the LDS copy of the tile, then one coalesced copy-out.
    int on[4];
    unroll<4>([&](auto q) { on[q] = loff(wr + l32, wc + 8 * q + 4 * lh); });
    unroll<FMM>([&](auto i) {
      unroll<FMN>([&](auto j) {
        unroll<4>([&](auto q) {
          constexpr int I = decltype(i)::value, J = decltype(j)::value, Q = decltype(q)::value;
          const int o = on[Q] + 32 * I * BK + (32 * J / BK) * TILE * BK;
          E::store4(lt + o, s * acc[I][J][4 * Q], s * acc[I][J][4 * Q + 1], s * acc[I][J][4 * Q + 2],
                    s * acc[I][J][4 * Q + 3]);
        });
      });
    });
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    barrier();
    copy_out(C + blk_tile(Lc, ti, tj));
  } else if constexpr (EPI == EPI_GRAM || EPI == EPI_POLY) {
    // Accumulator element (i, j, r) sits at tile row wr + 32 i + 8 q + 4 lh
    // + e (q = r / 4, e = r % 4) and column wc + 32 j + l32.  Its LDS offset
    // is a per-lane base plus a compile-time displacement:
    //   direct    (rr, cc): od[q % 2] + (32 i + 8 (q - q % 2) + e) BK
    //                        + (32 j / BK) TILE BK
    //   transposed (cc, rr): ot[q] + (32 i / BK) TILE BK + 32 j BK + e,
    //                        the four e consecutive (one 8- or 16-byte access)
    // (whole 32-row / 32-column steps keep the chunk permutation, which
    // depends on bits 2-3 of the row only).
    int od[2], ot[4];
    unroll<2>([&](auto q) { od[q] = loff(wr + 8 * q + 4 * lh, wc + l32); });
    unroll<4>([&](auto q) { ot[q] = loff(wc + l32, wr + 8 * q + 4 * lh); });
    auto doff = [&](auto i, auto j, auto r) {
      constexpr int I = decltype(i)::value, J = decltype(j)::value, R = decltype(r)::value;
      constexpr int Q = R / 4, e = R % 4;
      return od[Q % 2] + (32 * I + 8 * (Q - Q % 2) + e) * BK + (32 * J / BK) * TILE * BK;
    };
    auto toff = [&](auto i, auto j, auto q) {
      constexpr int I = decltype(i)::value, J = decltype(j)::value, Q = decltype(q)::value;
      return ot[Q] + (32 * I / BK) * TILE * BK + 32 * J * BK;
    };
    const bool diag = kSym && (ti == tj);

    if constexpr (EPI == EPI_POLY) {
      if constexpr (cap) {
        // b S is already in the accumulators (captured in the main loop)
        unroll<FMM>([&](auto i) {
          unroll<FMN>([&](auto j) {
            unroll<16>([&](auto r) {
              acc[decltype(i)::value][decltype(j)::value][decltype(r)::value] *= p.alpha;
            });
          });
        });
      } else {
        // b S + a I from the mirror tile S[tj, ti] (S is exactly symmetric):
        // element (rr, cc) of this tile is (cc, rr) there, so each lane reads
        // its four consecutive rows with one access
        const u32x4* dsrc = reinterpret_cast<const u32x4*>(D + blk_tile(Lc, tj, ti));
        for (int c = tid; c < kTileChunks; c += NT) {
          const int wave_base = c - lane;                  // uniform across the wave
          __builtin_amdgcn_global_load_lds(static_cast<void*>(const_cast<u32x4*>(dsrc + c)),
                                           MO_LDS(smem + wave_base), 16, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        barrier();
        unroll<FMM>([&](auto i) {
          unroll<FMN>([&](auto j) {
            unroll<4>([&](auto q) {
              constexpr int I = decltype(i)::value, J = decltype(j)::value, Q = decltype(q)::value;
              float d[4];
              E::load4(lt + toff(i, j, q), d);
              unroll<4>([&](auto e) {
                constexpr int R = 4 * Q + decltype(e)::value;
                acc[I][J][R] = p.alpha * acc[I][J][R] + p.beta * d[decltype(e)::value];
              });
            });
          });
        });
      }
      if (diag) {
        // a I on the blocks that straddle the diagonal
        unroll<FMM>([&](auto i) {
          unroll<FMN>([&](auto j) {
            constexpr int I = decltype(i)::value, J = decltype(j)::value;
            if (wr + 32 * I == wc + 32 * J) {
              unroll<16>([&](auto r) {
                constexpr int R = decltype(r)::value;
                if (l32 == 8 * (R / 4) + 4 * lh + (R % 4)) acc[I][J][R] += p.gamma;
              });
            }
          });
        });
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      barrier();                                  // the S tile is no longer needed
    } else {
      unroll<FMM>([&](auto i) {
        unroll<FMN>([&](auto j) {
          unroll<16>([&](auto r) {
            acc[decltype(i)::value][decltype(j)::value][decltype(r)::value] *= s;
          });
        });
      });
    }

    // transposed pass: value (rr, cc) to LDS position (cc, rr), four rows of
    // a lane in one store.  This is the mirror tile; on a diagonal tile it
    // puts every value at its mirror position and the direct pass below
    // then overwrites the lower triangle, leaving the tile exactly
    // symmetric.
    unroll<FMM>([&](auto i) {
      unroll<FMN>([&](auto j) {
        unroll<4>([&](auto q) {
          constexpr int I = decltype(i)::value, J = decltype(j)::value, Q = decltype(q)::value;
          E::store4(lt + toff(i, j, q), acc[I][J][4 * Q], acc[I][J][4 * Q + 1], acc[I][J][4 * Q + 2],
                    acc[I][J][4 * Q + 3]);
        });
      });
    });
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    barrier();
    if (!diag) {
      copy_out(C + blk_tile(Lc, tj, ti));
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      barrier();
    }
    // direct pass: value (rr, cc) to LDS position (rr, cc); on a diagonal
    // tile only the lower triangle rr >= cc
    auto direct_block = [&](auto i, auto j, bool lower_only) {
      constexpr int I = decltype(i)::value, J = decltype(j)::value;
      unroll<8>([&](auto h) {
        constexpr int R0 = 2 * decltype(h)::value;
        const int o0 = doff(i, j, std::integral_constant<int, R0>{});
        const int o1 = doff(i, j, std::integral_constant<int, R0 + 1>{});
        if (!lower_only) {
          E::store2(lt + o0, lt + o1, acc[I][J][R0], acc[I][J][R0 + 1]);
        } else {
          // rows 8 q + 4 lh + e against column l32 of the same 32x32 block
          const int rel = 8 * (R0 / 4) + 4 * lh + (R0 % 4);
          if (rel >= l32) E::store1(lt + o0, acc[I][J][R0]);
          if (rel + 1 >= l32) E::store1(lt + o1, acc[I][J][R0 + 1]);
        }
      });
    };
    if (!diag) {
      unroll<FMM>([&](auto i) { unroll<FMN>([&](auto j) { direct_block(i, j, false); }); });
    } else {
      unroll<FMM>([&](auto i) {
        unroll<FMN>([&](auto j) {
          const int br = wr + 32 * decltype(i)::value, bc = wc + 32 * decltype(j)::value;
          if (br > bc) direct_block(i, j, false);
          else if (br == bc) direct_block(i, j, true);
        });
      });
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    barrier();
    copy_out(C + blk_tile(Lc, ti, tj));
  } else {
    // EPI_APPLY / EPI_STORE: x = s acc, applied at the parameter's natural
    // position (transposed back when the matrix was oriented):
    //   W <- W - (lr wd W + lr scale x)   or   out <- x.
    // Each pass stages kPR tile rows of x (fp32) in LDS in the parameter's
    // orientation; then every thread handles groups of four elements that
    // are consecutive along a parameter row: one 16-byte LDS read, one
    // 16-byte load and store of W.
    if constexpr (EPI == EPI_APPLY) {
      if (p.rms_only) {
        // sum of squares of x = s acc only (the scale pass of the
        // update-norm scaling); padded rows and columns hold exact zeros
        float sq = 0.0f;
        unroll<FMM>([&](auto i) {
          unroll<FMN>([&](auto j) {
            unroll<16>([&](auto r) {
              const float x = s * acc[decltype(i)::value][decltype(j)::value][decltype(r)::value];
              sq += x * x;
            });
          });
        });
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 64);
        float* red = reinterpret_cast<float*>(smem);
        if (lane == 0) red[wave] = sq;
        __syncthreads();
        if (tid == 0) {
          float tot = 0.0f;
#pragma unroll
          for (int w = 0; w < NW; ++w) tot += red[w];
          g.rms_part[static_cast<int64_t>(b) * g.tiles_per_mat + t] = tot;
        }
        return;
      }
    }
    const MatDesc md = g.desc[b];
    const bool ori = md.oriented != 0;
    const int64_t ldw = ori ? g.m_true : g.n_true;         // parameter row length
    const int wrows = ori ? g.n_true : g.m_true;            // parameter rows
    const float lrwd = p.lrwd, stp = g.step_dev ? g.step_dev[b] : g.step;
    // global address space: plain global loads and stores, not flat ones
    typedef __attribute__((address_space(1))) float gfloat;
    typedef __attribute__((address_space(1))) T gT;
    gfloat* __restrict__ W = (gfloat*)md.param;
    gT* __restrict__ O = EPI == EPI_STORE ? (gT*)(static_cast<T*>(g.out) + b * g.s_out) : nullptr;
    float* const lf = reinterpret_cast<float*>(smem);
    // padded LDS row lengths (consecutive lanes write consecutive rows)
    constexpr int kLd = TILE + 4, kLdT = kPR + 4;
    const bool full = (ti + 1) * TILE <= g.m_true && (tj + 1) * TILE <= g.n_true && (ldw % 4) == 0;
    float sq = 0.0f;
    using True = std::integral_constant<bool, true>;
    using False = std::integral_constant<bool, false>;
    // x of this wave's accumulator blocks whose rows fall in pass `pc` into
    // LDS: [kPR][kLd] rows of W, or [TILE][kLdT] (oriented: W rows are tile
    // columns).  Lane l32 holds row 32 i + l32 and four consecutive columns.
    auto stage = [&](auto pc, auto oric) {
      constexpr int pass = decltype(pc)::value;
      constexpr bool kOri = decltype(oric)::value;
      const int r_base = wr - pass * kPR;
      unroll<FMM>([&](auto i) {
        unroll<FMN>([&](auto j) {
          unroll<4>([&](auto q) {
            constexpr int I = decltype(i)::value, J = decltype(j)::value, Q = decltype(q)::value;
            const int rr = r_base + 32 * I + l32;
            const int cc = wc + 32 * J + 8 * Q + 4 * lh;
            const float x0 = s * acc[I][J][4 * Q], x1 = s * acc[I][J][4 * Q + 1];
            const float x2 = s * acc[I][J][4 * Q + 2], x3 = s * acc[I][J][4 * Q + 3];
            if constexpr (kOri) {
              lf[(cc + 0) * kLdT + rr] = x0;
              lf[(cc + 1) * kLdT + rr] = x1;
              lf[(cc + 2) * kLdT + rr] = x2;
              lf[(cc + 3) * kLdT + rr] = x3;
            } else {
              *reinterpret_cast<float4*>(lf + rr * kLd + cc) = make_float4(x0, x1, x2, x3);
            }
          });
        });
      });
    };
    // Group g of a pass: four elements consecutive along one parameter row.
    // Returns the LDS offset; sets the parameter row and column.
    auto group = [&](auto pc, auto oric, int g, int& wrow, int& wcol) {
      constexpr int pass = decltype(pc)::value;
      if constexpr (decltype(oric)::value) {
        const int cc = g / (kPR / 4), r4 = (g % (kPR / 4)) * 4;
        wrow = tj * TILE + cc;
        wcol = ti * TILE + pass * kPR + r4;
        return cc * kLdT + r4;
      } else {
        const int r = g / (TILE / 4), c4 = (g % (TILE / 4)) * 4;
        wrow = ti * TILE + pass * kPR + r;
        wcol = tj * TILE + c4;
        return r * kLd + c4;
      }
    };
    constexpr int kGroups = kPR * TILE / 4;                 // groups per pass
    constexpr int kU = kGroups >= NT * 8 ? 8 : kGroups / NT;
    static_assert(kU >= 1 && kGroups % (NT * kU) == 0, "group loop");
    // Row length a multiple of 4: every group of four lies wholly inside or
    // wholly outside the parameter, so groups go as 16-byte accesses.  A
    // tile inside the parameter needs no check (guard false); a ragged one
    // skips the groups outside.  All of a step's loads (LDS x, W) are
    // issued before any store.
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(1))) f32x4_t gf4;
    auto copy_full = [&](auto pc, auto oric, auto guardc) {
      constexpr bool kGuard = decltype(guardc)::value;
#pragma unroll 1
      for (int g0 = 0; g0 < kGroups; g0 += NT * kU) {
        f32x4_t xv[kU], wv[kU];
        int64_t off[kU];
        bool in[kU];
        unroll<kU>([&](auto u) {
          constexpr int U = decltype(u)::value;
          int wrow, wcol;
          const int lo = group(pc, oric, g0 + U * NT + tid, wrow, wcol);
          in[U] = !kGuard || (wrow < wrows && wcol < ldw);
          off[U] = static_cast<int64_t>(wrow) * ldw + wcol;
          xv[U] = *reinterpret_cast<const f32x4_t*>(lf + lo);
          if constexpr (EPI == EPI_APPLY) {
            if (in[U]) wv[U] = *(const gf4*)(W + off[U]);
          }
        });
        unroll<kU>([&](auto u) {
          constexpr int U = decltype(u)::value;
          if (!in[U]) return;
          const f32x4_t x = xv[U];
          if constexpr (EPI == EPI_APPLY) {
            const f32x4_t w = wv[U];
            *(gf4*)(W + off[U]) = w - (lrwd * w + stp * x);
          } else {
            E::store4((T*)(O + off[U]), x[0], x[1], x[2], x[3]);
          }
          sq += (x[0] * x[0] + x[1] * x[1]) + (x[2] * x[2] + x[3] * x[3]);
        });
      }
    };
    // row length not a multiple of 4: element by element
    auto copy_edge = [&](auto pc, auto oric) {
#pragma unroll 1
      for (int g = tid; g < kGroups; g += NT) {
        int wrow, wcol;
        const int lo = group(pc, oric, g, wrow, wcol);
        if (wrow >= wrows) continue;
        const int64_t off = static_cast<int64_t>(wrow) * ldw + wcol;
        unroll<4>([&](auto k) {
          constexpr int K = decltype(k)::value;
          if (wcol + K < ldw) {
            const float x = lf[lo + K];
            if constexpr (EPI == EPI_APPLY) {
              const float w = W[off + K];
              W[off + K] = w - (lrwd * w + stp * x);
            } else {
              E::st((T*)(O + off + K), x);
            }
            sq += x * x;
          }
        });
      }
    };
    constexpr int kNP = TILE / kPR;
    auto run = [&](auto oric) {
      unroll<kNP>([&](auto pc) {
        if (decltype(pc)::value > 0) barrier();             // previous pass fully read
        if (wr / kPR == decltype(pc)::value) stage(pc, oric);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        barrier();
        if (full) copy_full(pc, oric, False{});
        else if ((ldw % 4) == 0) copy_full(pc, oric, True{});
        else copy_edge(pc, oric);
      });
    };
    if (ori) run(True{});
    else run(False{});
    if (g.rms_part) {
      // block reduction of the squared update (deterministic, no atomics)
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 64);
      barrier();                                            // LDS reads of the last pass done
      float* red = reinterpret_cast<float*>(smem);
      if (lane == 0) red[wave] = sq;
      __syncthreads();
      if (tid == 0) {
        float tot = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) tot += red[w];
        g.rms_part[static_cast<int64_t>(b) * g.tiles_per_mat + t] = tot;
      }
    }
  }
}

int tile_size(TileCfg t) { return t == TILE_256 ? 256 : (t == TILE_128 ? 128 : 64); }

template <typename T, int TILE, int NW>
static hipError_t launch_t(Epi epi, const GemmArgs& a, hipStream_t s) {
  const dim3 grid(8 * a.per_xcd), block(64 * NW);
  switch (epi) {
    case EPI_GRAM:   hipLaunchKernelGGL((ns_gemm_kernel<T, TILE, EPI_GRAM, NW>), grid, block, 0, s, a); break;
    case EPI_POLY:   hipLaunchKernelGGL((ns_gemm_kernel<T, TILE, EPI_POLY, NW>), grid, block, 0, s, a); break;
    case EPI_UPDATE: hipLaunchKernelGGL((ns_gemm_kernel<T, TILE, EPI_UPDATE, NW>), grid, block, 0, s, a); break;
    case EPI_APPLY:  hipLaunchKernelGGL((ns_gemm_kernel<T, TILE, EPI_APPLY, NW>), grid, block, 0, s, a); break;
    case EPI_STORE:  hipLaunchKernelGGL((ns_gemm_kernel<T, TILE, EPI_STORE, NW>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int ns_dt, TileCfg cfg, Epi epi, int waves, const GemmArgs& a, hipStream_t s) {
  if (ns_dt == BF16) {
    switch (cfg) {
      case TILE_256: return waves == 8 ? launch_t<uint16_t, 256, 8>(epi, a, s) : launch_t<uint16_t, 256, 4>(epi, a, s);
      case TILE_128: return launch_t<uint16_t, 128, 4>(epi, a, s);
      case TILE_64:  return launch_t<uint16_t, 64, 4>(epi, a, s);
    }
  } else {
    switch (cfg) {
      case TILE_256: return hipErrorInvalidValue;   // fp32 tiles stop at 128
      case TILE_128: return launch_t<float, 128, 4>(epi, a, s);
      case TILE_64:  return launch_t<float, 64, 4>(epi, a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace mo
