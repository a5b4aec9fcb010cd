// Fused Newton-Schulz for small matrices (m <= 128, bf16), gfx950.
//
// Eq. 2 of "Muon is Scalable for LLM Training" (section 2.1) on an oriented
// [m, n] matrix with m <= 128, one 512-thread workgroup per matrix, all N
// iterations and the apply of section 2.2, Eq. 4 in one kernel.  Every
// quantity of the iteration is a polynomial in the Gram matrix, so the
// kernel iterates on m x m matrices and touches X only twice:
//   S_0 = r^2 X_0 X_0^T                 (X_0 streamed, r = 1/(|N|+eps))
//   for k < N:  P_k = a I + b S_k + c S_k S_k
//               S_{k+1} = P_k S_k P_k   (= X_{k+1} X_{k+1}^T)
//               Q_{k+1} = P_k Q_k       (Q_1 = P_0)
//   X_N = r Q_N X_0                     (X_0 streamed again)
//   W <- W - (lr wd W + step X_N)
// X_{k+1} = P_k X_k gives X_N = P_{N-1} .. P_0 X_0 exactly; S, P and Q are
// symmetric and commute.  The Gram-space recursion amplifies the rounding
// of S in the directions of small singular values, so the m x m products
// run at about fp32 precision: S, P and Q are fp32, and each product is
// three bf16 matrix-core products of split operands, A B ~ Ah Bh + Ah Bl +
// Al Bh with Ah = bf16(A), Al = bf16(A - Ah) (16 significant bits per
// operand, fp32 accumulation).  X_0 enters exactly (bf16 storage of the
// momentum kernel's N); X_N = r X_0^T (Qh + Ql), transposed.  The bf16
// iterates X_k of the general kernels are never formed, so this path is
// the more accurate of the two (about 2e-3 against the fp64 oracle at
// [128, 2048], N = 5, against 7e-3).  The host runs it for N <= 5 only:
// rounding can turn the Gram eigenvalue of a direction with a tiny
// singular value negative, and P S P then grows it by about a^2 per step,
// unbounded (from N = 8 on this can overflow on rank-deficient inputs).
//
// Waves: 8.  The X_0 X_0^T product gives each wave a 64 x 32 part (2 x 4
// grid of 32x32 MFMA blocks).  The m x m products give each wave a
// 128 x 16 column strip (eight 16x16 blocks, v_mfma_f32_16x16x32_bf16):
// lane (l16, lq) holds rows 16 i + 4 lq + e, column 16 w + l16.  That
// register layout is directly a B operand of the next product when the K
// values of each 32-block are taken in the order 4 lq + e, 16 + 4 lq + e,
// and the A operand (the whole matrix, from LDS) is stored in that order.
#include "mo_internal.h"
#include "mo_layout.h"
#include "ns_common.h"

namespace mo {

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kT = 128;                 // panel height / output tile edge
constexpr int kBK = 32;                 // bf16 elements per 64-byte row piece
constexpr int kCPR = 4;                 // 16-byte chunks per row piece
constexpr int kNT = 512;                // threads
constexpr int kStage = kT * kCPR;       // chunks of one [128 rows][64 B] stage (8 KiB)
constexpr int kSub = 2;                 // K-stages per ring slot (one barrier per slot)
constexpr int kSlot = kSub * kStage;
// A split m x m matrix is two arrays (hi, lo) of [128 rows][16 chunks]:
// logical chunk c = 4 kb + lq of row r holds columns 32 kb + 4 lq + 0..3
// and 32 kb + 16 + 4 lq + 0..3 (8 bf16) and sits at position c ^ (r & 15)
// of the row.  Reads of 16 rows x 4 chunks (the A fragments) and the
// stores of a strip then fall on distinct banks; a row pitch of 17 chunks
// (the usual pad) leaves the reads with two-way conflicts on gfx950.
constexpr int kMat = kT * 16;           // chunks of one array (32 KiB)
constexpr int kOffSh = 0, kOffSl = kMat;            // S
constexpr int kOffPh = 2 * kMat, kOffPl = 3 * kMat; // P
constexpr int kOffEnd = 4 * kMat;
constexpr int kApLd = kT + 4;           // padded fp32 row (S_0 staging, apply staging)
// fp32 [128][kApLd] staging (S_0 before the iteration, X_N tiles in the
// apply) from the start of P on; it runs past the end of P.
constexpr int kOffStage = kOffPh;
constexpr int kStageChunks = kT * kApLd * 4 / 16;
constexpr int kLdsChunks = kOffStage + kStageChunks > kOffEnd ? kOffStage + kStageChunks : kOffEnd;
// X_0 streams through a ring of 16 KiB slots, all but one in flight: 8
// slots over S and P while S_0 is accumulated, 4 over S in the last
// product (the apply stages its tile above them meanwhile).  The fp32 S_0
// is staged once the first ring has drained.
constexpr int kNSTG = 8, kOffRingG = 0;
constexpr int kNSTA = 4, kOffRingA = 0;
static_assert(kNSTG * kSlot <= kOffEnd, "S_0 ring fits over S and P");
static_assert(kOffRingA + kNSTA * kSlot <= kOffStage, "last ring fits below the staging");
static_assert(kLdsChunks * 16 <= 160 * 1024, "LDS");

// Position of logical chunk c of row r of a split matrix.
__device__ __forceinline__ int sw_chunk(int r, int c) { return r * 16 + (c ^ (r & 15)); }

__device__ __forceinline__ f32x4_t mma16(const u32x4& a, const u32x4& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// v = hi + lo: hi = bf16(v) (nearest even), lo = bf16(v - hi); eight values
// (two groups of four) packed as bf16x8.
__device__ __forceinline__ void split8(const f32x4_t& v0, const f32x4_t& v1, u32x4& hi, u32x4& lo) {
  const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t h = pack_bf16x2(v[2 * q], v[2 * q + 1]);
    hi[q] = h;
    lo[q] = pack_bf16x2(v[2 * q] - __uint_as_float(h << 16), v[2 * q + 1] - __uint_as_float(h & 0xffff0000u));
  }
}

typedef float f4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) f4v gf4v;

}  // namespace

__global__ __launch_bounds__(512) void ns_small_kernel(SmallArgs p) {
  using T = uint16_t;
  using E = Elem<T>;
  __shared__ u32x4 smem[kLdsChunks];

  // matrix of this workgroup
  int bi = 0, b = blockIdx.x;
  while (bi + 1 < p.nbins && b >= p.bin[bi].count) {
    b -= p.bin[bi].count;
    ++bi;
  }
  const SmallBin& g = p.bin[bi];
  if (b >= g.count) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = (wave >> 2) * 64, wc = (wave & 3) * 32;
  const int l32 = lane & 31, lh = lane >> 5;
  const int rsw = (l32 >> 2) & 3;
  const int l16 = lane & 15, lq = lane >> 4;
  const int cs = 16 * wave;               // this wave's column strip of the m x m products
  const int nkx = g.n_pad / kBK;          // K-stages of X_0
  const int ntj = g.n_pad / kT;           // 128-column tiles
  const float r0 = g.rscale[b];
  const T* const x0 = static_cast<const T*>(g.x0) + b * g.x_stride;
  const uint32_t lane16 = static_cast<uint32_t>(lane * 16);

  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto lds_sync = [&]() {                 // own LDS accesses done, then barrier
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    barrier();
  };
  // X_0 stages stream through a ring of slots of kSub stages at chunk
  // `ring`; the stages are contiguous in the blocked layout (128 rows x 64
  // bytes each, one 1 KiB piece per wave)
  auto dma_stage = [&](int ring, int buf, int kt2) {
    unroll<kSub>([&](auto h) {
      constexpr int H = decltype(h)::value;
      const char* src = reinterpret_cast<const char*>(x0 + (kSub * kt2 + H) * (kT * kBK)) + wave * 1024;
      lds_dma16(src, lane16,
                __builtin_amdgcn_readfirstlane(lds_addr(smem + ring + buf * kSlot + H * kStage + wave * 64)));
    });
  };
  const int nk2 = nkx / kSub;             // n_pad is a multiple of 128

  // -------- S_0 = r^2 X_0 X_0^T: rows wr.., columns wc.. of this wave
  f32x16_t accs[2];
  unroll<2>([&](auto i) { unroll<16>([&](auto r) { accs[decltype(i)::value][decltype(r)::value] = 0.0f; }); });
  // NT operand rows of a [128 rows][64 B] stage at chunk `base`: this
  // lane's row `row`, K offsets 16 ks + 8 lh .. + 7
  auto frag_nt = [&](int base, int row, int ks) -> u32x4 {
    return smem[base + row * kCPR + ((ks * 2 + lh) ^ rsw)];
  };
  // One barrier per slot: before it a wave waits until its own pieces of
  // slot kt2 have landed (the next kNSTG - 2 slots may still be in flight)
  // and its LDS reads are done; after it every wave's part of slot kt2 is
  // visible and slot kt2 - 1 has been fully read, so its buffer takes slot
  // kt2 + kNSTG - 1.  Past the end the last slot is loaded again, so the
  // number of loads in flight is the same at every wait.
  for (int s = 0; s < kNSTG - 1; ++s) dma_stage(kOffRingG, s, min(s, nk2 - 1));
  for (int kt2 = 0; kt2 < nk2; ++kt2) {
    const int cur = kt2 % kNSTG;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((kNSTG - 2) * kSub));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    barrier();
    dma_stage(kOffRingG, cur == 0 ? kNSTG - 1 : cur - 1, min(kt2 + kNSTG - 1, nk2 - 1));
    unroll<kSub>([&](auto h) {
      const int base = kOffRingG + cur * kSlot + decltype(h)::value * kStage;
      unroll<2>([&](auto ks) {
        const u32x4 fb = frag_nt(base, wc + l32, decltype(ks)::value);
        unroll<2>([&](auto i) {
          const u32x4 fa = frag_nt(base, wr + 32 * decltype(i)::value + l32, decltype(ks)::value);
          accs[decltype(i)::value] = E::mma(fa, fb, accs[decltype(i)::value]);
        });
      });
    });
  }
  // every load has landed and every wave is done with the ring before the
  // fp32 S_0 is staged over it
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  lds_sync();
  float* const lf0 = reinterpret_cast<float*>(smem + kOffStage);
  unroll<2>([&](auto i) {
    unroll<16>([&](auto r) {
      constexpr int I = decltype(i)::value, R = decltype(r)::value;
      const int row = wr + 32 * I + 8 * (R / 4) + 4 * lh + (R % 4);
      lf0[row * kApLd + wc + l32] = r0 * r0 * accs[I][R];
    });
  });
  lds_sync();

  // -------- the m x m iteration
  // A strip D[i][e] = D[16 i + 4 lq + e][cs + l16] of a symmetric matrix is
  // stored (as its transpose, i.e. row cs + l16) into a split matrix; the
  // eight values of K-block kb are chunk 4 kb + lq of that row.
  auto store_split = [&](int off_hi, int off_lo, const f32x4_t (&D)[8]) {
    unroll<4>([&](auto kb) {
      constexpr int KB = decltype(kb)::value;
      u32x4 hi, lo;
      split8(D[2 * KB], D[2 * KB + 1], hi, lo);
      const int c = sw_chunk(cs + l16, 4 * KB + lq);
      smem[off_hi + c] = hi;
      smem[off_lo + c] = lo;
    });
  };
  // A strip kept split in registers (H[kb], L[kb]: the eight values of
  // K-block kb), and stored from there.
  auto split_strip = [](const f32x4_t (&D)[8], u32x4 (&H)[4], u32x4 (&L)[4]) {
    unroll<4>([&](auto kb) {
      constexpr int KB = decltype(kb)::value;
      split8(D[2 * KB], D[2 * KB + 1], H[KB], L[KB]);
    });
  };
  auto store_hl = [&](int off_hi, int off_lo, const u32x4 (&H)[4], const u32x4 (&L)[4]) {
    unroll<4>([&](auto kb) {
      constexpr int KB = decltype(kb)::value;
      const int c = sw_chunk(cs + l16, 4 * KB + lq);
      smem[off_hi + c] = H[KB];
      smem[off_lo + c] = L[KB];
    });
  };
  // B operand sources of the products: an fp32 strip split K-block by
  // K-block as it is consumed, or a strip kept split.
  auto b_f32 = [](const f32x4_t (&B)[8]) {
    return [&B](auto kb, u32x4& h, u32x4& l) {
      constexpr int KB = decltype(kb)::value;
      split8(B[2 * KB], B[2 * KB + 1], h, l);
    };
  };
  auto b_split = [](const u32x4 (&H)[4], const u32x4 (&L)[4]) {
    return [&H, &L](auto kb, u32x4& h, u32x4& l) {
      h = H[decltype(kb)::value];
      l = L[decltype(kb)::value];
    };
  };
  // D += A B: A the split matrix at (off_hi, off_lo), B this wave's strip
  // of a symmetric matrix in registers; three products per block.  The 32
  // (K-block, row-block) steps run as one sequence with the A fragments
  // read two steps ahead, so that each step's LDS reads are in flight under
  // the two previous steps' products.
  auto prod = [&](int off_hi, int off_lo, auto&& b_of, f32x4_t (&D)[8]) {
    auto a_at = [&](int kb, int i) { return sw_chunk(16 * i + l16, 4 * kb + lq); };
    u32x4 ah = smem[off_hi + a_at(0, 0)], al = smem[off_lo + a_at(0, 0)];
    u32x4 ah1 = smem[off_hi + a_at(0, 1)], al1 = smem[off_lo + a_at(0, 1)];
    u32x4 bh, bl;
    unroll<32>([&](auto t) {
      constexpr int T = decltype(t)::value, KB = T / 8, I = T % 8;
      if constexpr (I == 0) b_of(std::integral_constant<int, KB>{}, bh, bl);
      u32x4 nh, nl;
      if constexpr (T + 2 < 32) {
        nh = smem[off_hi + a_at((T + 2) / 8, (T + 2) % 8)];
        nl = smem[off_lo + a_at((T + 2) / 8, (T + 2) % 8)];
      }
      D[I] = mma16(ah, bh, D[I]);
      D[I] = mma16(ah, bl, D[I]);
      D[I] = mma16(al, bh, D[I]);
      ah = ah1;
      al = al1;
      if constexpr (T + 2 < 32) {
        ah1 = nh;
        al1 = nl;
      }
    });
  };
  auto zero8 = [](f32x4_t (&D)[8]) {
    unroll<8>([&](auto i) { D[decltype(i)::value] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}; });
  };

  // this wave's strip of S_0 (its rows cs.. of the staged copy, S_0 being
  // symmetric), then S_0 split into LDS.  P and Q are kept split in
  // registers: P is split once for its store and the B operand of S P, Q
  // once per step for the next P Q and, at the end, X_N.
  f32x4_t Ss[8], D[8];
  u32x4 ph[4], pl[4], qh[4], ql[4];
  unroll<8>([&](auto i) {
    constexpr int I = decltype(i)::value;
    const float4 v = *reinterpret_cast<const float4*>(lf0 + (cs + l16) * kApLd + 16 * I + 4 * lq);
    Ss[I] = f32x4_t{v.x, v.y, v.z, v.w};
  });
  store_split(kOffSh, kOffSl, Ss);
  lds_sync();                             // S split visible; staged S_0 read (P may be written)

  for (int k = 0; k < p.ns_steps; ++k) {
    const bool last = k + 1 == p.ns_steps;
    // P_k = a I + b S + c S S
    zero8(D);
    prod(kOffSh, kOffSl, b_f32(Ss), D);
    {
      f32x4_t Ps[8];
      unroll<8>([&](auto i) {
        constexpr int I = decltype(i)::value;
        unroll<4>([&](auto e) {
          constexpr int Ei = decltype(e)::value;
          float v = p.c * D[I][Ei] + p.b * Ss[I][Ei];
          if (16 * I + 4 * lq + Ei == cs + l16) v += p.a;
          Ps[I][Ei] = v;
        });
      });
      split_strip(Ps, ph, pl);
    }
    store_hl(kOffPh, kOffPl, ph, pl);
    lds_sync();
    // Q_{k+1} = P_k Q_k (P from LDS)
    if (k == 0) {
      unroll<4>([&](auto kb) {
        qh[decltype(kb)::value] = ph[decltype(kb)::value];
        ql[decltype(kb)::value] = pl[decltype(kb)::value];
      });
    } else {
      zero8(D);
      prod(kOffPh, kOffPl, b_split(qh, ql), D);
      split_strip(D, qh, ql);
    }
    if (!last) {
      // S_{k+1} = P (S P): T = S P first; every wave has read S before
      // S_{k+1} replaces it
      zero8(D);
      prod(kOffSh, kOffSl, b_split(ph, pl), D);
      lds_sync();
      zero8(Ss);
      prod(kOffPh, kOffPl, b_f32(D), Ss);
      store_split(kOffSh, kOffSl, Ss);
    }
    lds_sync();                           // P read by all; S_{k+1} visible
  }

  // -------- X_N = r Q X_0, 128 columns at a time, as (X_0^T Q)^T: for a
  // column tile j, D[n][c] = sum_k X_0[k][128 j + n] Q[k][c], with this
  // wave's columns c = cs.. of Q (B, kept split) and X_0^T (A) read from
  // the streamed stages with transposing LDS reads.
  // A fragment: X_0 rows 32 kb + 4 lq + 0..3 and 32 kb + 16 + 4 lq + 0..3
  // of column 16 ii + l16 of a [128 rows][32] stage at chunk `base`.
  // Within each 16-lane group lane i points at row k0 + i / 4, columns
  // n0 + 4 (i % 4) .. + 3, and the read returns to lane i the four rows
  // k0 .. k0 + 3 of column n0 + i.
  auto frag_tr = [&](int base, int kb, int ii) -> u32x4 {
    const T* st = reinterpret_cast<const T*>(smem + base);
    u32x4 r;
    unroll<2>([&](auto h) {
      const int kr = 32 * kb + 16 * decltype(h)::value + 4 * lq + (l16 >> 2);
      const int n = 16 * ii + 4 * (l16 & 3);
      const int off = kr * kBK + (((n >> 3) ^ ((kr >> 2) & 3)) << 3) + (n & 7);
      const v4s16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s16_t*)(st + off));
      const uint2 u = __builtin_bit_cast(uint2, v);
      r[2 * decltype(h)::value] = u.x;
      r[2 * decltype(h)::value + 1] = u.y;
    });
    return r;
  };

  const MatDesc md = g.desc[b];
  const bool ori = md.oriented != 0;
  float* const lf = reinterpret_cast<float*>(smem + kOffStage);
  float* const W = md.param;
  const int64_t ldw = ori ? g.m_true : g.n_true;
  float sq = 0.0f;
  constexpr int kG = kT * kT / 4 / kNT;   // 16-byte W groups per thread and tile
  // Group u of this thread in a full W tile: row rr, columns c4 .. c4 + 3 of
  // the tile in W's orientation.  A global (not generic) pointer, so that
  // the compiler's waits for these accesses count vector-memory operations
  // only and do not drain the ring's loads in flight.
  auto w_at = [&](int j, int u) -> gf4v* {
    const int gidx = tid + u * kNT, rr = gidx >> 5, c4 = (gidx & 31) * 4;
    const int64_t row0 = ori ? static_cast<int64_t>(j) * kT : 0;
    const int64_t col0 = ori ? 0 : static_cast<int64_t>(j) * kT;
    return (gf4v*)(W + (row0 + rr) * ldw + col0 + c4);
  };
  // Every tile is a full 128 x 128 block of W (m = 128 and n a multiple of
  // 128): each tile's W loads are issued right after the tile's last ring
  // slot, so that they are in flight under the tile's second half of
  // products and the staging, and no load the compiler does not track
  // follows them (its waits for W then hold back nothing else).  Loads
  // complete in order, so a ring wait counts the loads issued after its
  // slot: at least 12 from the second tile on (two slots and one tile's W
  // loads), 4 (two slots) in the first.  Otherwise W is read after the
  // staging, as a batch for full tiles or element by element for ragged
  // ones, and the ring waits as in the X_0 X_0^T loop.
  auto tile_loop = [&](auto full_c) {
    constexpr bool kFull = decltype(full_c)::value;
    for (int s = 0; s < kNSTA - 1; ++s) dma_stage(kOffRingA, s, min(s, nk2 - 1));
    for (int j = 0; j < ntj; ++j) {
      f4v w[kG];
      zero8(D);
      unroll<2>([&](auto u) {             // the tile's two ring slots
        const int kt2 = 2 * j + decltype(u)::value, cur = kt2 % kNSTA;
        if (kFull && j > 0) {
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kSub + kG));
        } else {
          __builtin_amdgcn_s_waitcnt(waitcnt_vm((kNSTA - 2) * kSub));
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        barrier();
        dma_stage(kOffRingA, cur == 0 ? kNSTA - 1 : cur - 1, min(kt2 + kNSTA - 1, nk2 - 1));
        if constexpr (kFull && decltype(u)::value == 1) {
          // W is read and written once per step: non-temporal
          unroll<kG>([&](auto v) {
            w[decltype(v)::value] = __builtin_nontemporal_load(w_at(j, decltype(v)::value));
          });
        }
        unroll<kSub>([&](auto h) {
          constexpr int S = 2 * decltype(u)::value + decltype(h)::value;   // stage within the tile
          const int base = kOffRingA + cur * kSlot + decltype(h)::value * kStage;
          unroll<2>([&](auto ii) {
            constexpr int I = 2 * S + decltype(ii)::value;                 // output block
            unroll<4>([&](auto kb) {
              const u32x4 a = frag_tr(base, decltype(kb)::value, decltype(ii)::value);
              D[I] = mma16(a, qh[decltype(kb)::value], D[I]);
              D[I] = mma16(a, ql[decltype(kb)::value], D[I]);
            });
          });
        });
      });

      // x = r D^T: lane (l16, lq) holds x[cs + l16][16 i + 4 lq + e] of the
      // tile, staged in W's orientation; then W <- W - (lr wd W + step x),
      // four consecutive W elements per group
      unroll<8>([&](auto i) {
        constexpr int I = decltype(i)::value;
        const int rr = cs + l16, cc = 16 * I + 4 * lq;
        const float v0 = r0 * D[I][0], v1 = r0 * D[I][1], v2 = r0 * D[I][2], v3 = r0 * D[I][3];
        if (ori) {
          lf[(cc + 0) * kApLd + rr] = v0;
          lf[(cc + 1) * kApLd + rr] = v1;
          lf[(cc + 2) * kApLd + rr] = v2;
          lf[(cc + 3) * kApLd + rr] = v3;
        } else {
          *reinterpret_cast<float4*>(lf + rr * kApLd + cc) = make_float4(v0, v1, v2, v3);
        }
      });
      lds_sync();
      // W rows of this tile: X rows (plain) or X columns (oriented)
      const int wrows = ori ? min(kT, g.n_true - j * kT) : g.m_true;
      const int wcols = ori ? g.m_true : min(kT, g.n_true - j * kT);
      const bool full = kFull || (wrows == kT && wcols == kT && (ldw % 4) == 0);
      if (full) {
        if constexpr (!kFull) {
          // all of this thread's groups are loaded before any is updated
          unroll<kG>([&](auto u) {
            w[decltype(u)::value] = __builtin_nontemporal_load(w_at(j, decltype(u)::value));
          });
        }
        unroll<kG>([&](auto u) {
          constexpr int U = decltype(u)::value;
          const int gidx = tid + U * kNT, rr = gidx >> 5, c4 = (gidx & 31) * 4;
          const float4 x = *reinterpret_cast<const float4*>(lf + rr * kApLd + c4);
          w[U][0] -= p.lrwd * w[U][0] + g.step * x.x;
          w[U][1] -= p.lrwd * w[U][1] + g.step * x.y;
          w[U][2] -= p.lrwd * w[U][2] + g.step * x.z;
          w[U][3] -= p.lrwd * w[U][3] + g.step * x.w;
          __builtin_nontemporal_store(w[U], w_at(j, U));
          sq += (x.x * x.x + x.y * x.y) + (x.z * x.z + x.w * x.w);
        });
      } else {
        const int64_t row0 = ori ? static_cast<int64_t>(j) * kT : 0;
        const int64_t col0 = ori ? 0 : static_cast<int64_t>(j) * kT;
        for (int gidx = tid; gidx < kT * kT / 4; gidx += kNT) {
          const int rr = gidx >> 5, c4 = (gidx & 31) * 4;
          if (rr >= wrows || c4 >= wcols) continue;
          const float* xv = lf + rr * kApLd + c4;
          float* wp = W + (row0 + rr) * ldw + col0 + c4;
          for (int e = 0; e < 4 && c4 + e < wcols; ++e) {
            const float x = xv[e];
            wp[e] -= p.lrwd * wp[e] + g.step * x;
            sq += x * x;
          }
        }
      }
      if (g.rms_part) {
        // per-tile partial (deterministic: fixed lanes and fixed order)
        float t = sq;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o, 64);
        lds_sync();                                   // staging reads done
        float* red = lf;                              // the ring is still in use
        if (lane == 0) red[wave] = t;
        lds_sync();
        if (tid == 0) {
          float tot = 0.0f;
#pragma unroll
          for (int w8 = 0; w8 < 8; ++w8) tot += red[w8];
          g.rms_part[static_cast<int64_t>(b) * ntj + j] = tot;
        }
        sq = 0.0f;
      }
      lds_sync();                                     // staging free for the next tile
    }
  };
  if (g.m_true == kT && g.n_true % kT == 0) {
    tile_loop(std::true_type{});
  } else {
    tile_loop(std::false_type{});
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

hipError_t launch_small(const SmallArgs& a, int total, hipStream_t s) {
  hipLaunchKernelGGL(ns_small_kernel, dim3(total), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace mo
