// Fused Newton-Schulz for small matrices (m <= 128, bf16), gfx950.
//
// Eq. 2 of "Muon is Scalable for LLM Training" (section 2.1) on an oriented
// [m, n] matrix with m <= 128: one 512-thread workgroup per matrix runs all
// N iterations and the apply of section 2.2, Eq. 4, with S and P' resident
// in LDS:
//   S_0 = r^2 X_0 X_0^T                 (X_0 streamed once, r = 1/(|N|+eps))
//   for k < N:  P'_k = a I + b S_k + c S_k S_k
//               X_{k+1} = P'_k X_k       (r folded in at k = 0)
//               S_{k+1} = X_{k+1} X_{k+1}^T, accumulated from each bf16
//               128-column tile of X_{k+1} as it is written
//   W <- W - (lr wd W + step X_N)       (last iteration, fp32 X_N)
// so every iteration reads X_k once and writes X_{k+1} once, instead of 15
// launches that each stream the whole matrix.  The operands, roundings and
// tile layout are those of the general kernels: X in the blocked layout of
// mo_layout.h with 128-row panels (one panel), S, P' and X_k stored as bf16
// with round-to-nearest-even, products accumulated in fp32.
//
// Waves: 8 in a 2 x 4 grid; every 128 x 128 product gives a wave a 64 x 32
// part (two 32x32 MFMA blocks).
#include "mo_internal.h"
#include "mo_layout.h"
#include "ns_common.h"

namespace mo {

namespace {

constexpr int kT = 128;                 // panel height / output tile edge
constexpr int kBK = 32;                 // bf16 elements per 64-byte row piece
constexpr int kCPR = 4;                 // 16-byte chunks per row piece
constexpr int kNT = 512;                // threads
constexpr int kStage = kT * kCPR;       // chunks of one [128 rows][64 B] stage (8 KiB)
constexpr int kSub = 2;                 // K-stages per ring slot (one barrier pair per slot)
constexpr int kSlot = kSub * kStage;
static_assert(4 % kSub == 0, "a 128-column tile's 4 K-stages fill whole slots");
constexpr int kNST = 3;                 // ring slots (two in flight)
// LDS map in 16-byte chunks.  P', S and the X' tile are [4 K-stages][128
// rows][64 B] (chunks permuted per row as in global memory); a ring slot
// holds kSub Gram stages [128 rows][64 B] or kSub update blocks [4 column
// blocks][32 rows][64 B].  The apply stages fp32 x over the S and X'
// regions and the tail.  S and X' come first: the LDS instructions' 16-bit
// immediate offsets then reach every access to them from one lane base,
// which keeps the kernel within its registers.
constexpr int kOffS = 0;
constexpr int kOffX = kOffS + 4 * kStage;
constexpr int kOffRing = kOffX + 4 * kStage + 256;
constexpr int kOffP = kOffRing + kNST * kSlot;
constexpr int kOffEnd = kOffP + 4 * kStage;
constexpr int kApLd = kT + 4;           // padded fp32 row of the apply staging
static_assert((kOffRing - kOffS) * 4 >= kT * kApLd, "apply staging fits");
static_assert(kOffEnd * 16 <= 160 * 1024, "LDS");

}  // namespace

__global__ __launch_bounds__(512) void ns_small_kernel(SmallArgs p) {
  using T = uint16_t;
  using E = Elem<T>;
  __shared__ u32x4 smem[kOffEnd];

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
  const int nkx = g.n_pad / kBK;         // K-stages of the Gram
  const int ntj = g.n_pad / kT;          // 128-column tiles
  const float r0 = g.rscale[b];
  const T* const x0 = static_cast<const T*>(g.x0) + b * g.x_stride;
  T* const x1 = static_cast<T*>(g.x1) + b * g.x_stride;
  const uint32_t lane16 = static_cast<uint32_t>(lane * 16);
  T* const lp = reinterpret_cast<T*>(smem + kOffP);
  T* const ls = reinterpret_cast<T*>(smem + kOffS);
  T* const lx = reinterpret_cast<T*>(smem + kOffX);

  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto lds_sync = [&]() {                 // own LDS accesses done, then barrier
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    barrier();
  };
  // element (row, k) of a [4 K-stages][128 rows][32] region
  auto koff = [](int row, int k) {
    const int st = k >> 5, w = k & 31, ch = w >> 3;
    return (st * kT + row) * kBK + ((ch ^ ((row >> 2) & 3)) << 3) + (w & 7);
  };

  // -------- fragments
  // NT operand rows of a [128 rows][64 B] stage at chunk `base`: this
  // lane's row `row`, K offsets 16 ks + 8 lh .. + 7
  auto frag_nt = [&](int base, int row, int ks) -> u32x4 {
    return smem[base + row * kCPR + ((ks * 2 + lh) ^ rsw)];
  };
  // K-major B fragment (update): stage [4 column blocks][32 rows][32] at
  // chunk `base`; this lane's column wc + l32, K values of substep ks
  // (two transposing reads, four K each)
  auto frag_km = [&](int base, int ks) -> u32x4 {
    const T* sB = reinterpret_cast<const T*>(smem + base);
    const int gi = lane & 15;
    const int n = wc + (l32 & 16) + 4 * (gi & 3);
    u32x4 r;
    unroll<2>([&](auto h) {
      const int k = ks * 16 + 8 * lh + 4 * decltype(h)::value + (gi >> 2);
      const int c = n >> 5, c2 = n & 31, ch = c2 >> 3;
      const int off = c * kBK * kBK + k * kBK + ((ch ^ ((k >> 2) & 3)) << 3) + (c2 & 7);
      const v4s16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s16_t*)(sB + off));
      const uint2 u = __builtin_bit_cast(uint2, v);
      r[2 * decltype(h)::value] = u.x;
      r[2 * decltype(h)::value + 1] = u.y;
    });
    return r;
  };

  f32x16_t acc[2], accs[2];
  auto zero = [&](f32x16_t (&a)[2]) {
    unroll<2>([&](auto i) { unroll<16>([&](auto r) { a[decltype(i)::value][decltype(r)::value] = 0.0f; }); });
  };
  // a += A B^T over the 4 K-stages of LDS regions ra (rows wr..) and rb
  // (rows wc..), both [4][128][64 B]
  auto nt_lds = [&](f32x16_t (&a)[2], int ra, int rb) {
    for (int kt = 0; kt < 4; ++kt) {
      unroll<2>([&](auto ks) {
        const u32x4 fb = frag_nt(rb + kt * kStage, wc + l32, decltype(ks)::value);
        unroll<2>([&](auto i) {
          const u32x4 fa = frag_nt(ra + kt * kStage, wr + 32 * decltype(i)::value + l32, decltype(ks)::value);
          a[decltype(i)::value] = E::mma(fa, fb, a[decltype(i)::value]);
        });
      });
    }
  };
  // accumulator (i, r) of an NT product: row wr + 32 i + 8 (r/4) + 4 lh + r%4,
  // column wc + l32.  Stores s * a as bf16 into a [4][128][64 B] region.
  auto store_nt = [&](T* dst, const f32x16_t (&a)[2], float s) {
    unroll<2>([&](auto i) {
      unroll<16>([&](auto r) {
        constexpr int I = decltype(i)::value, R = decltype(r)::value;
        const int row = wr + 32 * I + 8 * (R / 4) + 4 * lh + (R % 4);
        E::store1(dst + koff(row, wc + l32), s * a[I][R]);
      });
    });
  };

  // -------- the streamed loads: one 1 KiB piece per wave per K-stage,
  // kSub K-stages per ring slot
  auto dma_gram = [&](int buf, int kt2) {
    unroll<kSub>([&](auto h) {
      constexpr int H = decltype(h)::value;
      const char* src = reinterpret_cast<const char*>(x0 + (kSub * kt2 + H) * (kT * kBK)) + wave * 1024;
      lds_dma16(src, lane16,
                __builtin_amdgcn_readfirstlane(lds_addr(smem + kOffRing + buf * kSlot + H * kStage + wave * 64)));
    });
  };
  // update stream position q = 4 j + kt: rows 32 kt .. of column tile j of X
  auto dma_upd = [&](const T* xs, int buf, int q2) {
    unroll<kSub>([&](auto h) {
      constexpr int H = decltype(h)::value;
      const int q = kSub * q2 + H;
      const int j = q >> 2, kt = q & 3;
      const int cb = wave >> 1, within = (wave & 1) * 1024;
      const char* src = reinterpret_cast<const char*>(xs + ((4 * j + cb) * kT + 32 * kt) * kBK) + within;
      lds_dma16(src, lane16,
                __builtin_amdgcn_readfirstlane(lds_addr(smem + kOffRing + buf * kSlot + H * kStage + wave * 64)));
    });
  };

  // -------- S_0 = r^2 X_0 X_0^T
  zero(accs);
  const int nk2 = nkx / kSub;             // n_pad is a multiple of 128
  // One barrier per slot: before it a wave waits until its own pieces of
  // slot kt2 have landed (the next kNST - 2 slots may still be in flight)
  // and its LDS reads are done; after it every wave's part of slot kt2 is
  // visible and slot kt2 - 1 has been fully read, so its buffer takes slot
  // kt2 + kNST - 1.  Past the end the last slot is loaded again, so the
  // number of loads in flight is the same at every wait.
  auto prev = [](int cur) { return cur == 0 ? kNST - 1 : cur - 1; };
  for (int s = 0; s < kNST - 1; ++s) dma_gram(s, min(s, nk2 - 1));
  for (int kt2 = 0; kt2 < nk2; ++kt2) {
    const int cur = kt2 % kNST;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((kNST - 2) * kSub));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    barrier();
    dma_gram(prev(cur), min(kt2 + kNST - 1, nk2 - 1));
    unroll<kSub>([&](auto h) {
      const int base = kOffRing + cur * kSlot + decltype(h)::value * kStage;
      unroll<2>([&](auto ks) {
        const u32x4 fb = frag_nt(base, wc + l32, decltype(ks)::value);
        unroll<2>([&](auto i) {
          const u32x4 fa = frag_nt(base, wr + 32 * decltype(i)::value + l32, decltype(ks)::value);
          accs[decltype(i)::value] = E::mma(fa, fb, accs[decltype(i)::value]);
        });
      });
    });
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  store_nt(ls, accs, r0 * r0);
  lds_sync();

  float sq = 0.0f;
  for (int k = 0; k < p.ns_steps; ++k) {
    const bool last = k + 1 == p.ns_steps;
    const T* xs = (k & 1) ? x1 : x0;
    T* xd = (k & 1) ? const_cast<T*>(x0) : x1;
    const float s = k == 0 ? r0 : 1.0f;

    // -------- P' = a I + b S + c S S (S symmetric: S S = S S^T)
    zero(acc);
    nt_lds(acc, kOffS, kOffS);
    unroll<2>([&](auto i) {
      unroll<16>([&](auto r) {
        constexpr int I = decltype(i)::value, R = decltype(r)::value;
        const int row = wr + 32 * I + 8 * (R / 4) + 4 * lh + (R % 4), col = wc + l32;
        float v = p.c * acc[I][R] + p.b * bf2f(ls[koff(row, col)]);
        if (row == col) v += p.a;
        E::store1(lp + koff(row, col), v);
      });
    });
    lds_sync();

    // -------- X_{k+1} = s P' X_k, column tile by column tile
    if (!last) zero(accs);
    const int nq2 = 4 * ntj / kSub;
    for (int q2 = 0; q2 < kNST - 1; ++q2) dma_upd(xs, q2, min(q2, nq2 - 1));
    zero(acc);
    for (int q2 = 0; q2 < nq2; ++q2) {
      const int kt0 = (kSub * q2) & 3, j = (kSub * q2) >> 2, cur = q2 % kNST;
      __builtin_amdgcn_s_waitcnt(waitcnt_vm((kNST - 2) * kSub));   // as in the Gram loop
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      barrier();
      dma_upd(xs, prev(cur), min(q2 + kNST - 1, nq2 - 1));
      unroll<kSub>([&](auto h) {
        const int base = kOffRing + cur * kSlot + decltype(h)::value * kStage;
        const int kt = kt0 + decltype(h)::value;
        unroll<2>([&](auto ks) {
          const u32x4 fb = frag_km(base, decltype(ks)::value);
          unroll<2>([&](auto i) {
            const u32x4 fa = frag_nt(kOffP + kt * kStage, wr + 32 * decltype(i)::value + l32, decltype(ks)::value);
            acc[decltype(i)::value] = E::mma(fb, fa, acc[decltype(i)::value]);   // swapped: (row, 4 columns)
          });
        });
      });
      if (kt0 + kSub != 4) continue;

      // tile j complete.  Swapped operands: register r of block i holds row
      // wr + 32 i + l32, column wc + 8 (r/4) + 4 lh + r%4 of the tile.
      if (!last) {
        unroll<2>([&](auto i) {
          unroll<4>([&](auto qq) {
            constexpr int I = decltype(i)::value, Q = decltype(qq)::value;
            const int row = wr + 32 * I + l32;
            E::store4(lx + koff(row, wc + 8 * Q + 4 * lh), s * acc[I][4 * Q], s * acc[I][4 * Q + 1],
                      s * acc[I][4 * Q + 2], s * acc[I][4 * Q + 3]);
          });
        });
        lds_sync();
        // the tile is one contiguous 32 KiB range of X_{k+1}
        u32x4* dst = reinterpret_cast<u32x4*>(xd + 4 * j * kT * kBK);
        unroll<4>([&](auto u) { dst[tid + decltype(u)::value * kNT] = smem[kOffX + tid + decltype(u)::value * kNT]; });
        nt_lds(accs, kOffX, kOffX);                       // S_{k+1} += X' X'^T
        lds_sync();
      } else {
        // apply: x = s acc (fp32) staged in W's orientation, then
        // W <- W - (lr wd W + step x), four consecutive W elements per group
        const MatDesc md = g.desc[b];
        const bool ori = md.oriented != 0;
        float* const lf = reinterpret_cast<float*>(smem + kOffS);
        unroll<2>([&](auto i) {
          unroll<4>([&](auto qq) {
            constexpr int I = decltype(i)::value, Q = decltype(qq)::value;
            const int rr = wr + 32 * I + l32, cc = wc + 8 * Q + 4 * lh;
            const float v0 = s * acc[I][4 * Q], v1 = s * acc[I][4 * Q + 1];
            const float v2 = s * acc[I][4 * Q + 2], v3 = s * acc[I][4 * Q + 3];
            if (ori) {
              lf[(cc + 0) * kApLd + rr] = v0;
              lf[(cc + 1) * kApLd + rr] = v1;
              lf[(cc + 2) * kApLd + rr] = v2;
              lf[(cc + 3) * kApLd + rr] = v3;
            } else {
              *reinterpret_cast<float4*>(lf + rr * kApLd + cc) = make_float4(v0, v1, v2, v3);
            }
          });
        });
        lds_sync();
        // W rows of this tile: X rows (plain) or X columns (oriented)
        const int64_t ldw = ori ? g.m_true : g.n_true;
        const int wrows = ori ? min(kT, g.n_true - j * kT) : g.m_true;
        const int wcols = ori ? g.m_true : min(kT, g.n_true - j * kT);
        const int64_t row0 = ori ? static_cast<int64_t>(j) * kT : 0;
        const int64_t col0 = ori ? 0 : static_cast<int64_t>(j) * kT;
        float* const W = md.param;
        const bool full = wrows == kT && wcols == kT && (ldw % 4) == 0;
        for (int gidx = tid; gidx < kT * kT / 4; gidx += kNT) {
          const int rr = gidx >> 5, c4 = (gidx & 31) * 4;
          if (rr >= wrows || c4 >= wcols) continue;
          const float* xv = lf + rr * kApLd + c4;
          float* wp = W + (row0 + rr) * ldw + col0 + c4;
          if (full) {
            // W is read and written once per step: non-temporal (unlike X,
            // which this workgroup reads back in the next iteration)
            typedef float f4v __attribute__((ext_vector_type(4)));
            f4v w = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(wp));
            const float4 x = *reinterpret_cast<const float4*>(xv);
            w[0] -= p.lrwd * w[0] + g.step * x.x;
            w[1] -= p.lrwd * w[1] + g.step * x.y;
            w[2] -= p.lrwd * w[2] + g.step * x.z;
            w[3] -= p.lrwd * w[3] + g.step * x.w;
            __builtin_nontemporal_store(w, reinterpret_cast<f4v*>(wp));
            sq += (x.x * x.x + x.y * x.y) + (x.z * x.z + x.w * x.w);
          } else {
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
          lds_sync();                                     // staging reads done
          float* red = reinterpret_cast<float*>(smem + kOffS);
          if (lane == 0) red[wave] = t;
          lds_sync();
          if (tid == 0) {
            float tot = 0.0f;
#pragma unroll
            for (int w = 0; w < 8; ++w) tot += red[w];
            g.rms_part[static_cast<int64_t>(b) * ntj + j] = tot;
          }
          sq = 0.0f;
        }
        lds_sync();
      }
      zero(acc);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    if (!last) {
      store_nt(ls, accs, 1.0f);                            // S_{k+1}
      lds_sync();
    }
  }
}

hipError_t launch_small(const SmallArgs& a, int total, hipStream_t s) {
  hipLaunchKernelGGL(ns_small_kernel, dim3(total), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace mo
