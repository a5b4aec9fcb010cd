// Internal declarations shared by the library's translation units.
// Device code targets gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mo {

// Element type tags used for template dispatch.
enum Dt : int { F32 = 0, BF16 = 1 };

// One Muon matrix as the kernels see it.  `oriented` = 1 when rows > cols:
// the Newton-Schulz iterate is then the transpose of the parameter.
struct MatDesc {
  float* param;          // fp32 [rows, cols]
  const void* grad;      // [rows, cols]
  void* mom;             // [rows, cols]
  int32_t oriented;
  int32_t out_index;     // position in the caller's list (update RMS slot)
};
static_assert(sizeof(MatDesc) == 32, "descriptor layout");

// Momentum / X_0 preparation over one shape group (a "bin") chunk.
// Tiles of 64x64 cover the padded natural domain [A_pad, B_pad] of every
// matrix; each tile writes its part of the Newton-Schulz input X_0 in the
// oriented, blocked layout (one layout: the update reads X K-major from it).
struct PrepArgs {
  const MatDesc* desc;   // chunk's descriptors (chunk-local index)
  void* x;               // [chunk] blocked [m_pad, n_pad]  (ns dtype), oriented
  int64_t x_stride;      // m_pad * n_pad
  int tile;              // panel height of the blocked layout
  int m, n, m_pad, n_pad;
  int tiles_per_mat;     // (m_pad / 64) * (n_pad / 64)
  float mu;
  int nesterov;
  int has_mom;           // 0: N = grad (Newton-Schulz only)
  int grad_dt, mom_dt, ns_dt;
  float* norm_part;      // [chunk][tiles_per_mat]
};

// Per-matrix finalisation of the squared-norm partials: r = 1/(sqrt(s)+eps).
struct NormArgs {
  const float* part;     // [chunk][tiles]
  int tiles;
  float eps;
  float* rscale;         // [chunk]
};

// Epilogue kinds of the Newton-Schulz GEMM C = A * B^T.
// The linear term a X of Eq. 2 is folded into the polynomial matrix,
// P' = a I + b S + c S S, so the update is the plain product X' = P' X.
enum Epi : int {
  EPI_GRAM = 0,     // C = s^2 acc, lower tiles mirrored
  EPI_POLY = 1,     // C = alpha acc + beta D + gamma I, lower tiles mirrored
  EPI_UPDATE = 2,   // C = s acc (B given K-major)
  EPI_APPLY = 3,    // x = s acc; W -= lrwd W + step x (natural layout; B K-major)
  EPI_STORE = 4     // x = s acc; out = x (natural layout, ns dtype; B K-major)
};

// All matrices are in the blocked layout (mo_layout.h) with panels of
// TILE rows; s* are per-batch-entry strides in elements.
//
// One launch covers up to kMaxGroup shape groups (bins) at once: GemmBin
// holds what differs between them.  Each group's tiles are split evenly
// over the 8 XCDs (a contiguous range per XCD, for L2 reuse), and each XCD
// walks the groups in its own rotated order, so that tiles of different
// lengths -- and their output bursts -- overlap across the chip.
constexpr int kMaxGroup = 8;
struct GemmBin {
  const void* A;  int64_t sA;            // [M, K] per batch entry
  const void* B;  int64_t sB;            // [N, K]; [K, N] for EPI_UPDATE/APPLY/STORE
  const void* D;  int64_t sD;            // [M, N] epilogue operand
  void* C;        int64_t sC;            // [M, N] output
  const float* rscale;                   // per batch entry (applied if use_rscale)
  const MatDesc* desc;                   // EPI_APPLY / EPI_STORE, per batch entry
  void* out;  int64_t s_out;             // EPI_STORE output base, stride
  float* rms_part;                       // [batch][tiles_per_mat] or null
  int M, N, K;                           // padded sizes (tile multiples)
  int k_loop;                            // K stages visited: the padded K / stage depth, or fewer
                                         // when the tail stages multiply zero padding only
  int tiles_m, tiles_n, tiles_per_mat, batch;
  int m_true, n_true;
  float step;                            // EPI_APPLY: W <- W - (lrwd W + step x)
  const float* step_dev;                 // EPI_APPLY: per batch entry step (replaces step) or null
  int super_order;                       // tiles in 16x16-tile super-blocks (see ns_gemm.hip)
};
struct GemmArgs {
  GemmBin bin[kMaxGroup];
  int nbins;
  int rotate;                            // XCDs walk the groups in rotated order
  int per_xcd;                           // grid = 8 * per_xcd
  int use_rscale;                        // first iteration: scale by rscale
  float alpha, beta, gamma;              // EPI_POLY coefficients
  float lrwd;                            // EPI_APPLY
  int rms_only;                          // EPI_APPLY: only write the rms_part partials of x
};

// Fused Newton-Schulz + apply for matrices with m <= 128 (bf16, 128-row
// panels): one workgroup per matrix (ns_small.hip).
struct SmallBin {
  const MatDesc* desc;                   // per matrix
  const void* x0;                        // X_0 (unscaled N), blocked [128, n_pad]
  int64_t x_stride;                      // elements per matrix: 128 * n_pad
  const float* rscale;                   // 1 / (||N||_F + eps) per matrix
  float* rms_part;                       // [count][n_pad / 128] or null
  int n_pad, m_true, n_true, count;
  float step;                            // W <- W - (lrwd W + step X_N)
};
struct SmallArgs {
  SmallBin bin[kMaxGroup];
  int nbins;
  int ns_steps;                          // >= 1
  float a, b, c;                         // Eq. 2 coefficients
  float lrwd;
};

// Elementwise apply for ns_steps = 0 (X_N = X_0), and for EPI_STORE with 0
// steps in the Newton-Schulz-only entry point.
struct ApplyX0Args {
  const MatDesc* desc;
  const void* x;                         // [chunk] blocked [m_pad, n_pad], oriented
  int64_t x_stride;                      // m_pad * n_pad
  int tile;                              // panel height of the blocked layout
  int m, n, m_pad, n_pad;
  int tiles_per_mat;                     // 64x64 tiles of the true domain
  const float* rscale;
  float lrwd, step;
  const float* step_dev;                 // per matrix step (replaces step) or null
  int ns_dt;
  void* out; int64_t s_out;              // store mode when non-null
  float* rms_part;                       // [chunk][tiles_per_mat] or null
};

// Per matrix: rms = sqrt(sum(part) * mult * inv_count) with mult = rscale^2
// (partials of N, ns_steps = 0) or 1 (partials of X_N); writes rms to
// update_rms[out_index] and/or step = lr_scale / rms (0 when rms = 0).
struct RmsArgs {
  const MatDesc* desc;
  const float* part;
  int tiles;
  double inv_count;      // 1 / (rows * cols)
  float* update_rms;     // indexed by desc[i].out_index, or null
  const float* rscale;   // mult = rscale[i]^2 when non-null
  float* step;           // [chunk] or null
  float lr_scale;        // lr * rms_scale
};

constexpr int kAdamMaxTensors = 32;
struct AdamTensor {
  float* p; const void* g; float* m; float* v;
  int64_t n; int64_t block0;
};
struct AdamArgs {
  AdamTensor t[kAdamMaxTensors];
  int count;
  int grad_dt;
  float lr, wd, beta1, beta2, eps;
  float one_m_beta1;     // 1 - beta1 and 1 - beta2, formed on the host in
  float one_m_beta2;     // double (1 - 0.999f in fp32 loses 1e-5 relative)
  float bc1;             // 1 / (1 - beta1^t)
  float bc2_rsqrt;       // 1 / sqrt(1 - beta2^t)
};
constexpr int kAdamElemsPerBlock = 2048;   // 256 threads x 8

// Descriptor upload by kernel arguments: up to kDescPerCopy descriptors
// (3 KiB) per launch of a one-workgroup copy kernel.
constexpr int kDescPerCopy = 96;
struct DescCopyArgs {
  MatDesc d[kDescPerCopy];
  MatDesc* dst;
  int count;
};

// Tile configurations of the GEMM (square tiles).
enum TileCfg : int { TILE_256 = 0, TILE_128 = 1, TILE_64 = 2 };
int tile_size(TileCfg t);

// Launchers (return hipError_t of the launch).
hipError_t launch_prep(const PrepArgs& a, int chunk, hipStream_t s);
hipError_t launch_norm(const NormArgs& a, int chunk, hipStream_t s);
// waves: 4 (2 x 2 wave grid) or 8 (2 x 4; bf16 256-wide tiles only)
hipError_t launch_gemm(int ns_dt, TileCfg cfg, Epi epi, int waves, const GemmArgs& a,
                       hipStream_t s);
hipError_t launch_apply_x0(const ApplyX0Args& a, int chunk, hipStream_t s);
hipError_t launch_small(const SmallArgs& a, int total, hipStream_t s);
hipError_t launch_rms(const RmsArgs& a, int chunk, hipStream_t s);
hipError_t launch_adamw(const AdamArgs& a, int64_t blocks, hipStream_t s);
// copies count host descriptors to dst (device) on s, 96 per launch
hipError_t launch_desc_copy(const MatDesc* src, int64_t count, MatDesc* dst, hipStream_t s);

}  // namespace mo
