// Internal declarations of the SVD-entropy diagnostic (svd_entropy.hip and
// its host side).  Device code targets gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muon.h"

namespace mo {

// SVD-entropy diagnostic.  A chunk holds `batch` matrices that share
// m = min(rows, cols); their m x m fp64 Gram matrices sit back to back in
// the workspace, row-major, of which the block-lower 64 x 64 tiles (the
// diagonal tiles in full) are kept.
constexpr int kSvdTile = 64;                 // tile edge of the reduction passes (partial-product slots)
constexpr int kSvdMaxM = 8192;               // largest min(rows, cols)
constexpr int kSvdGramBatch = 192;           // matrices per Gram launch (kernel arguments < 4 KiB)
constexpr int kSvdOutBatch = 64;             // matrices per entropy launch
constexpr int kSvdPanel = 16;                // Householder steps per deferred update
struct SvdGramArgs {
  const void* src[kSvdGramBatch];            // [rows, cols] row-major inputs (one shape per launch)
  double* dst[kSvdGramBatch];                // their m x m Gram matrices
  int64_t ld;                                // cols (row length of the input)
  int m, n, trans;                           // trans: X = W^T (rows > cols); X is [m, n]
};
struct SvdTrdArgs {
  double* a;                                 // [batch][m][m] working matrices
  double* v;                                 // [2][batch][m] Householder vectors (by step parity)
  double* part;                              // [batch][nb][m] partial products, one slot per tile column
  double* d;                                 // [batch][m] tridiagonal: diagonal
  double* e;                                 // [batch][m] tridiagonal: subdiagonal (m - 1 used)
  double* pv;                                // [batch][kSvdPanel][m] the panel's v of each step
  double* pw;                                // [batch][kSvdPanel][m] and its w
  double* pdot;                              // [batch][nb][2 kSvdPanel] w_t . v, v_t . v per row block
  int m, nb, batch;
};
struct SvdEigArgs {
  const double* d;                           // [batch][m]
  const double* e;                           // [batch][m]
  double* lam;                               // [batch][m] eigenvalues, ascending
  int m;
};
struct SvdOutArgs {
  const double* lam;                         // chunk's eigenvalues [batch][m], ascending
  double* entropy;                           // caller's [count]
  double* sigma;                             // caller's packed singular values, or NULL
  int64_t out_index[kSvdOutBatch];           // entropy slot of each matrix
  int64_t sigma_off[kSvdOutBatch];           // offset of its singular values in sigma
  int first;                                 // chunk-local index of the launch's first matrix
  int m;
};

hipError_t launch_svd_gram(int dt, const SvdGramArgs& a, int count, hipStream_t s);
// one step of the Householder reduction: k = -1 .. m - 3, panel started at
// step k0 (see the kernels)
hipError_t launch_svd_trd_col(const SvdTrdArgs& a, int k, int k0, hipStream_t s);
hipError_t launch_svd_trd_pass(const SvdTrdArgs& a, int j, int np, hipStream_t s);
hipError_t launch_svd_trd_panel(const SvdTrdArgs& a, int r0, hipStream_t s);
hipError_t launch_svd_eig(const SvdEigArgs& a, int batch, hipStream_t s);
hipError_t launch_svd_out(const SvdOutArgs& a, int count, hipStream_t s);

}  // namespace mo
