// Blocked layout of the Newton-Schulz operands in the workspace.
//
// Every operand of the Newton-Schulz GEMMs (X, X^T, S, P) is a matrix
// [R, C] that a GEMM reads as row panels of T rows (T = the shape group's
// tile edge) while stepping along C in stages of 64 bytes (32 bf16 or 16
// fp32 elements).  The workspace stores such a matrix as
//     [R / T panels][C / bk stages][T rows][bk elements]
// so that the part one K-stage of one panel needs is a single contiguous
// T x 64-byte block, and a T x T output tile is a single contiguous range.
// Inside a 64-byte row the four 16-byte chunks are permuted: chunk c of row
// r is stored at position c ^ ((r >> 2) & 3).  A block is copied to LDS
// unchanged, and this permutation makes the 16 rows one quarter-wave of
// ds_read_b128 touches fall into distinct LDS bank groups.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mo {

struct Blocked {
  int T;      // panel height (tile edge)
  int nkb;    // stages per panel = C / bk
  int bk;     // elements per 64-byte row piece
  int vec;    // elements per 16-byte chunk (bk / 4)
};

__host__ __device__ inline Blocked blocked(int T, int cols, int esz) {
  Blocked L;
  L.T = T;
  L.bk = 64 / esz;
  L.vec = 16 / esz;
  L.nkb = cols / L.bk;
  return L;
}

// Element offset of (r, c) in a blocked matrix.
__host__ __device__ inline int64_t blk_off(const Blocked& L, int r, int c) {
  const int panel = r / L.T, rr = r - panel * L.T;
  const int stage = c / L.bk, cc = c - stage * L.bk;
  const int chunk = cc / L.vec, w = cc - chunk * L.vec;
  return (static_cast<int64_t>(panel) * L.nkb + stage) * L.T * L.bk +
         static_cast<int64_t>(rr) * L.bk + (chunk ^ ((rr >> 2) & 3)) * L.vec + w;
}

// First element of the T x T tile whose rows are panel `pi` and whose
// columns start at column cj * T (a contiguous range of T * T elements).
__host__ __device__ inline int64_t blk_tile(const Blocked& L, int pi, int cj) {
  return (static_cast<int64_t>(pi) * L.nkb + static_cast<int64_t>(cj) * (L.T / L.bk)) * L.T * L.bk;
}

}  // namespace mo
