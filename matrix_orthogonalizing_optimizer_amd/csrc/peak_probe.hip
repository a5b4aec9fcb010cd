// Roofline probes (declared in include/mo_probe.h): the bf16 matrix-core
// rate and the HBM streaming rates the chip sustains on their own.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <string>

#include "mo_probe.h"

namespace {

thread_local std::string g_probe_err;

int probe_fail(hipError_t e, const char* what) {
  g_probe_err = std::string(what) + ": " + hipGetErrorString(e);
  return -1;
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 4;    // independent accumulators per wave
constexpr int kPerIter = 8;   // MFMAs per loop iteration

// Register-only MFMA issue: the operands depend on the lane (so nothing is
// folded), and one sum per thread is stored so the loop is kept.
__global__ __launch_bounds__(256) void mfma_probe_kernel(float* out, int iters) {
  const unsigned t = threadIdx.x + 1u;
  u32x4 ua, ub;
  for (int k = 0; k < 4; ++k) {
    ua[k] = 0x3f803f80u ^ ((t * 2654435761u + k) & 0x00070007u);
    ub[k] = 0x3f803f80u ^ ((t * 40503u + 7 * k) & 0x00070007u);
  }
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ua), b = __builtin_bit_cast(bf16x8_t, ub);
  f32x16_t acc[kChains];
  for (int c = 0; c < kChains; ++c)
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kPerIter; ++k)
      acc[k % kChains] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k % kChains], 0, 0, 0);
  }
  float s = 0.0f;
  for (int c = 0; c < kChains; ++c)
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The same issue pattern on data that switches like a GEMM's: eight A and
// eight B operands per lane, each a random bf16 vector (random sign,
// exponents 2^-8 .. 2^-1, random mantissa), cycled so that consecutive MFMAs
// never see the same inputs.  The matrix cores' power then depends on real
// bit toggling, as in a product of random matrices, while nothing moves
// through memory.
__device__ inline unsigned probe_hash(unsigned x) {       // a 32-bit integer mix (xorshift-multiply)
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__device__ inline unsigned probe_bf16_pair(unsigned h) {  // two random bf16 of magnitude < 1
  const unsigned lo = (h & 0x807fu) | ((0x77u + ((h >> 7) & 7u)) << 7);
  const unsigned hi = ((h >> 16) & 0x807fu) | ((0x77u + ((h >> 23) & 7u)) << 7);
  return lo | (hi << 16);
}

constexpr int kOps = 8;       // distinct operand vectors per side

__global__ __launch_bounds__(256) void mfma_random_probe_kernel(float* out, int iters) {
  const unsigned t = blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8_t a[kOps], b[kOps];
#pragma unroll
  for (int o = 0; o < kOps; ++o) {
    u32x4 ua, ub;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      ua[k] = probe_bf16_pair(probe_hash(t * 64u + o * 8u + k));
      ub[k] = probe_bf16_pair(probe_hash(t * 64u + o * 8u + 4u + k) ^ 0x9e3779b9u);
    }
    a[o] = __builtin_bit_cast(bf16x8_t, ua);
    b[o] = __builtin_bit_cast(bf16x8_t, ub);
  }
  f32x16_t acc[kChains];
  for (int c = 0; c < kChains; ++c)
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kPerIter; ++k)
      acc[k % kChains] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k % kOps], b[(3 * k + 1) % kOps],
                                                                 acc[k % kChains], 0, 0, 0);
  }
  float s = 0.0f;
  for (int c = 0; c < kChains; ++c)
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Streaming kernels: each pass of the grid covers gridDim.x * 256 * U
// consecutive 16-byte words, thread t of a block taking words t, t + 256,
// .. t + 256 (U - 1) of its block's span (coalesced), U loads in flight
// before any use.
// Read-only stream: one partial per thread.
template <int U>
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ in, int64_t n,
                                                         unsigned* __restrict__ out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x * U;
  unsigned x = 0;
  for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * blockDim.x * U + threadIdx.x; i0 < n; i0 += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + static_cast<int64_t>(u) * blockDim.x;
      v[u] = i < n ? __builtin_nontemporal_load(in + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = x;
}

// Copy stream.
template <int U>
__global__ __launch_bounds__(256) void copy_probe_kernel(const u32x4* __restrict__ in, u32x4* __restrict__ out,
                                                         int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x * U;
  for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * blockDim.x * U + threadIdx.x; i0 < n; i0 += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + static_cast<int64_t>(u) * blockDim.x;
      if (i < n) v[u] = __builtin_nontemporal_load(in + i);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + static_cast<int64_t>(u) * blockDim.x;
      if (i < n) __builtin_nontemporal_store(v[u], out + i);
    }
  }
}

// Launch shapes tried by the HBM probe (the best rate of each stream is
// reported): which one a given box streams fastest with varies by 10-20%.
struct StreamShape {
  int unroll, blocks_per_cu;
};
constexpr StreamShape kShapes[] = {{1, 4}, {1, 16}, {2, 64}, {4, 64}};

void launch_stream(int kind, const StreamShape& sh, int blocks, const u32x4* a, u32x4* b, int64_t n,
                   unsigned* part) {
  if (kind == 0) {
    if (sh.unroll == 1) hipLaunchKernelGGL(read_probe_kernel<1>, dim3(blocks), dim3(256), 0, nullptr, a, n, part);
    else if (sh.unroll == 2) hipLaunchKernelGGL(read_probe_kernel<2>, dim3(blocks), dim3(256), 0, nullptr, a, n, part);
    else hipLaunchKernelGGL(read_probe_kernel<4>, dim3(blocks), dim3(256), 0, nullptr, a, n, part);
  } else {
    if (sh.unroll == 1) hipLaunchKernelGGL(copy_probe_kernel<1>, dim3(blocks), dim3(256), 0, nullptr, a, b, n);
    else if (sh.unroll == 2) hipLaunchKernelGGL(copy_probe_kernel<2>, dim3(blocks), dim3(256), 0, nullptr, a, b, n);
    else hipLaunchKernelGGL(copy_probe_kernel<4>, dim3(blocks), dim3(256), 0, nullptr, a, b, n);
  }
}

int cu_count(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  return e == hipSuccess ? 0 : probe_fail(e, "device query");
}

int mfma_probe(bool random_operands, int iters, int reps, double* tflops) {
  if (iters < 1 || reps < 1 || !tflops) {
    g_probe_err = "iters and reps must be >= 1, tflops non-NULL";
    return -2;
  }
  int cus = 0;
  if (cu_count(&cus)) return -1;
  const int blocks = cus * 8;                 // 8 x 4 waves per CU: two per SIMD
  float* out = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipMalloc(&out, static_cast<size_t>(blocks) * 256 * sizeof(float));
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  double best = 0.0;
  for (int r = 0; r <= reps && e == hipSuccess; ++r) {   // the first launch warms up
    e = hipEventRecord(e0, nullptr);
    if (e == hipSuccess) {
      if (random_operands)
        hipLaunchKernelGGL(mfma_random_probe_kernel, dim3(blocks), dim3(256), 0, nullptr, out, iters);
      else
        hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, nullptr, out, iters);
      e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(e1, nullptr);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e == hipSuccess && r > 0 && ms > 0.0f) {
      const double flops = 32768.0 * kPerIter * static_cast<double>(iters) * blocks * 4.0;
      best = std::max(best, flops / (ms * 1e-3) / 1e12);
    }
  }
  const hipError_t run = e;
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (out) (void)hipFree(out);
  if (run != hipSuccess) return probe_fail(run, "mfma probe");
  *tflops = best;
  return 0;
}

}  // namespace

extern "C" {

const char* mo_probe_last_error(void) { return g_probe_err.c_str(); }

int mo_probe_mfma_bf16(int iters, int reps, double* tflops) { return mfma_probe(false, iters, reps, tflops); }

int mo_probe_mfma_bf16_random(int iters, int reps, double* tflops) {
  return mfma_probe(true, iters, reps, tflops);
}

int mo_probe_hbm(size_t bytes, int reps, double* read_gbs, double* copy_gbs) {
  if (reps < 1 || !read_gbs || !copy_gbs || bytes < (size_t{1} << 16)) {
    g_probe_err = "bytes >= 64 KiB, reps >= 1 and non-NULL outputs required";
    return -2;
  }
  const int64_t n = static_cast<int64_t>(bytes >> 16) << 12;     // 16-byte words
  int cus = 0;
  if (cu_count(&cus)) return -1;
  int max_bpc = 0;
  for (const StreamShape& sh : kShapes) max_bpc = std::max(max_bpc, sh.blocks_per_cu);
  u32x4 *a = nullptr, *b = nullptr;
  unsigned* part = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipMalloc(&a, n * 16);
  if (e == hipSuccess) e = hipMalloc(&b, n * 16);
  if (e == hipSuccess) e = hipMalloc(&part, static_cast<size_t>(cus) * max_bpc * 256 * sizeof(unsigned));
  if (e == hipSuccess) e = hipMemset(a, 0x5a, n * 16);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  double best_r = 0.0, best_c = 0.0;
  for (int kind = 0; kind < 2 && e == hipSuccess; ++kind) {
    for (const StreamShape& sh : kShapes) {
      for (int r = 0; r <= reps && e == hipSuccess; ++r) {   // the first launch of a shape warms up
        e = hipEventRecord(e0, nullptr);
        if (e == hipSuccess) {
          launch_stream(kind, sh, cus * sh.blocks_per_cu, a, b, n, part);
          e = hipGetLastError();
        }
        if (e == hipSuccess) e = hipEventRecord(e1, nullptr);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
        float ms = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
        if (e == hipSuccess && r > 0 && ms > 0.0f) {
          const double gbs = (kind == 0 ? 1.0 : 2.0) * n * 16.0 / (ms * 1e-3) / 1e9;
          if (kind == 0) best_r = std::max(best_r, gbs);
          else best_c = std::max(best_c, gbs);
        }
      }
    }
  }
  const hipError_t run = e;
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (a) (void)hipFree(a);
  if (b) (void)hipFree(b);
  if (part) (void)hipFree(part);
  if (run != hipSuccess) return probe_fail(run, "hbm probe");
  *read_gbs = best_r;
  *copy_gbs = best_c;
  return 0;
}

}  // extern "C"
