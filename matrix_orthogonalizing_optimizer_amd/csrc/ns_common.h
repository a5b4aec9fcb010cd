// Device helpers shared by the Newton-Schulz kernels (gfx950): element
// types and MFMA wrappers, compile-time unrolling, wait-count encodings,
// direct-to-LDS loads and cross-lane moves.
#pragma once

#include <utility>

#include "mo_internal.h"

namespace mo {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // one 16-byte chunk
typedef short v4s16_t __attribute__((ext_vector_type(4)));

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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32,
// packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {          // bf16 storage
  static constexpr int kVec = 8;             // elements per 16-byte chunk
  __device__ static float ld(const uint16_t* p) { return bf2f(*p); }
  __device__ static void st(uint16_t* p, float v) { *p = f2bf(v); }
  // four consecutive elements (8-byte aligned) in one store / one load
  __device__ static void store4(uint16_t* p, float a, float b, float c, float d) {
    uint2 q;
    q.x = pack_bf16x2(a, b);
    q.y = pack_bf16x2(c, d);
    *reinterpret_cast<uint2*>(p) = q;
  }
  __device__ static void load4(const uint16_t* p, float (&v)[4]) {
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(q.x << 16);
    v[1] = __uint_as_float(q.x & 0xffff0000u);
    v[2] = __uint_as_float(q.y << 16);
    v[3] = __uint_as_float(q.y & 0xffff0000u);
  }
  __device__ static void store1(uint16_t* p, float a) { *p = static_cast<uint16_t>(pack_bf16x2(a, a)); }
  // two elements to two unrelated places (one conversion)
  __device__ static void store2(uint16_t* p0, uint16_t* p1, float a, float b) {
    const uint32_t u = pack_bf16x2(a, b);
    *p0 = static_cast<uint16_t>(u);
    *p1 = static_cast<uint16_t>(u >> 16);
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
  __device__ static void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
  __device__ static void load4(const float* p, float (&v)[4]) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
  __device__ static void store1(float* p, float a) { *p = a; }
  __device__ static void store2(float* p0, float* p1, float a, float b) {
    *p0 = a;
    *p1 = b;
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

// One wave-wide direct-to-LDS load: lane l copies the 16 bytes at
// sbase + voff (its own address) to LDS byte address lds_base + 16 l.
// sbase (a scalar 64-bit base) and lds_base must be wave-uniform; voff is the
// lane's 32-bit byte offset, the same register for every load of a kernel,
// so no address register is ever rewritten while a load that read it is in
// flight.  (The instruction's immediate offset would move the LDS
// destination as well as the source, so it stays 0.)  Written as asm so
// that the compiler does not track these LDS writes: it would otherwise
// drain every load in flight before each transposing LDS read it cannot
// disambiguate.  The main loop orders them explicitly (s_waitcnt vmcnt
// before each barrier, vmcnt(0) before LDS is reused).  The instruction
// writes no registers.
__device__ __forceinline__ void lds_dma16(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}
// x of lane l ^ 32 (the other half of the wave), without LDS.
__device__ __forceinline__ uint32_t lane_xor32(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (threadIdx.x & 32) ? r[0] : r[1];
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(MO_LDS(p)));
}

}  // namespace mo
