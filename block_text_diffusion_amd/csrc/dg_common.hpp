// Device-side helpers shared by the gfx950 kernels: the counter-based generator,
// bf16 packing, wavefront reductions, the temperature rule.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg.h"

namespace dg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

// Generator streams (the third-from-last counter word is gstep, the last the stream).
enum : uint32_t { kStreamGumbel = 0, kStreamRenoise = 1, kStreamInit = 2,
                  kStreamSynChoose = 4, kStreamSynTarget = 5, kStreamSynNoise = 6 };

// Philox4x32-10 (Salmon et al., "Parallel random numbers: as easy as 1, 2, 3",
// SC'11): ten rounds of two 32x32->64 multiplies on words 0 and 2, the high
// halves xored with the other two words and the round key, the key stepped by
// two Weyl increments between rounds.
struct Philox4 { uint32_t w0, w1, w2, w3; };

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0;
    const uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return Philox4{c0, c1, c2, c3};
}

__device__ __forceinline__ uint32_t seed_lo(uint64_t s) { return (uint32_t)s; }
__device__ __forceinline__ uint32_t seed_hi(uint64_t s) { return (uint32_t)(s >> 32); }

// floor(h * n / 2^32): an integer in [0, n) (Lemire's multiply-shift reduction).
__device__ __forceinline__ uint32_t range_draw(uint32_t h, uint32_t n) {
  return (uint32_t)(((uint64_t)h * (uint64_t)n) >> 32);
}

// u = (2*(h >> 9) + 1) * 2^-24, exact in float32 and strictly inside (0, 1);
// Gumbel noise g = -ln(-ln u), evaluated with the hardware base-2 logarithm
// (v_log_f32) and ln x = ln2 * log2 x.  u is never denormal or 1, so both
// logarithm arguments are normal; the result is within a few ulp of the
// correctly rounded value, far inside the score gap that decides a candidate.
__device__ __forceinline__ float gumbel_from_bits(uint32_t h) {
  const float u = (float)(((h >> 9) << 1) | 1u) * 5.9604644775390625e-08f;
  const float t = -kLn2 * __builtin_amdgcn_logf(u);
  return -kLn2 * __builtin_amdgcn_logf(t);
}

// Temperature rule, evaluated in float32 with no contraction:
// T = t_start, or t_start + (t_end - t_start) * (s / (s_max - 1)) on a schedule.
__device__ __forceinline__ float temperature(const dg_ctrl& c) {
  if ((c.flags & DG_T_SCHEDULE) && c.s_max > 1u) {
    const float span = __fsub_rn(c.t_end, c.t_start);
    const float frac = __fdiv_rn((float)c.s_in_block, (float)(c.s_max - 1u));
    return __fadd_rn(c.t_start, __fmul_rn(span, frac));
  }
  return c.t_start;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// (value, id) argmax with ties to the smaller id; NaN values never win.
__device__ __forceinline__ bool better(float v, uint32_t i, float bv, uint32_t bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void wave_argmax(float& v, uint32_t& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o);
    const uint32_t oi = __shfl_xor(i, o);
    if (better(ov, oi, v, i)) { v = ov; i = oi; }
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 h = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }

// Split two floats into bf16 pairs hi = bf16(x), lo = bf16(x - hi): hi + lo
// carries about 16 significant bits of x.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  const float ra = a - bf16_lo_to_f32(hi);
  const float rb = b - bf16_hi_to_f32(hi);
  lo = pack_bf16x2(ra, rb);
}


// ---- global-to-LDS DMA, wait counters and barriers (gfx950) ----
constexpr int kBufFlags = 0x00020000;  // raw 32-bit buffer access (gfx9 family)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufFlags);
}

// vmcnt(n) with the LDS / export counters left open (gfx9 s_waitcnt encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// vmcnt(n) and lgkmcnt(0) together.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// Workgroup barrier without the memory fences of __syncthreads(): those would
// make every wave drain all outstanding vector loads (including the LDS DMA of
// later stages) at each barrier.  LDS DMA completion is handled by the explicit
// vmcnt waits; the asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
typedef __attribute__((address_space(3))) void* lds_ptr_t;

}  // namespace dg
