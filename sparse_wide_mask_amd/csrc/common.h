// Shared device helpers for libwide (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define WIDE_DEV __device__ __forceinline__

namespace wide {

constexpr int kWave = 64;

WIDE_DEV float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bf16 bits, round to nearest even (values here are finite).
WIDE_DEV uint16_t f2bf(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

WIDE_DEV uint32_t pack_bf2(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// silu(x) = x / (1 + e^-x), with the hardware exp2 and reciprocal (about 1 ulp
// each; the result is rounded to bf16).  x -> -inf gives -0, x -> +inf gives x.
WIDE_DEV float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}

// 64-bit wave ballot and the number of set lanes below this lane.
WIDE_DEV uint64_t ballot(bool p) { return __ballot(p); }
WIDE_DEV int lane_id() { return __lane_id(); }
WIDE_DEV int popc64(uint64_t x) { return __popcll(x); }
WIDE_DEV int mbcnt(uint64_t word) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(word >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)word, 0u));
}

WIDE_DEV f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
WIDE_DEV f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 MFMA accumulator held by (lane, register i); the column is lane % 32.
WIDE_DEV int acc32_row(int lane, int i) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }
// Row of the 16x16 MFMA accumulator held by (lane, register i); the column is lane % 16.
WIDE_DEV int acc16_row(int lane, int i) { return 4 * (lane >> 4) + i; }

}  // namespace wide
