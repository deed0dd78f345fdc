// One row of the pre-norm layer's RMSNorm, y = x / sqrt(mean(x^2) + eps) * gamma,
// fp32 arithmetic, bf16 in and out, done by 256 threads (four waves) of a
// work-group; each thread moves 16-byte chunks.  `red` is four floats of LDS
// owned by these 256 threads; the caller's barrier structure is the work-group's
// (every thread of the work-group calls this the same number of times).  yr null:
// compute without storing.
#pragma once

#include "common.h"

namespace wide {

WIDE_DEV void rms_row(const uint16_t* __restrict__ xr, const uint16_t* __restrict__ gamma, int d,
                      float eps, uint16_t* __restrict__ yr, int t256, float* red) {
  // rows up to kNormHeld * 2048 elements stay in registers for the second pass
  constexpr int kNormHeld = 4;
  u32x4 held[kNormHeld];
  float ss = 0.f;
  for (int c = t256 * 8, it = 0; c < d; c += 256 * 8, ++it) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(xr + c);
#pragma unroll
    for (int q = 0; q < kNormHeld; ++q)
      if (q == it) held[q] = v;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = __uint_as_float(v[k] << 16), b = __uint_as_float(v[k] & 0xffff0000u);
      ss += a * a + b * b;
    }
  }
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if ((t256 & 63) == 0) red[t256 >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float inv = rsqrtf(tot / (float)d + eps);
  for (int c = t256 * 8, it = 0; c < d; c += 256 * 8, ++it) {
    u32x4 v;
    if (it < kNormHeld) {
#pragma unroll
      for (int q = 0; q < kNormHeld; ++q)
        if (q == it) v = held[q];
    } else {
      v = *reinterpret_cast<const u32x4*>(xr + c);
    }
    const u32x4 gm = *reinterpret_cast<const u32x4*>(gamma + c);
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = __uint_as_float(v[k] << 16) * inv * __uint_as_float(gm[k] << 16);
      const float b = __uint_as_float(v[k] & 0xffff0000u) * inv * __uint_as_float(gm[k] & 0xffff0000u);
      o[k] = pack_bf2(a, b);
    }
    if (yr) *reinterpret_cast<u32x4*>(yr + c) = o;
  }
}

}  // namespace wide
