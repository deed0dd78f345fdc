// RMSNorm of the pre-norm decoder layer: y = x / sqrt(mean(x^2) + eps) * gamma,
// fp32 arithmetic, bf16 in and out.  One work-group of 256 threads per token row;
// each thread moves 16-byte chunks.
#include "common.h"
#include "internal.h"

namespace wide {

__global__ void __launch_bounds__(256) rmsnorm_rows(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ gamma, int d,
                                                    float eps, uint16_t* __restrict__ y) {
  __shared__ float red[4];
  const size_t row = blockIdx.x;
  const uint16_t* xr = x + row * d;
  // rows up to kNormHeld * 2048 elements stay in registers for the second pass
  constexpr int kNormHeld = 4;
  u32x4 held[kNormHeld];
  float ss = 0.f;
  for (int c = threadIdx.x * 8, it = 0; c < d; c += 256 * 8, ++it) {
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
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float inv = rsqrtf(tot / (float)d + eps);
  uint16_t* yr = y + row * d;
  for (int c = threadIdx.x * 8, it = 0; c < d; c += 256 * 8, ++it) {
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
    *reinterpret_cast<u32x4*>(yr + c) = o;
  }
}

void launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, int T, int d, float eps, uint16_t* y,
                    hipStream_t s) {
  {
    WIDE_TRACE("rmsnorm_rows", s);
    rmsnorm_rows<<<T, 256, 0, s>>>(x, gamma, d, eps, y);
  }
}

}  // namespace wide
