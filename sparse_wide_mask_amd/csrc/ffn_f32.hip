// Masked SwiGLU FFN in fp32 (gist.science technical summary §2.A: contiguous
// channel groups of the intermediate dimension D', one execute/skip bit per token
// and group), for problems checked at fp32 precision rather than run fast: fp32
// operands, fp32 products and sums on the vector units (fmaf), no matrix cores.
//
// up   H[t, c] = silu(X[t] . Wg[c]) * (X[t] . Wu[c]) where token t keeps the group
//      of channel c, else exactly 0.
// down Y[t, j] = sum over c of H[t, c] Wd[c, j], c ascending; the dropped channels
//      hold exact zeros and add nothing, so this is the sum over the kept groups.
//
// A work-group owns 16 tokens x 64 output columns; a thread owns one token and the
// columns tx, tx + 16, tx + 32, tx + 48 of the tile.  K runs in chunks of 64 staged
// in LDS (rows padded to 65 words: the 16 column rows a wave reads at one K index
// fall in 16 different banks).  A tile whose tokens keep none of its groups writes
// zeros at once (up) or passes the K chunks of such groups (down): block-level
// skipping.  Every sum runs in one fixed order, so results repeat bit for bit.
#include "common.h"
#include "internal.h"
#include "wide.h"

namespace wide {

constexpr int kF32Rows = 16;
constexpr int kF32Cols = 64;
constexpr int kF32K = 64;
constexpr int kF32Threads = 256;
constexpr int kF32Pad = kF32K + 1;

__global__ void __launch_bounds__(kF32Threads)
    ffn_up_f32(const float* __restrict__ X, const uint8_t* __restrict__ mask,
               const float* __restrict__ Wg, const float* __restrict__ Wu, int T, int d, int F,
               int n, float* __restrict__ H) {
  __shared__ float sX[kF32Rows][kF32Pad];
  __shared__ float sG[kF32Cols][kF32Pad];
  __shared__ float sU[kF32Cols][kF32Pad];
  __shared__ uint8_t sKeep[kF32Rows][kF32Cols];
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int c0 = blockIdx.x * kF32Cols, t0 = blockIdx.y * kF32Rows;
  const int G = F / n, t = t0 + ty;
  bool any = false;
  for (int i = tid; i < kF32Rows * kF32Cols; i += kF32Threads) {
    const int r = i / kF32Cols, cc = i % kF32Cols, tt = t0 + r, c = c0 + cc;
    const bool k = tt < T && c < F && mask[(size_t)tt * n + c / G] != 0;
    sKeep[r][cc] = k ? 1 : 0;
    any = any || k;
  }
  if (!__syncthreads_or(any)) {  // l=0: no token of the tile keeps a group of these channels
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = c0 + tx + 16 * j;
      if (t < T && c < F) H[(size_t)t * F + c] = 0.f;
    }
    return;
  }
  float ag[4] = {0.f, 0.f, 0.f, 0.f}, au[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < d; k0 += kF32K) {
    for (int i = tid; i < kF32Rows * kF32K; i += kF32Threads) {
      const int r = i / kF32K, kk = i % kF32K;
      sX[r][kk] = (t0 + r < T && k0 + kk < d) ? X[(size_t)(t0 + r) * d + k0 + kk] : 0.f;
    }
    for (int i = tid; i < kF32Cols * kF32K; i += kF32Threads) {
      const int cc = i / kF32K, kk = i % kF32K;
      const bool ok = c0 + cc < F && k0 + kk < d;
      sG[cc][kk] = ok ? Wg[(size_t)(c0 + cc) * d + k0 + kk] : 0.f;
      sU[cc][kk] = ok ? Wu[(size_t)(c0 + cc) * d + k0 + kk] : 0.f;
    }
    __syncthreads();
    const int kn = min(kF32K, d - k0);
    for (int kk = 0; kk < kn; ++kk) {
      const float x = sX[ty][kk];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ag[j] = fmaf(x, sG[tx + 16 * j][kk], ag[j]);
        au[j] = fmaf(x, sU[tx + 16 * j][kk], au[j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = c0 + tx + 16 * j;
    if (t >= T || c >= F) continue;
    float h = 0.f;
    if (sKeep[ty][tx + 16 * j]) h = ag[j] / (1.f + expf(-ag[j])) * au[j];
    H[(size_t)t * F + c] = h;
  }
}

__global__ void __launch_bounds__(kF32Threads)
    ffn_down_f32(const float* __restrict__ H, const uint8_t* __restrict__ mask,
                 const float* __restrict__ Wd, int T, int d, int F, int n,
                 float* __restrict__ Y) {
  __shared__ float sH[kF32Rows][kF32Pad];
  __shared__ float sW[kF32K][kF32Cols + 1];
  __shared__ uint8_t sUnion[WIDE_MAX_GROUPS];
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int c0 = blockIdx.x * kF32Cols, t0 = blockIdx.y * kF32Rows;
  const int G = F / n, t = t0 + ty;
  for (int g = tid; g < n; g += kF32Threads) {
    bool u = false;
    for (int r = 0; r < kF32Rows && t0 + r < T; ++r) u = u || mask[(size_t)(t0 + r) * n + g] != 0;
    sUnion[g] = u ? 1 : 0;
  }
  __syncthreads();
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < F; k0 += kF32K) {
    const int kn = min(kF32K, F - k0);
    // l=0: a chunk of channels whose groups no token of the tile keeps holds only
    // zeros of H (the same for every thread of the work-group)
    bool live = false;
    for (int g = k0 / G; g <= (k0 + kn - 1) / G; ++g) live = live || sUnion[g];
    if (!live) continue;
    for (int i = tid; i < kF32Rows * kF32K; i += kF32Threads) {
      const int r = i / kF32K, kk = i % kF32K;
      sH[r][kk] = (t0 + r < T && kk < kn) ? H[(size_t)(t0 + r) * F + k0 + kk] : 0.f;
    }
    for (int i = tid; i < kF32K * kF32Cols; i += kF32Threads) {
      const int kk = i / kF32Cols, cc = i % kF32Cols;
      sW[kk][cc] = (kk < kn && c0 + cc < d) ? Wd[(size_t)(k0 + kk) * d + c0 + cc] : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < kn; ++kk) {
      const float h = sH[ty][kk];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = fmaf(h, sW[kk][tx + 16 * j], acc[j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = c0 + tx + 16 * j;
    if (t < T && c < d) Y[(size_t)t * d + c] = acc[j];
  }
}

void launch_ffn_f32(const float* X, const uint8_t* mask, const float* Wg, const float* Wu,
                    const float* Wd, int T, int d, int F, int n, float* H, float* Y,
                    hipStream_t s) {
  const int ty = (T + kF32Rows - 1) / kF32Rows;
  {
    WIDE_TRACE("ffn_up_f32", s);
    ffn_up_f32<<<dim3((F + kF32Cols - 1) / kF32Cols, ty), kF32Threads, 0, s>>>(X, mask, Wg, Wu,
                                                                               T, d, F, n, H);
  }
  {
    WIDE_TRACE("ffn_down_f32", s);
    ffn_down_f32<<<dim3((d + kF32Cols - 1) / kF32Cols, ty), kF32Threads, 0, s>>>(H, mask, Wd, T,
                                                                                 d, F, n, Y);
  }
}

}  // namespace wide
