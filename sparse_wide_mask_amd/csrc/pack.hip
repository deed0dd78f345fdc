// Packing of K-masked weights: W [n*G, d] -> Wp [n, d, G] (per group, the block
// transposed), so a kept group's weights are one contiguous region with the
// contraction index innermost.  A pure permutation, run once at weight load.
#include "common.h"
#include "internal.h"

namespace wide {

__global__ void __launch_bounds__(256) pack_kmajor(const uint16_t* __restrict__ W, int G, int d,
                                                   uint16_t* __restrict__ Wp) {
  __shared__ uint16_t tile[64][65];
  const int c0 = blockIdx.x * 64, j0 = blockIdx.y * 64, g = blockIdx.z;
  const int jn = min(64, G - j0);  // rows of the group's block in this tile (G = 32: 32)
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const uint16_t* src = W + ((size_t)g * G + j0) * d + c0;
  for (int j = ty; j < jn; j += 4) tile[j][tx] = src[(size_t)j * d + tx];
  __syncthreads();
  uint16_t* dst = Wp + ((size_t)g * d + c0) * G + j0;
  for (int c = ty; c < 64; c += 4)
    if (tx < jn) dst[(size_t)c * G + tx] = tile[tx][c];
}

void launch_pack_kmajor(const uint16_t* W, int n, int G, int d, uint16_t* Wp, hipStream_t s) {
  dim3 grid(d / 64, (G + 63) / 64, n);
  {
    WIDE_TRACE("pack_kmajor", s);
    pack_kmajor<<<grid, 256, 0, s>>>(W, G, d, Wp);
  }
}

}  // namespace wide
