// RMSNorm of the pre-norm decoder layer (the second norm of a prefill layer and
// both norms of a decode layer): one work-group of 256 threads per token row.
// The first norm of a prefill layer runs inside the reorder launch (reorder.hip).
#include "common.h"
#include "internal.h"
#include "norm_row.h"

namespace wide {

__global__ void __launch_bounds__(256) rmsnorm_rows(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ gamma, int d,
                                                    float eps, uint16_t* __restrict__ y) {
  __shared__ float red[4];
  const size_t row = blockIdx.x;
  rms_row(x + row * d, gamma, d, eps, y + row * d, threadIdx.x, red);
}

void launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, int T, int d, float eps, uint16_t* y,
                    hipStream_t s) {
  {
    WIDE_TRACE("rmsnorm_rows", s);
    rmsnorm_rows<<<T, 256, 0, s>>>(x, gamma, d, eps, y);
  }
}

}  // namespace wide
