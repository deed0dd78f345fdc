// Router and top-k selection, the step before the masked path (gist.science
// technical summary §2.A: a router gives every token one binary execute/skip
// decision per group; the abstract: each token selects its own groups).
//
//   logits[t, g] = X[t, :] . R[g, :]        bf16 operands, fp32 accumulation
//   mask[t, g]   = 1 for the k largest logits of token t, ties to the lower
//                  group index (-0.0 and +0.0 are equal)
//   packed[t, w] = the mask's little-endian bit words (what the reorder packs)
//
// R is used in "fragment order" (wide_pack_router): for every 16-group tile j and
// 32-wide K step s, the 64 lanes' 16-byte B fragments of v_mfma_f32_16x16x32_bf16
// are one contiguous 1 KB block, so every work-group's reads of R (all of it, from
// L2) are whole cache lines instead of 16 rows x 64 bytes.
//
// One work-group = 32 tokens, 8 waves.  The 32-wide K steps are dealt to the
// waves round-robin, so each wave reads only its share of X and R and keeps
// several steps of loads in flight (K is short and a step's MFMAs are few: the
// kernel is bound by load latency, not arithmetic).  Each wave accumulates all
// the 16-group MFMA column tiles (v_mfma_f32_16x16x32_bf16) of its steps; the
// eight partial sums are added through LDS in a fixed tree order, so the logits
// (and therefore the selection) are the same on every run.  Then one wave per
// token selects: the k-th largest logit by a 32-step bisection over
// order-preserving integer keys (counts by ballot + popcount), then the ties at
// that value in group order.
#include "common.h"
#include "gemm_tile.h"
#include "internal.h"
#include "wide.h"

#include <algorithm>

namespace wide {

constexpr int kRtTok = 32;                 // tokens per work-group
constexpr int kRtWaves = 8;
constexpr int kRtThreads = 64 * kRtWaves;

// Order-preserving integer key of a finite float (a > b iff key(a) > key(b));
// -0.0 maps to the key of +0.0.
WIDE_DEV uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// NT: 16-group column tiles computed (>= the n_groups / 16 rounded up); U: K steps
// whose loads are issued together.
template <int NT, int U>
__global__ void __launch_bounds__(kRtThreads)
    router_topk_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Rp, int T,
                       int d, int n, int k, float* __restrict__ logits,
                       uint8_t* __restrict__ mask, uint64_t* __restrict__ packed) {
  constexpr int NG = 16 * NT;
  // partial sums of waves 4..7 (then 2..3, then 1), and at the end the logits
  __shared__ float sP[4][kRtTok][NG + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kRtTok;
  const int rows = min(kRtTok, T - t0);
  const int ch = lane & 15, koff = 8 * (lane >> 4);
  const rsrc_t xr = make_rsrc(X + (size_t)t0 * d, (uint32_t)((size_t)rows * d * 2));
  const int ntiles = (n + 15) / 16, nsteps = d / 32;
  const rsrc_t rr = make_rsrc(Rp, (uint32_t)((size_t)ntiles * 16 * d * 2));

  f32x4 acc[NT][2];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j][0] = acc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  // this wave's K steps: wave, wave + 8, ...  (d % 64 == 0: d / 32 is even)
  const int mine = (nsteps - wave + kRtWaves - 1) / kRtWaves;
  for (int i0 = 0; i0 < mine; i0 += U) {
    bf16x8 a[U][2], b[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = i0 + u < mine;
      const int step = wave + kRtWaves * (i0 + u);
      const int col = step * 32 + koff;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const u32x4 v = ldbuf16(xr, live ? (uint32_t)(((rb * 16 + ch) * d + col) * 2) : kSkip);
        a[u][rb] = *reinterpret_cast<const bf16x8*>(&v);
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const u32x4 v = ldbuf16(rr, live && j < ntiles
                                        ? (uint32_t)((((size_t)j * nsteps + step) * 64 + lane) * 16)
                                        : kSkip);
        b[u][j] = *reinterpret_cast<const bf16x8*>(&v);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) acc[j][rb] = mfma16(a[u][rb], b[u][j], acc[j][rb]);
  }

  // fixed-order tree over the waves: 4..7 -> 0..3, 2..3 -> 0..1, 1 -> 0
  for (int half = kRtWaves / 2; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half) {
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sP[wave - half][rb * 16 + acc16_row(lane, i)][j * 16 + ch] = acc[j][rb][i];
    }
    __syncthreads();
    if (wave < half) {
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[j][rb][i] += sP[wave][rb * 16 + acc16_row(lane, i)][j * 16 + ch];
    }
    __syncthreads();
  }
  float (*sL)[NG + 1] = sP[0];
  if (wave == 0) {
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sL[rb * 16 + acc16_row(lane, i)][j * 16 + ch] = acc[j][rb][i];
  }
  __syncthreads();

  // selection: one wave per token; group g = lane + 64 i
  const int nw = (n + 63) / 64;
  for (int tt = wave; tt < rows; tt += kRtWaves) {
    const size_t t = (size_t)(t0 + tt);
    float v[4];
    uint32_t key[4];
    bool valid[4], keep[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = lane + 64 * i;
      valid[i] = g < n;
      v[i] = valid[i] ? sL[tt][g] : 0.f;
      key[i] = valid[i] ? order_key(v[i]) : 0u;
      keep[i] = valid[i] && k >= n;
    }
    if (k > 0 && k < n) {
      // the k-th largest key: the largest value with at least k keys >= it
      uint32_t kth = 0u;
      for (int b = 31; b >= 0; --b) {
        const uint32_t cand = kth | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) cnt += popc64(ballot(valid[i] && key[i] >= cand));
        if (cnt >= k) kth = cand;
      }
      int above = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) above += popc64(ballot(valid[i] && key[i] > kth));
      // keys equal to the k-th: the first k - above of them in group order
      const int need = k - above;
      int before = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool eq = valid[i] && key[i] == kth;
        const uint64_t bal = ballot(eq);
        const int rank = before + popc64(bal & ((1ull << lane) - 1ull));
        keep[i] = (valid[i] && key[i] > kth) || (eq && rank < need);
        before += popc64(bal);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = lane + 64 * i;
      const uint64_t word = ballot(keep[i]);
      if (i < nw && lane == 0 && packed) packed[t * nw + i] = word;
      if (g < n) {
        mask[t * n + g] = keep[i] ? 1 : 0;
        if (logits) logits[t * n + g] = v[i];
      }
    }
  }
}

// R [n, d] -> fragment order [ceil(n/16)][d/32][64 lanes][8]: lane l of block
// (j, s) holds R[16 j + (l mod 16)][32 s + 8 (l / 16) .. +7], zeros past n.
__global__ void __launch_bounds__(256)
    pack_router_kernel(const uint16_t* __restrict__ R, int n, int d, uint16_t* __restrict__ Rp) {
  const int ntiles = (n + 15) / 16, nsteps = d / 32;
  const size_t total = (size_t)ntiles * nsteps * 64;
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
    const int l = (int)(i % 64);
    const size_t js = i / 64;
    const int s = (int)(js % nsteps), j = (int)(js / nsteps);
    const int g = j * 16 + (l & 15), k = s * 32 + 8 * (l >> 4);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (g < n) v = *reinterpret_cast<const u32x4*>(R + (size_t)g * d + k);
    *reinterpret_cast<u32x4*>(Rp + i * 8) = v;
  }
}

void launch_pack_router(const uint16_t* R, int n, int d, uint16_t* Rp, hipStream_t s) {
  WIDE_TRACE("pack_router", s);
  const size_t chunks = (size_t)((n + 15) / 16) * (d / 32) * 64;
  const int grid = (int)std::min<size_t>((chunks + 255) / 256, 4096);
  pack_router_kernel<<<grid, 256, 0, s>>>(R, n, d, Rp);
}

void launch_router_topk(const uint16_t* X, const uint16_t* R, int T, int d, int n, int k,
                        float* logits, uint8_t* mask, uint64_t* packed, hipStream_t s) {
  WIDE_TRACE("router_topk", s);
  const int ntiles = (n + 15) / 16;
  const dim3 grid((T + kRtTok - 1) / kRtTok);
  auto kern = ntiles <= 1   ? router_topk_kernel<1, 8>
              : ntiles <= 2 ? router_topk_kernel<2, 8>
              : ntiles <= 4 ? router_topk_kernel<4, 6>
              : ntiles <= 8 ? router_topk_kernel<8, 4>
                            : router_topk_kernel<16, 2>;
  kern<<<grid, kRtThreads, 0, s>>>(X, R, T, d, n, k, logits, mask, packed);
}

}  // namespace wide
