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
// waves in pairs (wave w takes steps 2w, 2w + 1, 2w + 16, 2w + 17, ...), so both
// halves of an X row's 128-byte line are read by one wave one step apart, and
// each wave reads only its share of X and R.  A wave walks its pairs from a
// start that differs between the work-groups of an XCD (all of which read the
// whole of R), so that they do not all request the same lines of R at once
// (8192 tokens x 112 groups: 34.0 -> 29.5 us); each token's sums still run in
// one fixed order.  K is short and a step's MFMAs are
// few, so the kernel is bound by load latency: a wave keeps two register sets of
// U steps and issues the loads of one set before the MFMAs of the other (one set
// when 16 column tiles take most of the registers).  Each
// wave accumulates all the 16-group MFMA column tiles (v_mfma_f32_16x16x32_bf16)
// of its steps; the eight partial sums are added through LDS in a fixed tree
// order, so the logits (and therefore the selection) are the same on every run.
// Then each wave selects for 4 tokens at once (four independent chains of
// ballots): the k-th largest logit by a 32-step bisection over order-preserving
// integer keys (counts by ballot + popcount), then the ties at that value in
// group order.
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

// One router of a launch: its groups are the logit columns col0 .. col0 + n - 1
// (whole 16-column tiles from col0); outputs as wide_router_topk (logits and
// packed may be null).
struct RtSet {
  int col0, n, k;
  float* logits;
  uint8_t* mask;
  uint64_t* packed;
};

// Selection of one router for the wave's TPW tokens (w, w + 8, ...) from the
// logits in LDS: groups g = lane + 64 i, i < the set's word count (uniform).
template <int NWC, int TPW, int LD>
WIDE_DEV void rt_select(const float* __restrict__ sL, const RtSet& st, int wave, int lane,
                        int t0, int rows) {
  const int n = st.n, k = st.k, nw = (n + 63) / 64;
  bool valid[NWC];
#pragma unroll
  for (int i = 0; i < NWC; ++i) valid[i] = lane + 64 * i < n;
  float v[TPW][NWC];
  // key 0 for groups past n: every threshold the search tests is at least 1, so
  // they never count, and each ballot is one compare with no branch on the word
  // count (words past it hold only such lanes)
  uint32_t key[TPW][NWC];
  bool keep[TPW][NWC];
#pragma unroll
  for (int q = 0; q < TPW; ++q)
#pragma unroll
    for (int i = 0; i < NWC; ++i) {
      v[q][i] = valid[i] ? sL[(wave + kRtWaves * q) * LD + st.col0 + lane + 64 * i] : 0.f;
      key[q][i] = valid[i] ? order_key(v[q][i]) : 0u;
      keep[q][i] = valid[i] && k >= n;
    }
  if (k > 0 && k < n) {
    // the k-th largest key: the largest value with at least k keys >= it (the
    // TPW tokens' searches are independent chains of ballots)
    uint32_t kth[TPW];
#pragma unroll
    for (int q = 0; q < TPW; ++q) kth[q] = 0u;
    for (int b = 31; b >= 0; --b) {
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        const uint32_t cand = kth[q] | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < NWC; ++i) cnt += popc64(ballot(key[q][i] >= cand));
        kth[q] = cnt >= k ? cand : kth[q];
      }
    }
#pragma unroll
    for (int q = 0; q < TPW; ++q) {
      int above = 0;
#pragma unroll
      for (int i = 0; i < NWC; ++i) above += popc64(ballot(key[q][i] > kth[q]));
      // keys equal to the k-th: the first k - above of them in group order
      const int need = k - above;
      int before = 0;
#pragma unroll
      for (int i = 0; i < NWC; ++i) {
        const bool eq = valid[i] && key[q][i] == kth[q];
        const uint64_t bal = ballot(eq);
        const int rank = before + popc64(bal & ((1ull << lane) - 1ull));
        keep[q][i] = key[q][i] > kth[q] || (eq && rank < need);
        before += popc64(bal);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int tt = wave + kRtWaves * q;
    if (tt >= rows) break;
    const size_t t = (size_t)(t0 + tt);
#pragma unroll
    for (int i = 0; i < NWC; ++i) {
      if (i >= nw) break;
      const int g = lane + 64 * i;
      const uint64_t word = ballot(keep[q][i]);
      if (lane == 0 && st.packed) st.packed[t * nw + i] = word;
      if (g < n) {
        st.mask[t * n + g] = keep[q][i] ? 1 : 0;
        if (st.logits) st.logits[t * n + g] = v[q][i];
      }
    }
  }
}

// NT: 16-group column tiles computed (>= the tiles of both routers); U: K steps
// per register set.  Tiles 0 .. ntA - 1 come from RpA (router a, columns from 0),
// tiles ntA .. ntA + ntB - 1 from RpB (router b, columns from 16 ntA; ntB = 0:
// one router).
template <int NT, int U>
__global__ void __launch_bounds__(kRtThreads)
    router_topk_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ RpA,
                       int ntA, const uint16_t* __restrict__ RpB, int ntB, int T, int d,
                       RtSet sa, RtSet sb) {
  constexpr int NG = 16 * NT;
  constexpr int NWC = (NG + 63) / 64;  // 64-group words of a token's logits
  constexpr int TPW = kRtTok / kRtWaves;  // tokens per wave in the selection
  // partial sums of waves 4..7 (then 2..3, then 1), and at the end the logits
  __shared__ float sP[4][kRtTok][NG + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kRtTok;
  const int rows = min(kRtTok, T - t0);
  const int ch = lane & 15, koff = 8 * (lane >> 4);
  const rsrc_t xr = make_rsrc(X + (size_t)t0 * d, (uint32_t)((size_t)rows * d * 2));
  const int nsteps = d / 32;
  const rsrc_t ra = make_rsrc(RpA, (uint32_t)((size_t)ntA * 16 * d * 2));
  const rsrc_t rb2 = make_rsrc(RpB, RpB ? (uint32_t)((size_t)ntB * 16 * d * 2) : 0u);

  f32x4 acc[NT][2];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j][0] = acc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  // this wave's steps, in pairs: the i-th is 2 wave + (i & 1) + 16 j with
  // j = (i >> 1) + rot mod mine / 2 (d % 64 == 0: d / 32 is even)
  const int mine = 2 * ((nsteps / 2 - wave + kRtWaves - 1) / kRtWaves);
  // this wave's pairs, mine / 2 of them, from pair rot on (XCD x runs work-groups
  // x, x + 8, ...: neighbours there get different starts)
  const int jw = mine / 2 > 0 ? mine / 2 : 1;
  const int rot = (int)((blockIdx.x >> 3) % (unsigned)jw);
  // steps i0 .. i0 + U - 1 of the wave; past `mine` every load reads zeros (and
  // its step index, which may then pass the wave's pairs, is not used)
  auto load = [&](int i0, bf16x8 (&a)[U][2], bf16x8 (&b)[U][NT]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u;
      const bool live = i < mine;
      int pj = (i >> 1) + rot;
      pj = pj >= jw ? pj - jw : pj;
      const int step = 2 * wave + (i & 1) + 2 * kRtWaves * pj;
      const int col = step * 32 + koff;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const u32x4 v = ldbuf16(xr, live ? (uint32_t)(((rb * 16 + ch) * d + col) * 2) : kSkip);
        a[u][rb] = *reinterpret_cast<const bf16x8*>(&v);
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const bool first = j < ntA;
        const int jt = first ? j : j - ntA;
        const u32x4 v = ldbuf16(first ? ra : rb2,
                                live && j < ntA + ntB
                                    ? (uint32_t)((((size_t)jt * nsteps + step) * 64 + lane) * 16)
                                    : kSkip);
        b[u][j] = *reinterpret_cast<const bf16x8*>(&v);
      }
    }
  };
  auto mma = [&](const bf16x8 (&a)[U][2], const bf16x8 (&b)[U][NT]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) acc[j][rb] = mfma16(a[u][rb], b[u][j], acc[j][rb]);
  };
  if constexpr (NT <= 8) {
    bf16x8 a0[U][2], b0[U][NT], a1[U][2], b1[U][NT];
    load(0, a0, b0);
    for (int i0 = 0; i0 < mine; i0 += 2 * U) {
      load(i0 + U, a1, b1);
      mma(a0, b0);
      if (i0 + U >= mine) break;
      load(i0 + 2 * U, a0, b0);
      mma(a1, b1);
    }
  } else {  // 16 tiles: the accumulators leave room for one register set
    for (int i0 = 0; i0 < mine; i0 += U) {
      bf16x8 a[U][2], b[U][NT];
      load(i0, a, b);
      mma(a, b);
    }
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

  // selection, router by router, over as many 64-group words as the router has
  auto select = [&](const RtSet& st) {
    if constexpr (NWC > 1) {
      if (st.n <= 64) {
        rt_select<1, TPW, NG + 1>(&sL[0][0], st, wave, lane, t0, rows);
        return;
      }
    }
    rt_select<NWC, TPW, NG + 1>(&sL[0][0], st, wave, lane, t0, rows);
  };
  select(sa);
  if (ntB > 0) select(sb);
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

static auto router_kernel_for(int ntiles) {
  return ntiles <= 1   ? router_topk_kernel<1, 4>
         : ntiles <= 2 ? router_topk_kernel<2, 4>
         : ntiles <= 4 ? router_topk_kernel<4, 4>
         : ntiles <= 8 ? router_topk_kernel<8, 2>
                       : router_topk_kernel<16, 2>;
}

void launch_router_topk(const uint16_t* X, const uint16_t* R, int T, int d, int n, int k,
                        float* logits, uint8_t* mask, uint64_t* packed, hipStream_t s) {
  WIDE_TRACE("router_topk", s);
  const int ntiles = (n + 15) / 16;
  const dim3 grid((T + kRtTok - 1) / kRtTok);
  router_kernel_for(ntiles)<<<grid, kRtThreads, 0, s>>>(
      X, R, ntiles, nullptr, 0, T, d, RtSet{0, n, k, logits, mask, packed},
      RtSet{0, 0, 0, nullptr, nullptr, nullptr});
}

void launch_router_topk2(const uint16_t* X, int T, int d, const uint16_t* Ra, int na, int ka,
                         uint8_t* mask_a, uint64_t* packed_a, const uint16_t* Rb, int nb, int kb,
                         uint8_t* mask_b, uint64_t* packed_b, hipStream_t s) {
  const int ta = (na + 15) / 16, tb = (nb + 15) / 16;
  if (ta + tb > 16) {
    launch_router_topk(X, Ra, T, d, na, ka, nullptr, mask_a, packed_a, s);
    launch_router_topk(X, Rb, T, d, nb, kb, nullptr, mask_b, packed_b, s);
    return;
  }
  WIDE_TRACE("router_topk", s);
  const dim3 grid((T + kRtTok - 1) / kRtTok);
  router_kernel_for(ta + tb)<<<grid, kRtThreads, 0, s>>>(
      X, Ra, ta, Rb, tb, T, d, RtSet{0, na, ka, nullptr, mask_a, packed_a},
      RtSet{16 * ta, nb, kb, nullptr, mask_b, packed_b});
}

}  // namespace wide
