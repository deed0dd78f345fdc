// Masked SwiGLU FFN, prefill (gist.science technical summary §2.A units, §2.B
// reordering, §2.C skipping).
//
// up   (N-masked): one output tile = (group g, 256 consecutive entries of g's
//      kept-token list, 128 channels of g).  Rows of X are gathered through
//      group_perm, so only kept (token, group) pairs are multiplied; a tile past
//      group_count[g] exits at once (l=0), rows past it are never loaded (l=1)
//      and their MFMA row blocks are skipped (l=2).  B interleaves 32-channel
//      slabs of W_gate and W_up so each lane holds gate and up of the same
//      (token, channel) and applies silu(gate) * up in registers.  H is written
//      token-major [T, d_ff] at the kept blocks only.
// down (K-masked): one output tile = (256 consecutive tokens, 256 columns of
//      d_model); K runs over the groups that some token of the tile keeps
//      (tile_groups, l=0 for the others), G channels each.  A rows of tokens that
//      dropped the group are not loaded (zeros, l=1) and 32-row MFMA blocks with
//      no such token are skipped (l=2).  W_down is read in the packed K-major
//      group layout.
#include "common.h"
#include "gemm_tile.h"
#include "internal.h"

namespace wide {

// Work-group id -> (group, rest) so that the tiles of one group land on one XCD
// (work-groups are dealt to the 8 XCDs round-robin) and share its L2.
WIDE_DEV void xcd_group_split(int bid, int n_groups, int per_group, int& g, int& rest) {
  if ((n_groups & 7) == 0) {
    const int x = bid & 7, l = bid >> 3;
    g = (l / per_group) * 8 + x;
    rest = l % per_group;
  } else {
    g = bid / per_group;
    rest = bid % per_group;
  }
}

template <int BM, int BN>
__global__ void __launch_bounds__(256, 1)
    ffn_up_prefill(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wg,
                   const uint16_t* __restrict__ Wu, const int32_t* __restrict__ gcount,
                   const int32_t* __restrict__ gperm, int T, int d, int F, int n, int G,
                   int mtiles, int ntn, uint16_t* __restrict__ H) {
  using C = TileCfg<BM, BN>;
  constexpr int BNH = BN / 2;  // channels per tile (gate and up each)
  __shared__ __attribute__((aligned(16))) uint16_t sA[C::LDS_A];
  __shared__ __attribute__((aligned(16))) uint16_t sB[C::LDS_B];
  __shared__ int sTok[BM];

  int g, rest;
  xcd_group_split(blockIdx.x, n, mtiles * ntn, g, rest);
  const int mt = rest % mtiles, nt = rest / mtiles;
  const int cnt = gcount[g];
  const int row0 = mt * BM;
  if (row0 >= cnt) return;  // l=0: no kept token left in this tile
  const int rows = min(BM, cnt - row0);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  for (int r = tid; r < BM; r += C::kThreads) sTok[r] = r < rows ? gperm[(size_t)g * T + row0 + r] : -1;
  __syncthreads();

  // Chunk i of this thread: tile row (tid >> 3) + 32 i, 16-byte column kc = tid & 7.
  const int crow = tid >> 3, kc8 = (tid & 7) * 8;
  const int dst0 = crow * kLdsLd + kc8;
  int aOff[C::A_CHUNKS];
#pragma unroll
  for (int i = 0; i < C::A_CHUNKS; ++i) {
    const int tok = sTok[crow + 32 * i];
    aOff[i] = tok >= 0 ? tok * d + kc8 : -1;
  }
  const uint16_t* bSrc[C::B_CHUNKS];
#pragma unroll
  for (int i = 0; i < C::B_CHUNKS; ++i) {
    const int nrow = crow + 32 * i;
    const int w = nrow / C::WN, local = nrow % C::WN, blk = local >> 5;
    const int ch = nt * BNH + w * (C::WN / 2) + (blk >> 1) * 32 + (local & 31);
    bSrc[i] = ((blk & 1) ? Wu : Wg) + (size_t)(g * G + ch) * d + kc8;
  }

  uint32_t rb_live = 0;
#pragma unroll
  for (int i = 0; i < C::RB; ++i)
    if (wm * C::WM + i * 32 < rows) rb_live |= 1u << i;

  u32x4 ra[C::A_CHUNKS], rbuf[C::B_CHUNKS];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::A_CHUNKS; ++i) ra[i] = aOff[i] >= 0 ? ld16(X + aOff[i] + k0) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < C::B_CHUNKS; ++i) rbuf[i] = ld16(bSrc[i] + k0);
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < C::A_CHUNKS; ++i) st16(sA + dst0 + 32 * i * kLdsLd, ra[i]);
#pragma unroll
    for (int i = 0; i < C::B_CHUNKS; ++i) st16(sB + dst0 + 32 * i * kLdsLd, rbuf[i]);
  };

  WaveAcc<BM, BN> acc;
  acc.zero();
  const int nk = d / kBK;
  gload(0);
  lstore();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload((kt + 1) * kBK);
    acc.sweep(sA, sB, wm, wn, lane, rb_live);
    __syncthreads();
    if (kt + 1 < nk) {
      lstore();
      __syncthreads();
    }
  }

  // epilogue: H[token, gG + ch] = silu(gate) * up
#pragma unroll
  for (int i = 0; i < C::RB; ++i) {
    if (!((rb_live >> i) & 1u)) continue;
#pragma unroll
    for (int jp = 0; jp < C::CB / 2; ++jp) {
      const f32x16 gt = acc.acc[i][2 * jp], up = acc.acc[i][2 * jp + 1];
      const int ch = nt * BNH + wn * (C::WN / 2) + jp * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = wm * C::WM + i * 32 + acc32_row(lane, e);
        if (row < rows) H[(size_t)sTok[row] * F + g * G + ch] = f2bf(silu(gt[e]) * up[e]);
      }
    }
  }
}

template <int BM, int BN>
__global__ void __launch_bounds__(256, 1)
    ffn_down_prefill(const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wdp,
                     const uint64_t* __restrict__ packed, const int32_t* __restrict__ tcount,
                     const int32_t* __restrict__ tgroups, int T, int d, int F, int n, int G,
                     int nw, int ntn, const uint16_t* __restrict__ residual,
                     uint16_t* __restrict__ Y) {
  using C = TileCfg<BM, BN>;
  __shared__ __attribute__((aligned(16))) uint16_t sA[C::LDS_A];
  __shared__ __attribute__((aligned(16))) uint16_t sB[C::LDS_B];
  __shared__ uint64_t sBits[BM * 4];
  __shared__ int sGroups[256];

  const int mt = blockIdx.x / ntn, nt = blockIdx.x % ntn;
  const int t0 = mt * BM, rows = min(BM, T - t0), n0 = nt * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int ng = tcount[mt];
  for (int i = tid; i < BM * nw; i += C::kThreads) {
    const int r = i / nw, w = i % nw;
    sBits[r * 4 + w] = r < rows ? packed[(size_t)(t0 + r) * nw + w] : 0ull;
  }
  for (int i = tid; i < ng; i += C::kThreads) sGroups[i] = tgroups[(size_t)mt * n + i];
  __syncthreads();

  // Chunk i of this thread: tile row (tid >> 3) + 32 i, 16-byte column kc = tid & 7.
  const int crow = tid >> 3, kc8 = (tid & 7) * 8;
  const int dst0 = crow * kLdsLd + kc8;
  const size_t aBase = (size_t)(t0 + crow) * F + kc8;
  const size_t bBase = (size_t)(n0 + crow) * G + kc8;

  const int kpg = G / kBK;
  const int nk = ng * kpg;
  u32x4 ra[C::A_CHUNKS], rbuf[C::B_CHUNKS];
  auto gload = [&](int it) {
    const int g = sGroups[it / kpg], kk = (it % kpg) * kBK;
    const uint64_t sel = 1ull << (g & 63);
    const int w = g >> 6;
#pragma unroll
    for (int i = 0; i < C::A_CHUNKS; ++i) {
      const int row = crow + 32 * i;
      const bool keep = row < rows && (sBits[row * 4 + w] & sel);
      ra[i] = keep ? ld16(H + aBase + (size_t)32 * i * F + g * G + kk) : u32x4{0, 0, 0, 0};
    }
    const uint16_t* wb = Wdp + (size_t)g * d * G + bBase + kk;
#pragma unroll
    for (int i = 0; i < C::B_CHUNKS; ++i)
      rbuf[i] = n0 + crow + 32 * i < d ? ld16(wb + (size_t)32 * i * G) : u32x4{0, 0, 0, 0};
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < C::A_CHUNKS; ++i) st16(sA + dst0 + 32 * i * kLdsLd, ra[i]);
#pragma unroll
    for (int i = 0; i < C::B_CHUNKS; ++i) st16(sB + dst0 + 32 * i * kLdsLd, rbuf[i]);
  };
  // Row blocks of this wave holding at least one token that keeps group g.
  auto live_blocks = [&](int g) {
    const uint64_t sel = 1ull << (g & 63);
    const int w = g >> 6;
    uint32_t live = 0;
#pragma unroll
    for (int i = 0; i < C::RB; ++i) {
      const int row = wm * C::WM + i * 32 + (lane & 31);
      const bool k = row < rows && (sBits[row * 4 + w] & sel);
      if (ballot(k)) live |= 1u << i;
    }
    return live;
  };

  WaveAcc<BM, BN> acc;
  acc.zero();
  if (nk > 0) {
    gload(0);
    lstore();
    __syncthreads();
  }
  uint32_t rb_live = 0;
  for (int it = 0; it < nk; ++it) {
    if (it % kpg == 0) rb_live = live_blocks(sGroups[it / kpg]);
    if (it + 1 < nk) gload(it + 1);
    acc.sweep(sA, sB, wm, wn, lane, rb_live);
    __syncthreads();
    if (it + 1 < nk) {
      lstore();
      __syncthreads();
    }
  }

  // The residual pointer passes through an empty asm here so its loads are not
  // hoisted into the K loop, where they would push accumulators out of registers.
  const uint16_t* res = residual;
  asm volatile("" : "+s"(res));
#pragma unroll
  for (int i = 0; i < C::RB; ++i)
#pragma unroll
    for (int j = 0; j < C::CB; ++j) {
      const int col = n0 + wn * C::WN + j * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = wm * C::WM + i * 32 + acc32_row(lane, e);
        if (row < rows && col < d) {
          const size_t o = (size_t)(t0 + row) * d + col;
          float v = acc.acc[i][j][e];
          if (res) v += bf2f(res[o]);
          Y[o] = f2bf(v);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
}

constexpr int kDownBM = 256, kDownBN = 256;
int ffn_down_tile_m() { return kDownBM; }

void launch_ffn_prefill(const uint16_t* X, const uint16_t* Wg, const uint16_t* Wu,
                        const uint16_t* Wdp, const ReorderView& rv, int T, int d, int F, int n,
                        const uint16_t* residual, uint16_t* H, uint16_t* Y, hipStream_t s) {
  const int G = F / n;
  const int nw = (n + 63) / 64;
  // up
  if (G % 128 == 0) {
    constexpr int BM = 256, BN = 256;
    const int mtiles = (T + BM - 1) / BM, ntn = G / (BN / 2);
    ffn_up_prefill<BM, BN><<<n * mtiles * ntn, 256, 0, s>>>(X, Wg, Wu, rv.count, rv.perm, T, d, F,
                                                             n, G, mtiles, ntn, H);
  } else {
    constexpr int BM = 256, BN = 128;
    const int mtiles = (T + BM - 1) / BM, ntn = G / (BN / 2);
    ffn_up_prefill<BM, BN><<<n * mtiles * ntn, 256, 0, s>>>(X, Wg, Wu, rv.count, rv.perm, T, d, F,
                                                             n, G, mtiles, ntn, H);
  }
  // down
  const int mtiles = (T + kDownBM - 1) / kDownBM, ntn = (d + kDownBN - 1) / kDownBN;
  ffn_down_prefill<kDownBM, kDownBN><<<mtiles * ntn, 256, 0, s>>>(
      H, Wdp, rv.packed, rv.tile_count, rv.tile_groups, T, d, F, n, G, nw, ntn, residual, Y);
}

}  // namespace wide
