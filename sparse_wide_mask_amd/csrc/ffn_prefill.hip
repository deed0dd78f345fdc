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
//      token-major [T, d_ff] at the kept blocks only.  A group's last tile of at
//      most 64 rows is done by one of the grid's last work-groups with 64-row
//      tiles and three LDS stages, on a compute unit that is done with its full
//      tiles.
// down (K-masked): one output tile = (256 consecutive tokens, 256 columns of
//      d_model); K runs over the groups that some token of the tile keeps
//      (tile_groups, l=0 for the others), G channels each.  A rows of tokens that
//      dropped the group are not loaded (zeros, l=1) and 32-row MFMA blocks with
//      no such token are skipped (l=2).  W_down is read in the packed K-major
//      group layout.
#include "common.h"
#include "gemm_tile.h"
#include "internal.h"

#include <type_traits>

namespace wide {

// Work-group id -> (group, row tile, column tile) of the up projection.  Work-groups
// are dealt to the 8 XCDs round-robin; when n_groups is a multiple of 8, XCD x
// takes the groups x, x+8, ... and walks them in 4-row-tile x 8-column blocks:
// tiles of one group share its weight rows, and the same row-tile index of
// different groups gathers tokens from the same stretch of X.
WIDE_DEV void up_tile(int bid, int n_groups, int mtiles, int ntn, int& g, int& mt, int& nt) {
  int c;
  if ((n_groups & 7) == 0) {
    const int x = bid & 7;
    block_raster(bid >> 3, mtiles, (n_groups >> 3) * ntn, 4, 8, mt, c);
    g = x + 8 * (c / ntn);
  } else {
    block_raster(bid, mtiles, n_groups * ntn, 4, 8, mt, c);
    g = c / ntn;
  }
  nt = c % ntn;
}

// A group's last row tile with at most kUpTailParts * kUpTailRows rows is left by
// the row tiles to the tail work-groups (64-row tiles, three LDS stages; a tile of
// 65-128 rows is two of them, on two compute units).  Such a tile streams all of
// the group's weight columns for few rows; as a 256-row tile it is bound by load
// latency, takes most of a full tile's time and, coming last in the raster, adds a
// round of its own (masks whose counts spread past 64 rows over a multiple of 256).
constexpr int kUpTailRows = 64;
constexpr int kUpTailParts = 2;

// One output tile of the up projection: rows row0 .. row0 + rows - 1 of group g's
// kept-token list, channel tile nt.  NSA / NSB = LDS stages of A and B (2 / 2,
// 3 / 3, or 2 / 3).  TL: the tile's token list is staged in LDS (sTok); without
// it (when the stages fill the LDS) each lane reads the tokens of its own load
// and store rows from group_perm.
template <int BM, int BN, int NWM, int NWN, int NSA, int NSB, bool TL>
WIDE_DEV void ffn_up_tile(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wg,
                          const uint16_t* __restrict__ Wu, const int32_t* __restrict__ gperm,
                          int T, int d, int F, int G, int g, int row0, int rows, int nt,
                          uint16_t* sA, uint16_t* sB, int* sTok, uint16_t* __restrict__ H) {
  using C = TileCfg<BM, BN, NWM, NWN>;
  constexpr int NW = C::kWaves;
  constexpr int BNH = BN / 2;  // channels per tile (gate and up each)
  const uint32_t ldsA = lds_addr(sA), ldsB = lds_addr(sB);

  constexpr bool kTokLds = TL;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave / NWN, wn = wave % NWN;
  const int32_t* gp = gperm + (size_t)g * T + row0;
  if constexpr (kTokLds) {
    for (int r = tid; r < BM; r += C::kThreads) sTok[r] = r < rows ? gp[r] : -1;
    __syncthreads();
  }
  auto tok = [&](int r) { return kTokLds ? sTok[r] : (r < rows ? gp[r] : -1); };

  const int chunk8 = dma_chunk(dma_row<NW>(wave, 0, lane), lane) * 8;
  const i32x4 rX = make_srd(X, (uint32_t)T * d * 2u);
  const i32x4 rG = make_srd(Wg, (uint32_t)F * d * 2u);
  const i32x4 rU = make_srd(Wu, (uint32_t)F * d * 2u);
  uint32_t aOff[C::A_INST];
#pragma unroll
  for (int q = 0; q < C::A_INST; ++q) {
    const int t = tok(dma_row<NW>(wave, q, lane));
    aOff[q] = t >= 0 ? (uint32_t)(t * d + chunk8) * 2u : kSkip;  // l=1: no load
  }
  // B row nrow: wave column nrow / WN; 32-row slabs alternate gate / up so that a
  // lane holds gate and up of the same channel.
  uint32_t bOff[C::B_INST];
  int bUp[C::B_INST];
#pragma unroll
  for (int q = 0; q < C::B_INST; ++q) {
    const int nrow = dma_row<NW>(wave, q, lane);
    const int w = nrow / C::WN, local = nrow % C::WN, blk = local >> 5;
    const int ch = nt * BNH + w * (C::WN / 2) + (blk >> 1) * 32 + (local & 31);
    bOff[q] = (uint32_t)((g * G + ch) * d + chunk8) * 2u;
    bUp[q] = __builtin_amdgcn_readfirstlane(blk & 1);
  }
  auto issueA = [&](int kt, int st) {
    const uint32_t a = ldsA + st * C::SA * 2, kb = (uint32_t)kt * kBK * 2u;
#pragma unroll
    for (int q = 0; q < C::A_INST; ++q) lds_dma16(rX, dma_dst<NW>(a, wave, q), aOff[q] + kb);
  };
  auto issueB = [&](int kt, int st) {
    const uint32_t b = ldsB + st * C::SB * 2, kb = (uint32_t)kt * kBK * 2u;
#pragma unroll
    for (int q = 0; q < C::B_INST; ++q)
      lds_dma16(bUp[q] ? rU : rG, dma_dst<NW>(b, wave, q), bOff[q] + kb);
  };
  auto issue = [&](int kt, int st) {
    issueA(kt, st);
    issueB(kt, st);
  };
  // store rows of this lane in the epilogue (below): their tokens, read now
  constexpr int HCH = C::WN / 2;  // channels of the wave
  constexpr int CPR = HCH / 8;    // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;   // rows per store instruction
  constexpr int NST = C::WM / RPI;
  int stTok[NST];
#pragma unroll
  for (int it = 0; it < NST; ++it) stTok[it] = kTokLds ? 0 : tok(wm * C::WM + it * RPI + lane / CPR);

  uint32_t rb_live = 0;
#pragma unroll
  for (int i = 0; i < C::RB; ++i)
    if (wm * C::WM + i * 32 < rows) rb_live |= 1u << i;

  WaveAcc<BM, BN, NWM, NWN> acc;
  acc.zero();
  const int nk = d / kBK;
  auto live = [&](int) { return rb_live; };
  auto run = [&](auto all_tag) {
    constexpr bool ALL = decltype(all_tag)::value;
    if constexpr (NSA == 2 && NSB == 3)
      acc.template run_a2b3<ALL, C::B_INST>(nk, sA, sB, wm, wn, lane, issueA, issueB, live);
    else if constexpr (NSA == 3)
      acc.template run3<ALL, C::LOADS>(nk, sA, sB, wm, wn, lane, issue, live);
    else
      acc.template run<ALL, C::LOADS>(nk, sA, sB, wm, wn, lane, issue, live);
  };
  if (rb_live == C::kAllRows)  // every row block of this wave holds kept rows
    run(std::true_type{});
  else  // tail tile of the group: l=2 skips the row blocks with no kept token
    run(std::false_type{});

  // epilogue: H[token, gG + ch] = silu(gate) * up.  Each wave parks its WM x WN/2
  // bf16 results in LDS (the stages are free once every wave is past its last
  // fragment read) and writes them back as 16-byte chunks of its rows, a whole
  // 128-byte line per row (64 channels) where the tile is 256 wide; one bf16 per
  // lane per store (the accumulator layout) made the epilogue cost as much as a
  // tenth of the kernel.  32-bit byte offsets into H (T F 2 < 2^31); rows past the
  // count exist only in a group's last tile and are not written.
  static_assert(NW * C::WM * HCH <= NSA * C::SA && C::WM % RPI == 0, "epilogue tile fits the stages");
  __syncthreads();
  uint16_t* sH = sA + wave * C::WM * HCH;
#pragma unroll
  for (int i = 0; i < C::RB; ++i) {
    if (!((rb_live >> i) & 1u)) continue;
#pragma unroll
    for (int jp = 0; jp < C::CB / 2; ++jp) {
      const f32x16 gt = acc.acc[i][2 * jp], up = acc.acc[i][2 * jp + 1];
#pragma unroll
      for (int e = 0; e < 16; ++e)
        sH[(i * 32 + acc32_row(lane, e)) * HCH + jp * 32 + (lane & 31)] = f2bf(silu(gt[e]) * up[e]);
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  const rsrc_t hr = make_rsrc(H, (uint32_t)((size_t)T * F * 2));
  const int chbase = g * G + nt * BNH + wn * HCH;
#pragma unroll
  for (int it = 0; it < C::WM / RPI; ++it) {
    const int r = it * RPI + lane / CPR, c = lane % CPR;
    const int row = wm * C::WM + r;
    const u32x4 v = *reinterpret_cast<const u32x4*>(sH + r * HCH + c * 8);
    const int t = kTokLds ? (row < rows ? sTok[row] : -1) : stTok[it];
    const uint32_t off = t >= 0 ? (uint32_t)(t * F + chbase + c * 8) * 2u : kSkip;
    __builtin_amdgcn_raw_buffer_store_b128(v, hr, (int)off, 0, kNtStore);
  }
}

// Tail tiles: 64 rows in a 2 x 4 wave layout (each wave still holds gate and up
// of its 32 channels), three LDS stages.
constexpr int kTailNWM = 2, kTailNWN = 4, kTailStages = 3;
using TailCfg = TileCfg<kUpTailRows, 256, kTailNWM, kTailNWN>;
static_assert(TailCfg::kThreads == kGemmThreads, "one launch shape");

// The up projection.  Work-groups below n_main take the row tiles (up_tile) but,
// when TAILS, not a group's last tile of at most kUpTailParts * kUpTailRows rows;
// the kUpTailParts * n * ntn work-groups after them take exactly those tails, one
// per (64-row part, group, channel tile), first parts first.  Being last in the
// grid, the tails run on the compute units that finish their share of full tiles
// first.
template <int BM, int BN, int NWM, int NWN, bool TAILS, bool B3>
__global__ void __launch_bounds__(kGemmThreads, 1)
    ffn_up_prefill(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wg,
                   const uint16_t* __restrict__ Wu, const int32_t* __restrict__ gcount,
                   const int32_t* __restrict__ gperm, int T, int d, int F, int n, int G,
                   int mtiles, int ntn, int n_main, uint16_t* __restrict__ H) {
  using C = TileCfg<BM, BN, NWM, NWN>;
  // LDS stages of the row tiles: three when the weight tile is at most 128 columns
  // (groups of 64 or 32 channels; at the 8B layer with groups of 64 FFN up went
  // 1137 -> 944 us), two beside 256-column weight tiles, where a third does not
  // fit.  B3: three stages of the 256-column weight tiles beside two of A, which
  // fill the LDS, so the tiles' token lists stay in registers (TL false).
  constexpr int NSA = BN <= 128 ? 3 : kStages;
  constexpr int NSB = BN <= 128 || B3 ? 3 : kStages;
  constexpr bool TL = !B3;
  constexpr int kMain = NSA * C::SA + NSB * C::SB;
  constexpr int kTail = TAILS ? kTailStages * (TailCfg::SA + TailCfg::SB) : 0;
  constexpr int kStg = kMain > kTail ? kMain : kTail;
  __shared__ __attribute__((aligned(16))) uint16_t sbuf[kStg + (TL ? 2 * BM : 0)];
  int* sTok = reinterpret_cast<int*>(sbuf + kStg);  // the token list (TL only)
  if (TAILS && (int)blockIdx.x >= n_main) {
    const int id = blockIdx.x - n_main, per = n * ntn;
    const int part = id / per, g = (id % per) / ntn, nt = id % ntn;
    const int cnt = gcount[g];
    if (cnt == 0) return;
    const int last = (cnt - 1) / BM * BM;  // the group's last row tile
    if (cnt - last > kUpTailParts * kUpTailRows) return;  // a row tile like the others
    const int row0 = last + part * kUpTailRows;
    if (row0 >= cnt) return;
    ffn_up_tile<kUpTailRows, 256, kTailNWM, kTailNWN, kTailStages, kTailStages, TL>(
        X, Wg, Wu, gperm, T, d, F, G, g, row0, min(kUpTailRows, cnt - row0), nt, sbuf,
        sbuf + kTailStages * TailCfg::SA, sTok, H);
    return;
  }
  int g, mt, nt;
  up_tile(blockIdx.x, n, mtiles, ntn, g, mt, nt);
  const int cnt = gcount[g];
  const int row0 = mt * BM;
  if (row0 >= cnt) return;  // l=0: no kept token left in this tile
  const int rows = min(BM, cnt - row0);
  if (TAILS && row0 + BM >= cnt && rows <= kUpTailParts * kUpTailRows) return;  // the tails
  ffn_up_tile<BM, BN, NWM, NWN, NSA, NSB, TL>(X, Wg, Wu, gperm, T, d, F, G, g, row0, rows, nt,
                                               sbuf, sbuf + NSA * C::SA, sTok, H);
}

// GPS = groups per 64-wide K slice: 1 for groups of 64 or more channels; 2 for
// groups of 32, where a slice covers groups 2p and 2p + 1 (K runs over the tile's
// union of such pairs; each lane's 16-byte chunk belongs to one of the two
// groups, which decides its row's keep bit and its weight block).
template <int BM, int BN, int USE, int GPS>
__global__ void __launch_bounds__(kGemmThreads, 1)
    kmask_gemm_prefill(const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wdp,
                       const uint64_t* __restrict__ packed, const int32_t* __restrict__ tcount,
                       const int32_t* __restrict__ tgroups, const int32_t* __restrict__ order,
                       const int32_t* __restrict__ tile_perm, int T, int d, int F, int n, int G,
                       int nw, int ntn,
                       const uint16_t* __restrict__ residual, uint16_t* __restrict__ Y) {
  using C = TileCfg<BM, BN>;
  // LDS stages: a third fits beside 128-column B tiles (144 KB of stages; 2048-token
  // 8B attention output projection 65.3 -> 62.0 us), not beside wider ones
  constexpr int NS = BN <= 128 ? 3 : kStages;
  __shared__ __attribute__((aligned(16))) uint16_t sA[NS * C::SA];
  __shared__ __attribute__((aligned(16))) uint16_t sB[NS * C::SB];
  const uint32_t ldsA = lds_addr(sA), ldsB = lds_addr(sB);
  __shared__ uint64_t sBits[BM * 4];
  __shared__ int sTok[BM];  // token of each tile row
  __shared__ int sGroups[256];
  __shared__ uint8_t sLive[256 * C::kWaves];
  __shared__ int sNsg;

  // XCD x takes a contiguous stretch of the block-rasterised tile order.
  const int mtiles = (T + BM - 1) / BM, n_tiles = mtiles * ntn;
  const int p = (blockIdx.x & 7) * ((n_tiles + 7) >> 3) + (blockIdx.x >> 3);
  if (p >= n_tiles) return;
  int mt, nt;
  if (tile_perm) {
    // row tiles balanced over the XCDs by group union, each XCD's in descending
    // union order; walked row by row, so a compute unit that ran a large tile
    // early takes a small one late
    mt = tile_perm[p / ntn];
    nt = p % ntn;
  } else {
    block_raster(p, mtiles, ntn, 4, 8, mt, nt);
  }
  const int t0 = mt * BM, rows = min(BM, T - t0), n0 = nt * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave / kGemmWN, wn = wave % kGemmWN;
  // tgroups null: the tile's union is the OR of its rows' mask words (tokens in a
  // pattern order whose key ranges do not give the unions)
  __shared__ uint32_t sU32[8];
  __shared__ int sNg;
  int ng = tgroups ? tcount[mt] : 0;
  // tile rows are tokens t0.. in order, or order[t0..] (tokens sorted by mask
  // pattern, so row blocks share dropped groups)
  for (int i = tid; i < BM; i += C::kThreads)
    sTok[i] = i < rows ? (order ? order[t0 + i] : t0 + i) : 0;
  if (tid < 8) sU32[tid] = 0u;
  __syncthreads();
  for (int i = tid; i < BM * nw; i += C::kThreads) {
    const int r = i / nw, w = i % nw;
    sBits[r * 4 + w] = r < rows ? packed[(size_t)sTok[r] * nw + w] : 0ull;
  }
  if (tgroups) {
    for (int i = tid; i < ng; i += C::kThreads) sGroups[i] = tgroups[(size_t)mt * n + i];
    __syncthreads();
  } else {
    __syncthreads();
    for (int w = 0; w < nw; ++w) {
      uint64_t v = 0;
      for (int r = tid; r < rows; r += C::kThreads) v |= sBits[r * 4 + w];
      uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
      for (int off = 32; off >= 1; off >>= 1) lo |= __shfl_xor(lo, off), hi |= __shfl_xor(hi, off);
      if (lane == 0) {
        if (lo) atomicOr(&sU32[2 * w], lo);
        if (hi) atomicOr(&sU32[2 * w + 1], hi);
      }
    }
    __syncthreads();
    if (wave == 0) {  // ascending group list
      int written = 0;
      for (int w = 0; w < nw; ++w) {
        const uint64_t u = ((uint64_t)sU32[2 * w + 1] << 32) | sU32[2 * w];
        if ((u >> lane) & 1ull) sGroups[written + popc64(u & ((1ull << lane) - 1ull))] = 64 * w + lane;
        written += popc64(u);
      }
      if (lane == 0) sNg = written;
    }
    __syncthreads();
    ng = sNg;
  }
  int nsg = ng;  // the tile's K units: groups, or pairs of groups when GPS == 2
  if constexpr (GPS == 2) {
    if (tid == 0) {  // ascending groups -> ascending distinct pairs, in place
      int m = 0;
      for (int i = 0; i < ng; ++i) {
        const int pr = sGroups[i] >> 1;
        if (m == 0 || sGroups[m - 1] != pr) sGroups[m++] = pr;
      }
      sNsg = m;
    }
    __syncthreads();
    nsg = sNsg;
  }

  const int chunk8 = dma_chunk(dma_row(wave, 0, lane), lane) * 8;
  const i32x4 rH = make_srd(H, (uint32_t)T * F * 2u);
  const i32x4 rW = make_srd(Wdp, (uint32_t)F * d * 2u);
  int aRow[C::A_INST];
  uint32_t aBase[C::A_INST], bOff[C::B_INST];
#pragma unroll
  for (int q = 0; q < C::A_INST; ++q) {
    aRow[q] = dma_row(wave, q, lane);
    aBase[q] = (uint32_t)(sTok[aRow[q]] * F + chunk8) * 2u;
  }
  // GPS == 2: this lane's chunk lies in the pair's second group when chunk8 >= 32
  const int half_l = GPS == 2 && chunk8 >= 32 ? 1 : 0;
#pragma unroll
  for (int q = 0; q < C::B_INST; ++q) {
    const int nrow = n0 + dma_row(wave, q, lane);
    const uint32_t o = GPS == 2 ? (uint32_t)(nrow * G + (chunk8 & 31)) * 2u
                                : (uint32_t)(nrow * G + chunk8) * 2u;
    bOff[q] = nrow < d ? o : kSkip;
  }
  const int kpg = GPS == 2 ? 1 : G / kBK;  // K slices per K unit
  const int nk = nsg * kpg;
  // The issues walk the slices in order, so the slice's group comes from running
  // counters; the next group is read from LDS one call ahead, and each lane keeps
  // the mask word of its A rows that holds the current group's bit (reloaded
  // only when the group crosses a 64-group word).
  int is_gi = 0, is_s = 0, is_w = -1;
  int is_gv = nsg > 0 ? sGroups[0] : 0;  // read ahead; made scalar when used
  uint64_t rw[C::A_INST];
  auto issue = [&](int, int st) {
    const int g = __builtin_amdgcn_readfirstlane(is_gv);  // group, or pair (GPS == 2)
    const int g0 = GPS * g;  // first group of the slice
    if ((g0 >> 6) != is_w) {
      is_w = g0 >> 6;
#pragma unroll
      for (int q = 0; q < C::A_INST; ++q)
        rw[q] = aRow[q] < rows ? sBits[aRow[q] * 4 + is_w] : 0ull;
    }
    const uint32_t a = ldsA + st * C::SA * 2, b = ldsB + st * C::SB * 2;
    const int kk = is_s * kBK;
    // this lane's group: the slice's, or its chunk's of the pair
    const int gl = g0 + half_l;
    const uint32_t ka = (uint32_t)(g0 * G + kk) * 2u;
#pragma unroll
    for (int q = 0; q < C::A_INST; ++q) {
      // l=1: rows of tokens that dropped the group (or past T) are not fetched (zeros)
      const bool keep = (rw[q] >> (gl & 63)) & 1ull;
      lds_dma16(rH, dma_dst(a, wave, q), keep ? aBase[q] + ka : kSkip);
    }
    const uint32_t kb = (uint32_t)(gl * d * G + kk) * 2u;
#pragma unroll
    for (int q = 0; q < C::B_INST; ++q)
      lds_dma16(rW, dma_dst(b, wave, q), bOff[q] == kSkip ? kSkip : bOff[q] + kb);
    if (++is_s == kpg) {
      is_s = 0;
      if (++is_gi < nsg) is_gv = sGroups[is_gi];
    }
  };
  // l=2: per K unit of the tile, the row blocks of each wave that hold at least one
  // token keeping it (either group of a pair; sLive[unit index][wave]); a wave
  // whose blocks are all live for every unit runs the branch-free loop.
  bool all_live = true;
  for (int gi = 0; gi < nsg; ++gi) {
    const int g0 = GPS * sGroups[gi];
    const uint64_t sel = (GPS == 2 ? 3ull : 1ull) << (g0 & 63);
    const int w = g0 >> 6;
    uint32_t live = 0;
#pragma unroll
    for (int i = 0; i < C::RB; ++i) {
      const int row = wm * C::WM + i * 32 + (lane & 31);
      const bool k = row < rows && (sBits[row * 4 + w] & sel);
      if (ballot(k)) live |= 1u << i;
    }
    if (lane == 0) sLive[gi * C::kWaves + wave] = (uint8_t)live;
    all_live = all_live && live == C::kAllRows;
  }
  __syncthreads();

  WaveAcc<BM, BN> acc;
  acc.zero();
  if (all_live) {
    if constexpr (NS == 3)
      acc.template run3<true, C::LOADS>(nk, sA, sB, wm, wn, lane, issue, [](int) { return 0u; });
    else
      acc.template run<true, C::LOADS>(nk, sA, sB, wm, wn, lane, issue, [](int) { return 0u; });
  } else {
    // live row blocks of the slices in order, the next group's read one call ahead
    int lv_gi = 0, lv_s = 0;
    uint32_t lv = nsg > 0 ? sLive[wave] : 0u;
    auto live_rows = [&](int) {
      const uint32_t v = lv;
      if (++lv_s == kpg) {
        lv_s = 0;
        if (++lv_gi < nsg) lv = sLive[lv_gi * C::kWaves + wave];
      }
      return v;
    };
    if constexpr (NS == 3)
      acc.template run3<false, C::LOADS>(nk, sA, sB, wm, wn, lane, issue, live_rows);
    else
      acc.template run<false, C::LOADS>(nk, sA, sB, wm, wn, lane, issue, live_rows);
  }

  // Epilogue: Y[token, col] = acc (+ residual).  Each wave parks one 32-row block
  // of its fp32 accumulators in LDS at a time (waves 0-3 in the A stages, 4-7 in
  // the B stages, free once every wave is past its last fragment read) and moves
  // it as 8-column chunks: one 16-byte residual load and one 16-byte store per
  // lane, the residual loads of the block issued before the first store (Y may
  // alias the residual: a lane reads its chunk before it writes it).  Rows past
  // the tile's tokens and columns past d take the kSkip offset, so their loads
  // read 0 and their stores are dropped; without a residual the descriptor has no
  // records and every load reads 0.  32-bit byte offsets (T d 2 < 2^31).  The
  // residual pointer passes through an empty asm so the loads are not scheduled
  // into the K loop.
  constexpr int CPR = C::WN / 8;        // 8-column chunks per row of the wave
  constexpr int NIT = 32 * CPR / 64;    // instructions per 32-row block: lane l of
  static_assert(32 * CPR % 64 == 0, "");  // instruction it takes chunk 64 it + l
  constexpr int kHalfWaves = C::kWaves / 2;
  static_assert(kHalfWaves * 32 * C::WN * 4 <= NS * C::SA * 2 &&
                    kHalfWaves * 32 * C::WN * 4 <= NS * C::SB * 2,
                "epilogue blocks fit the stages");
  __syncthreads();
  float* sY = reinterpret_cast<float*>(wave < kHalfWaves ? sA : sB) +
              (wave % kHalfWaves) * 32 * C::WN;
  const uint16_t* res = residual;
  asm volatile("" : "+s"(res));
  const rsrc_t yr = make_rsrc(Y, (uint32_t)((size_t)T * d * 2));
  const rsrc_t rr = make_rsrc(res, res ? (uint32_t)((size_t)T * d * 2) : 0u);
#pragma unroll
  for (int i = 0; i < C::RB; ++i) {
#pragma unroll
    for (int j = 0; j < C::CB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        sY[acc32_row(lane, e) * C::WN + j * 32 + (lane & 31)] = acc.acc[i][j][e];
    uint32_t off[NIT];
    u32x4 rv[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int r = (it * 64 + lane) / CPR, c = (it * 64 + lane) % CPR;
      const int row = wm * C::WM + i * 32 + r, col = n0 + wn * C::WN + c * 8;
      off[it] = row < rows && col < d ? (uint32_t)(sTok[row] * d + col) * 2u : kSkip;
      rv[it] = ldbuf16(rr, off[it]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int r = (it * 64 + lane) / CPR, c = (it * 64 + lane) % CPR;
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(sY + r * C::WN + c * 8);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(sY + r * C::WN + c * 8 + 4);
      const u32x4 q = rv[it];
      u32x4 o;
      o[0] = pack_bf2(a0[0] + __uint_as_float(q[0] << 16), a0[1] + __uint_as_float(q[0] & 0xffff0000u));
      o[1] = pack_bf2(a0[2] + __uint_as_float(q[1] << 16), a0[3] + __uint_as_float(q[1] & 0xffff0000u));
      o[2] = pack_bf2(a1[0] + __uint_as_float(q[2] << 16), a1[1] + __uint_as_float(q[2] & 0xffff0000u));
      o[3] = pack_bf2(a1[2] + __uint_as_float(q[3] << 16), a1[3] + __uint_as_float(q[3] & 0xffff0000u));
      __builtin_amdgcn_raw_buffer_store_b128(o, yr, (int)off[it], 0, kNtStore);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();  // the block's reads before the next block's writes
  }
}

constexpr int kDownBM = 256;
int ffn_down_tile_m() { return kDownBM; }

// K-masked GEMM Y[t] = sum over groups g kept by t of A[t, gG:(g+1)G] Wp[g]^T
// (+ residual), A token-major [T, F], Wp packed [n, d, G].  The column tile (256,
// 192 or 128 columns) is chosen to fill the 256 CUs best (rounds x tile width; the
// wider tile on a tie): at d = 3072 and 4096 tokens, 192 columns make exactly 256
// tiles where 256 columns leave a quarter of the CUs idle.  The trace labels the
// launch as FFN down or attention output projection.
template <int USE>
void launch_kmask_gemm_as(const uint16_t* A, const uint16_t* Wp, const ReorderView& rv, int T,
                          int d, int F, int n, const uint16_t* residual, uint16_t* Y,
                          hipStream_t s) {
  const int G = F / n;
  const int nw = (n + 63) / 64;
  const int mtiles = (T + kDownBM - 1) / kDownBM;
  int best_bn = 256;
  long best_cost = -1;
  for (int bn : {256, 192, 128}) {
    const long tiles = (long)mtiles * ((d + bn - 1) / bn);
    const long cost = ((tiles + 255) / 256) * bn;
    if (best_cost < 0 || cost < best_cost) best_cost = cost, best_bn = bn;
  }
  const int ntn = (d + best_bn - 1) / best_bn;
  const int grid = 8 * ((mtiles * ntn + 7) / 8);
  WIDE_TRACE(USE == kUseAttnO ? "attn_o" : "ffn_down", s);
  auto pick = [&](auto gps_tag) {
    constexpr int P = decltype(gps_tag)::value;
    return best_bn == 256   ? kmask_gemm_prefill<kDownBM, 256, USE, P>
           : best_bn == 192 ? kmask_gemm_prefill<kDownBM, 192, USE, P>
                            : kmask_gemm_prefill<kDownBM, 128, USE, P>;
  };
  using G1 = std::integral_constant<int, 1>;
  using G2 = std::integral_constant<int, 2>;
  auto k = pick(G1{});
  if constexpr (USE == kUseFfnDown)
    if (G % 64 != 0) k = pick(G2{});  // groups of 32: pairs per slice
  k<<<grid, kGemmThreads, 0, s>>>(A, Wp, rv.packed, rv.tile_count, rv.tile_groups, rv.order,
                                  rv.tile_perm, T, d, F, n, G, nw, ntn, residual, Y);
}

void launch_kmask_gemm(KmUse use, const uint16_t* A, const uint16_t* Wp, const ReorderView& rv,
                       int T, int d, int F, int n, const uint16_t* residual, uint16_t* Y,
                       hipStream_t s) {
  if (use == kUseAttnO)
    launch_kmask_gemm_as<kUseAttnO>(A, Wp, rv, T, d, F, n, residual, Y, s);
  else
    launch_kmask_gemm_as<kUseFfnDown>(A, Wp, rv, T, d, F, n, residual, Y, s);
}

void launch_ffn_prefill(const uint16_t* X, const uint16_t* Wg, const uint16_t* Wu,
                        const uint16_t* Wdp, const ReorderView& rv, int T, int d, int F, int n,
                        const uint16_t* residual, uint16_t* H, uint16_t* Y, hipStream_t s) {
  const int G = F / n;
  // up
  if (G % 128 == 0) {
    constexpr int BM = 256, BN = 256;
    const int mtiles = (T + BM - 1) / BM, ntn = G / (BN / 2);
    {
      WIDE_TRACE("ffn_up_prefill", s);
      const int n_main = n * mtiles * ntn;
      ffn_up_prefill<BM, BN, kGemmWM, kGemmWN, true, true>
          <<<n_main + kUpTailParts * n * ntn, kGemmThreads, 0, s>>>(
          X, Wg, Wu, rv.count, rv.perm, T, d, F, n, G, mtiles, ntn, n_main, H);
    }
  } else if (G % 64 == 0) {
    constexpr int BM = 256, BN = 128;
    const int mtiles = (T + BM - 1) / BM, ntn = G / (BN / 2);
    {
      WIDE_TRACE("ffn_up_prefill", s);
      const int n_main = n * mtiles * ntn;
      ffn_up_prefill<BM, BN, kGemmWM, kGemmWN, false, false><<<n_main, kGemmThreads, 0, s>>>(
          X, Wg, Wu, rv.count, rv.perm, T, d, F, n, G, mtiles, ntn, n_main, H);
    }
  } else {
    // groups of 32 channels: 64-column tiles (32 gate + 32 up), eight waves of
    // 32 rows, each holding gate and up of the tile's 32 channels
    constexpr int BM = 256, BN = 64;
    const int mtiles = (T + BM - 1) / BM, ntn = G / (BN / 2);
    {
      WIDE_TRACE("ffn_up_prefill", s);
      const int n_main = n * mtiles * ntn;
      ffn_up_prefill<BM, BN, 8, 1, false, false><<<n_main, kGemmThreads, 0, s>>>(
          X, Wg, Wu, rv.count, rv.perm, T, d, F, n, G, mtiles, ntn, n_main, H);
    }
  }
  launch_kmask_gemm(kUseFfnDown, H, Wdp, rv, T, d, F, n, residual, Y, s);
}

}  // namespace wide
