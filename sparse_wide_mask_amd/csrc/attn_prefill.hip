// Masked attention sublayer, prefill (gist.science technical summary §2.A: head
// groups aligned with GQA; §2.B reordering; §2.C skipping).
//
// Group g = KV head g with its r query heads.  After the reordering, the kept
// tokens of g form the prefix group_perm[g, 0:count) in ascending token order,
// so attention "over kept groups only" is ordinary causal attention over that
// compacted sequence (a kept token sees the earlier tokens that also kept g).
//
// attn_qkv_prefill  N-masked GEMM over the compacted rows of each group; tile =
//                   (group, 256 kept tokens, 256 of the group's 768 output
//                   columns: q heads 0-1 | q heads 2-3 | k,v).  Each wave holds
//                   one 128-wide head, so the RoPE pair (j, j+64) sits in the same
//                   lane; rotation uses the token's original position.  Writes
//                   Qc [n_kv][r][T][hd], Kc [n_kv][T][hd] and V transposed,
//                   Vt [n_kv][hd][vtp] (column i = i-th kept token of the group,
//                   permuted inside 16-key groups; zero up to a whole group).
// attn_core_prefill one work-group = (group, one of B bins of its tiles of 32
//                   compacted queries, dealt heaviest first in snake order),
//                   one wave per query head; two work-groups per CU, whose
//                   waves share the SIMDs without sharing barriers.  K and V^T
//                   blocks arrive by buffer->LDS loads one key step ahead.
//                   S^T = K Q^T puts a query in each lane's column, so the
//                   softmax is per lane (+ one cross-half swap,
//                   v_permlane32_swap) and P stays in registers as the B
//                   operand of O^T = V^T P^T; V is
//                   read in the key order the S^T accumulator layout gives.  A
//                   row's reference max is fixed by its first keys, so O is never
//                   rescaled in the key loop; a tile in which some row's scores
//                   outgrow it by the headroom is recomputed once with the true
//                   row maxima.
//                   Output O is written token-major [T, n_q*hd] at the kept
//                   (token, group) blocks only.
// The O projection is the K-masked GEMM of the FFN down projection with group
// depth r*hd (see ffn_prefill.hip).
#include "common.h"
#include "gemm_tile.h"
#include "internal.h"

#include <algorithm>

namespace wide {

constexpr int kHd = 128;

// ------------------------------------------------------------- QKV projection

// A RoPE frequency (radians per position) as revolutions per position, split so
// that the angle of any position below 2^16 reduces exactly: hi keeps 8
// significant bits (pos * hi is exact in fp32), lo the rest (its product is
// small).  sin and cos of the reduced angle come from v_sin/v_cos, which take
// revolutions.  Angle error ~1e-5 rad up to position 65535 (sincosf on the raw
// fp32 angle costs ~170 instructions per call through its large-argument path).
struct RopeFreq {
  float hi, lo;
  WIDE_DEV explicit RopeFreq(float inv) {
    const double rev = (double)inv * 0.15915494309189535;  // 1 / (2 pi)
    hi = __uint_as_float(__float_as_uint((float)rev) & 0xffff0000u);
    lo = (float)(rev - (double)hi);
  }
  WIDE_DEV void sincos(int pos, float& sn, float& cs) const {
    const float p = (float)pos;
    float t = p * hi;
    t = (t - floorf(t)) + p * lo;
    t -= floorf(t);
    sn = __builtin_amdgcn_sinf(t);
    cs = __builtin_amdgcn_cosf(t);
  }
};

// One tile of the QKV projection: rows row0 .. row0 + rows - 1 of group g's
// kept-token list (at most 256), and BN / 128 heads of the 256-column tile nt of
// the group's (q heads | k, v) columns, starting at head hsel0 of that tile.  NS
// LDS stages: 2 for the two-head units, 3 for the one-head halves, whose smaller
// weight stages leave room for a third (2048-token 8B attention, where every unit
// is split: QKV 66.1 -> 60.1 us).
// Waves: 256 / (8 / NWN) rows x one 128-column head each, so the RoPE pair
// (j, j + 64) of a head sits in one lane.
template <int BN, int NWN, int NS>
WIDE_DEV void qkv_tile(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wq,
                       const uint16_t* __restrict__ Wk, const uint16_t* __restrict__ Wv,
                       const int32_t* __restrict__ gperm, int T, int d, int n_kv, int r, int g,
                       int row0, int rows, int nt, int hsel0, int vtp, float log2_theta,
                       uint16_t* sA, uint16_t* sB, int* sTok, uint16_t* __restrict__ Qc,
                       uint16_t* __restrict__ Kc, uint16_t* __restrict__ Vt) {
  constexpr int BM = 256, NWM = 8 / NWN;
  using C = TileCfg<BM, BN, NWM, NWN>;
  static_assert(C::WN == kHd, "one head per wave column");
  const uint32_t ldsA = lds_addr(sA), ldsB = lds_addr(sB);
  const int ntn = (r + 1) / 2 + 1;  // q tiles (2 heads each) + one k|v tile
  const bool kv_tile = nt == ntn - 1;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave / NWN, wn = wave % NWN;
  for (int i = tid; i < BM; i += C::kThreads) sTok[i] = i < rows ? gperm[(size_t)g * T + row0 + i] : -1;
  __syncthreads();

  const int chunk8 = dma_chunk(dma_row(wave, 0, lane), lane) * 8;
  const int nq = n_kv * r;
  const i32x4 rX = make_srd(X, (uint32_t)T * d * 2u);
  const i32x4 rQ = make_srd(Wq, (uint32_t)nq * kHd * d * 2u);
  const i32x4 rK = make_srd(Wk, (uint32_t)n_kv * kHd * d * 2u);
  const i32x4 rV = make_srd(Wv, (uint32_t)n_kv * kHd * d * 2u);
  uint32_t aOff[C::A_INST];
#pragma unroll
  for (int q = 0; q < C::A_INST; ++q) {
    const int tok = sTok[dma_row(wave, q, lane)];
    aOff[q] = tok >= 0 ? (uint32_t)(tok * d + chunk8) * 2u : kSkip;
  }
  // B row of the tile: head hh = hsel0 + row / 128 of tile nt; q tile -> Wq row
  // g*r*hd + (2 nt + hh)*hd + row % 128; k|v tile -> Wk (hh = 0) or Wv (hh = 1)
  // row g*hd + row % 128.  An instruction's 64 rows lie in one head.
  uint32_t bOff[C::B_INST];
  int bV[C::B_INST];
#pragma unroll
  for (int q = 0; q < C::B_INST; ++q) {
    const int row = dma_row(wave, q, lane);
    const int hh = hsel0 + row / kHd, rr = row & (kHd - 1);
    const int wrow = kv_tile ? g * kHd + rr : g * r * kHd + (2 * nt + hh) * kHd + rr;
    bOff[q] = (uint32_t)(wrow * d + chunk8) * 2u;
    bV[q] = __builtin_amdgcn_readfirstlane(hh);
  }
  auto issue = [&](int kt, int st) {
    const uint32_t a = ldsA + st * C::SA * 2, b = ldsB + st * C::SB * 2;
    const uint32_t kb = (uint32_t)kt * kBK * 2u;
#pragma unroll
    for (int q = 0; q < C::A_INST; ++q) lds_dma16(rX, dma_dst(a, wave, q), aOff[q] + kb);
    if (kv_tile) {
#pragma unroll
      for (int q = 0; q < C::B_INST; ++q)
        lds_dma16(bV[q] ? rV : rK, dma_dst(b, wave, q), bOff[q] + kb);
    } else {
#pragma unroll
      for (int q = 0; q < C::B_INST; ++q) lds_dma16(rQ, dma_dst(b, wave, q), bOff[q] + kb);
    }
  };
  uint32_t rb_live = 0;
#pragma unroll
  for (int i = 0; i < C::RB; ++i)
    if (wm * C::WM + i * 32 < rows) rb_live |= 1u << i;

  WaveAcc<BM, BN, NWM, NWN> acc;
  acc.zero();
  const int nk = d / kBK;
  auto live = [&](int) { return rb_live; };
  if constexpr (NS == 3) {
    if (rb_live == C::kAllRows)
      acc.template run3<true, C::LOADS>(nk, sA, sB, wm, wn, lane, issue, live);
    else
      acc.template run3<false, C::LOADS>(nk, sA, sB, wm, wn, lane, issue, live);
  } else {
    if (rb_live == C::kAllRows)
      acc.template run<true, C::LOADS>(nk, sA, sB, wm, wn, lane, issue, live);
    else
      acc.template run<false, C::LOADS>(nk, sA, sB, wm, wn, lane, issue, live);
  }

  // epilogue.  This wave's 128 columns are one head, hsel = hsel0 + wn of the
  // tile: q head 2*nt + hsel, or k / v.  (With an odd head ratio the last q
  // tile's second head reads zeros or the next group's rows and is not written.)
  // Every wave is past its last fragment read here, so the stages are free for
  // the q / k rows' staging below.
  __syncthreads();
  const int hsel = hsel0 + wn;
  if (!kv_tile && 2 * nt + hsel >= r) return;
  const bool is_v = kv_tile && hsel == 1;
  const bool rope = log2_theta > 0.f && !is_v;
  const int c0 = lane & 31;
  // theta^(-2j/hd) for j = c0 and c0 + 32, in revolutions per position
  const RopeFreq f0 = rope ? RopeFreq(exp2f(-(2.f * c0 / kHd) * log2_theta)) : RopeFreq(0.f);
  const RopeFreq f1 =
      rope ? RopeFreq(exp2f(-(2.f * (c0 + 32) / kHd) * log2_theta)) : RopeFreq(0.f);
  // this wave's staging rows: WM x 128 bf16, in the A stages (and the B stages
  // for the upper half of the waves when the A stages cannot hold them all)
  constexpr int kRegion = C::WM * kHd;
  constexpr bool kSplit = C::kWaves * kRegion > NS * C::SA;
  static_assert(!kSplit || (C::kWaves / 2 * kRegion <= NS * C::SA &&
                            C::kWaves / 2 * kRegion <= NS * C::SB),
                "q / k staging fits the stages");
  uint16_t* const sQK = kSplit ? (wave < C::kWaves / 2 ? sA : sB) + (wave % (C::kWaves / 2)) * kRegion
                               : sA + wave * kRegion;
  uint16_t* qdst = Qc + ((size_t)(g * r + 2 * nt + hsel) * T) * kHd;
  uint16_t* kdst = Kc + (size_t)g * T * kHd;
  uint16_t* vdst = Vt + (size_t)g * kHd * vtp;
#pragma unroll
  for (int i = 0; i < C::RB; ++i) {
    if (!((rb_live >> i) & 1u)) continue;
    if (is_v) {
      // V^T: lane holds hd column cb*32 + c0 and rows 4 (l/32) + 8 q + {0..3}.
      // Keys are stored permuted inside 16-key groups (4-key quarter q -> slot
      // [0, 2, 1, 3][q]) so that the attention core reads a lane's 8 keys as one
      // 16-byte chunk.  Rows past the count hold zeros (their A rows were not
      // loaded), and are written up to a whole 16-key group.
      const int rows16 = (rows + 15) & ~15;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int rr = wm * C::WM + i * 32 + 8 * q4 + 4 * (lane >> 5);
          if (rr >= rows16) continue;
          const f32x16& a = acc.acc[i][cb];
          const uint32_t lo = pack_bf2(a[4 * q4], a[4 * q4 + 1]);
          const uint32_t hi = pack_bf2(a[4 * q4 + 2], a[4 * q4 + 3]);
          const int key = row0 + rr, qtr = (key >> 2) & 3;
          const int slot = (key & ~15) | ((((qtr & 1) << 1) | (qtr >> 1)) << 2);
          *reinterpret_cast<u32x2*>(vdst + (size_t)(cb * 32 + c0) * vtp + slot) = u32x2{lo, hi};
        }
      continue;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = wm * C::WM + i * 32 + acc32_row(lane, e);
      if (row >= rows) continue;
      float v0 = acc.acc[i][0][e], v1 = acc.acc[i][1][e];
      float v2 = acc.acc[i][2][e], v3 = acc.acc[i][3][e];
      if (rope) {
        const int pos = sTok[row];
        float s0, co0, s1, co1;
        f0.sincos(pos, s0, co0);
        f1.sincos(pos, s1, co1);
        const float r0 = v0 * co0 - v2 * s0, r2 = v2 * co0 + v0 * s0;
        const float r1 = v1 * co1 - v3 * s1, r3 = v3 * co1 + v1 * s1;
        v0 = r0, v1 = r1, v2 = r2, v3 = r3;
      }
      uint16_t* p = sQK + (i * 32 + acc32_row(lane, e)) * kHd + c0;
      p[0] = f2bf(v0);
      p[32] = f2bf(v1);
      p[64] = f2bf(v2);
      p[96] = f2bf(v3);
    }
  }
  if (is_v) return;
  // q / k: the wave's rows are consecutive rows of the group's compacted list,
  // 256 bytes each, so they leave LDS as 16-byte chunks of one contiguous block
  // (one bf16 per lane per store, the accumulator layout, cost about as much as
  // the kernel's last K slices)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  uint16_t* dst = (kv_tile ? kdst : qdst) + (size_t)(row0 + wm * C::WM) * kHd;
#pragma unroll
  for (int it = 0; it < C::WM / 4; ++it) {
    const int rr = it * 4 + (lane >> 4), c = lane & 15;
    if (wm * C::WM + rr < rows)
      *reinterpret_cast<u32x4*>(dst + (size_t)rr * kHd + c * 8) =
          *reinterpret_cast<const u32x4*>(sQK + rr * kHd + c * 8);
  }
}


constexpr int kCoreCUs = 256;   // compute units of the chip

// The QKV projection.  A group's tiles are units of 256 kept tokens x 256
// columns (two heads), U = ceil(count / 256) * ntn of them, dealt in row-major
// order; P = compute units per group.  The units past the last full round of P,
// rem = U mod P, are split into two one-head tiles each (256 x 128, eight waves
// of 32 rows, three LDS stages) when the 2 rem halves fit in one round: they then
// take about half a unit's time instead of a whole second round of units.  The
// halves come after all full units of every group in the grid.
__global__ void __launch_bounds__(kGemmThreads, 1)
    attn_qkv_prefill(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wq,
                     const uint16_t* __restrict__ Wk, const uint16_t* __restrict__ Wv,
                     const int32_t* __restrict__ gcount, const int32_t* __restrict__ gperm, int T,
                     int d, int n_kv, int r, int P, bool lanes, int vtp, float log2_theta,
                     uint16_t* __restrict__ Qc, uint16_t* __restrict__ Kc,
                     uint16_t* __restrict__ Vt) {
  using Big = TileCfg<256, 256>;
  using Half = TileCfg<256, 128, 8, 1>;
  constexpr int kBig = kStages * (Big::SA + Big::SB), kHalf = 3 * (Half::SA + Half::SB);
  __shared__ __attribute__((aligned(16))) uint16_t sbuf[kBig > kHalf ? kBig : kHalf];
  __shared__ int sTok[256];
  const int ntn = (r + 1) / 2 + 1;
  // Compute-unit lanes: lane l = 32 x + c is CU slot c of XCD x; work-group b runs
  // in lane 32 (b mod 8) + (b / 8) mod 32, round (b / 8) / 32.  The 256 lanes are
  // shared out among the groups by their units (each group with units keeps at
  // least one; near-equal unit counts get P = 256 / n_kv lanes each), as
  // contiguous lane ranges, so a group's weights and rows stay in one or few XCDs'
  // L2.  Work-group (lane, round) of group g takes its sequence index w = round *
  // P_g + (lane - first lane of g).
  __shared__ int sLane[3];  // group, its lanes P, the sequence index (-1: no group)
  if (!lanes) {  // many groups: group b mod n_kv, P lanes each
    if (threadIdx.x == 0) {
      sLane[0] = blockIdx.x % n_kv;
      sLane[1] = P;
      sLane[2] = blockIdx.x / n_kv;
    }
  } else if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int b = blockIdx.x, s = b >> 3;
    const int ln = 32 * (b & 7) + (s & 31), round = s >> 5;
    int tot = 0, umax = 0;
    for (int g0 = 0; g0 < n_kv; g0 += 64) {
      const int g = g0 + lane;
      const int u = g < n_kv ? ntn * ((gcount[g] + 255) / 256) : 0;
      int sum = u, mx = u;
      for (int off = 32; off >= 1; off >>= 1) {
        sum += __shfl_xor(sum, off);
        mx = max(mx, __shfl_xor(mx, off));
      }
      tot += sum;
      umax = max(umax, mx);
    }
    const bool equal = 4 * umax * n_kv <= 5 * tot;  // every group within 25 % of the mean
    if (lane == 0) sLane[0] = -1;
    int base = 0;
    for (int g0 = 0; g0 < n_kv && tot > 0; g0 += 64) {
      const int g = g0 + lane;
      int pl = 0;
      if (g < n_kv) {
        const int u = ntn * ((gcount[g] + 255) / 256);
        pl = equal ? P : (u > 0 ? 1 + (int)((long long)(kCoreCUs - n_kv) * u / tot) : 0);
      }
      int incl = pl;
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      const int start = base + incl - pl;
      if (pl > 0 && ln >= start && ln < start + pl) {
        sLane[0] = g;
        sLane[1] = pl;
        sLane[2] = round * pl + (ln - start);
      }
      base += __shfl(incl, 63);
    }
  }
  __syncthreads();
  const int g = sLane[0];
  if (g < 0) return;  // l=0: a lane no group needs
  P = sLane[1];
  const int w = sLane[2];
  const int cnt = gcount[g];
  const int U = ntn * ((cnt + 255) / 256);
  int rem = U % P;
  if (2 * rem > P) rem = 0;
  const int nbig = U - rem;
  int unit, half = -1;
  if (w < nbig) {
    unit = w;
  } else if (w < nbig + 2 * rem) {
    unit = nbig + (w - nbig) / 2;
    half = (w - nbig) & 1;
  } else {
    return;  // l=0
  }
  const int mt = unit / ntn, nt = unit % ntn;
  const int row0 = mt * 256, rows = min(256, cnt - row0);
  if (half < 0)
    qkv_tile<256, kGemmWN, kStages>(X, Wq, Wk, Wv, gperm, T, d, n_kv, r, g, row0, rows, nt, 0,
                                    vtp, log2_theta, sbuf, sbuf + kStages * Big::SA, sTok, Qc,
                                    Kc, Vt);
  else
    qkv_tile<128, 1, 3>(X, Wq, Wk, Wv, gperm, T, d, n_kv, r, g, row0, rows, nt, half, vtp,
                        log2_theta, sbuf, sbuf + 3 * Half::SA, sTok, Qc, Kc, Vt);
}

// ---------------------------------------------------------- attention core

constexpr int kBQ = 32;        // queries per tile: one wave of 32 per head
constexpr int kBKey = 64;  // keys per step
constexpr int kCoreWaves = 4;  // one per query head of a 4-head chunk
constexpr int kCoreWgPerCU = 2;  // resident work-groups per CU (LDS 64 KB, <= 256 VGPRs each)
// One LDS stage: K block [64 keys][128 hd] (16-byte chunk c of key row k at slot
// c ^ (k & 15)) and V^T block [128 hd][64 keys] (chunk c of row j at slot
// c ^ ((j >> 1) & 7)); both 16 KB, filled by buffer->LDS loads.
constexpr int kStageK = kBKey * kHd;  // elements
constexpr int kStageV = kHd * kBKey;
// P = 2^(s scale - m) may reach 2^kPHeadroom above the reference max m: bf16 P
// and the fp32 sums stay finite
constexpr float kPHeadroom = 64.f;

// The values of x in lanes l and l ^ 32, in some order (v_permlane32_swap).
WIDE_DEV void xhalf(float x, float& a, float& b) {
  const auto v =
      __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(v[0]);
  b = __uint_as_float(v[1]);
}

__global__ void __launch_bounds__(64 * kCoreWaves, kCoreWgPerCU)
    attn_core_prefill(const uint16_t* __restrict__ Qc, const uint16_t* __restrict__ Kc,
                      const uint16_t* __restrict__ Vt, const int32_t* __restrict__ gcount,
                      const int32_t* __restrict__ gperm, int T, int n_kv, int r, int nbins,
                      int vtp, float scale_log2, uint16_t* __restrict__ O) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[2 * kStageK];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2 * kStageV];
  __shared__ int sRedo;  // some wave's rows outgrew their reference max

  // work-group -> (group, bin j of the group's B bins, chunk of 4 query heads).
  // Query tile qt of a group takes qt / 2 + 1 key steps, so a group's work grows
  // with the square of its count.  The grid's nbins * n_kv bin slots are shared
  // out among the groups by that work (each group keeps at least one; near-equal
  // counts get an equal share, nbins each), and the groups' slots are laid out
  // XCD by XCD (slot p on XCD p / (slots / 8)), so a group's K and V stay in one
  // or few XCDs' L2.  The group's tiles, heaviest first, are dealt to its B bins
  // in snake order: bin j takes the tiles of rank j, 2B-1-j, 2B+j, 4B-1-j, ...,
  // so the bins of a group do nearly the same number of key steps (with B = half
  // the tiles this is the heavy + light pairing).
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int sSlot[3];  // group, bin, bins of the group (-1: no work)
  const int nslots = nbins * n_kv;
  const int hc = blockIdx.x / nslots;
  if (wave == 0) {
    const int w = blockIdx.x % nslots;
    const int p = (nslots & 7) == 0 ? (w & 7) * (nslots >> 3) + (w >> 3) : w;
    // per-group work (key steps, about qtiles^2 / 4) and its total
    long long tot = 0, wmax = 0;
    for (int g0 = 0; g0 < n_kv; g0 += 64) {
      const int g = g0 + lane;
      const long long q = g < n_kv ? (gcount[g] + kBQ - 1) / kBQ : 0;
      const long long wg = q * (q + 3) / 4;
      long long sum = wg, mx = wg;
      for (int off = 32; off >= 1; off >>= 1) {
        sum += __shfl_xor(sum, off);
        mx = max(mx, (long long)__shfl_xor(mx, off));
      }
      tot += sum;
      wmax = max(wmax, mx);
    }
    const bool equal = 4 * wmax * n_kv <= 5 * tot;  // every group within 25 % of the mean
    if (lane == 0) sSlot[0] = -1;
    int base = 0;
    for (int g0 = 0; g0 < n_kv && tot > 0; g0 += 64) {
      const int g = g0 + lane;
      int b = 0;
      if (g < n_kv) {
        const int q = (gcount[g] + kBQ - 1) / kBQ;
        const long long wg = (long long)q * (q + 3) / 4;
        b = equal ? nbins
                  : (q > 0 ? 1 + (int)((long long)(nslots - n_kv) * wg / tot) : 0);
        b = min(b, q);  // a bin takes at least one tile
      }
      int incl = b;  // inclusive prefix over the lanes
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      const int start = base + incl - b;
      if (b > 0 && p >= start && p < start + b) {
        sSlot[0] = g;
        sSlot[1] = p - start;
        sSlot[2] = b;
      }
      base += __shfl(incl, 63);
    }
  }
  __syncthreads();
  const int g = sSlot[0];
  if (g < 0) return;  // l=0: a slot no group's tiles need
  const int j = sSlot[1];
  nbins = sSlot[2];
  const int cnt = gcount[g];
  const int qtiles = (cnt + kBQ - 1) / kBQ;
  const int hw = wave;  // head of the chunk
  const bool head_ok = hc * 4 + hw < r;  // waves past the group's heads only help load
  const int h = g * r + min(hc * 4 + hw, r - 1);
  const int c0 = lane & 31, half = lane >> 5;

  const i32x4 kSrd = make_srd(Kc + (size_t)g * T * kHd, (uint32_t)((size_t)T * kHd * 2));
  const i32x4 vSrd = make_srd(Vt + (size_t)g * kHd * vtp, (uint32_t)((size_t)kHd * vtp * 2));
  const uint32_t ldsK = lds_addr(sK), ldsV = lds_addr(sV);
  // buffer->LDS loads of key block kb into stage st: instruction i of wave w fills
  // K rows 4 (4 i + w) .. +3 and V^T rows 8 (4 i + w) .. +7 (1 KB each)
  auto issue = [&](int kb, int st) {
    const int k0 = kb * kBKey;
#pragma unroll
    for (int i = 0; i < 16 / kCoreWaves; ++i) {
      const int n = kCoreWaves * i + wave;
      const int krow = 4 * n + (lane >> 4), kslot = lane & 15;
      const int kchunk = kslot ^ (krow & 15);
      const uint32_t koff =
          k0 + krow < cnt ? (uint32_t)(((k0 + krow) * kHd + kchunk * 8) * 2) : kSkip;
      lds_dma16(kSrd, ldsK + (st * kStageK + n * 512) * 2, koff);
      const int vrow = 8 * n + (lane >> 3), vslot = lane & 7;
      const int vchunk = vslot ^ ((vrow >> 1) & 7);
      // chunk c holds half of the 16-key group c / 2 (zero-padded past the count)
      const int kg = k0 + 16 * (vchunk >> 1);
      const uint32_t voff =
          kg < cnt ? (uint32_t)((vrow * vtp + k0 + vchunk * 8) * 2) : kSkip;
      lds_dma16(vSrd, ldsV + (st * kStageV + n * 512) * 2, voff);
    }
  };

  for (int it = 0;; ++it) {
    const int rank = (it >> 1) * 2 * nbins + ((it & 1) ? 2 * nbins - 1 - j : j);
    if (rank >= qtiles) break;
    const int qt = qtiles - 1 - rank;
    const int q0 = qt * kBQ;
    const int q_last = min(cnt, q0 + kBQ) - 1;
    const int nkb = q_last / kBKey + 1;
    const int q = q0 + c0;  // this lane's query (its S^T column)

    // Q^T fragments as B operands: lane holds query q, hd 16 ks + 8 half.
    bf16x8 qf[8];
    const uint16_t* qbase = Qc + (size_t)h * T * kHd;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (q < cnt)
        qf[ks] = *reinterpret_cast<const bf16x8*>(qbase + (size_t)q * kHd + ks * 16 + half * 8);
      else
        qf[ks] = bf16x8{};
    }
    f32x16 o[4];  // O^T: 4 hd blocks x this wave's 32 queries
    float l_run;
    // The reference max m of a query is the max of its first keys (O and l are
    // still 0 then) and is not raised afterwards, so O is never rescaled inside
    // the key loop (O / l is the same for any common offset).  A later score
    // more than kPHeadroom above m sets `over`; then the tile is computed again
    // with the true row max (m_true, tracked in the first pass) as m, which no
    // score exceeds, so there are at most two passes.
    float m_ref = -INFINITY, m_true = -INFINITY;
    for (int pass = 0; pass < 2; ++pass) {
      lds_barrier();  // the previous pass's or tile's last stage reads are done
      if (tid == 0) sRedo = 0;
      issue(0, 0);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[a][e] = 0.f;
      l_run = 0.f;
      bool over = false;

      for (int kb = 0; kb < nkb; ++kb) {
        const int k0 = kb * kBKey, st = kb & 1;
        // every wave's loads of block kb have landed (this wave's loads of block
        // kb + 1 may stay in flight)
        if (kb + 1 < nkb) {
          issue(kb + 1, st ^ 1);
          stage_barrier<32 / kCoreWaves>();
        } else {
          stage_barrier<0>();
        }
        const uint16_t* cK = sK + st * kStageK;
        const uint16_t* cV = sV + st * kStageV;
        auto kfrag = [&](int ks, int a) {
          const int row = a * 32 + c0;
          return *reinterpret_cast<const bf16x8*>(cK + row * kHd +
                                                  (((2 * ks + half) ^ (row & 15)) * 8));
        };
        auto vfrag = [&](int a, int sp, int hb) {
          const int row = hb * 32 + c0, chunk = 2 * (2 * a + sp) + half;
          return *reinterpret_cast<const bf16x8*>(cV + row * kBKey +
                                                  ((chunk ^ ((row >> 1) & 7)) * 8));
        };
        // the stage's two 32-key halves in turn
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int kk0 = k0 + a * 32;
          // S^T [32 keys x 32 queries] = K Q^T; the K fragment of step ks + 1 is read
          // from LDS before the MFMA of step ks
          f32x16 s;
#pragma unroll
          for (int e = 0; e < 16; ++e) s[e] = 0.f;
          bf16x8 kc = kfrag(0, a);
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) {
            bf16x8 kn;
            if (ks < 7) kn = kfrag(ks + 1, a);
            s = mfma32(kc, qf[ks], s);
            if (ks < 7) kc = kn;
          }
          // the V^T fragments of the first P V step, read while the softmax runs
          bf16x8 vc[4];
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) vc[hb] = vfrag(a, 0, hb);

          // softmax numerators in the log2 domain.  Masks (causal in compacted
          // order, keys past the count) only on the blocks that need them.
          if (kk0 + 32 > q0 || kk0 + 32 > cnt) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int key = kk0 + acc32_row(lane, e);
              if (key > q || key >= cnt) s[e] = -INFINITY;
            }
          }
          float mx = s[0];
#pragma unroll
          for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e]);
          float xa, xb;
          xhalf(mx, xa, xb);
          mx = fmaxf(xa, xb) * scale_log2;
          m_ref = m_ref == -INFINITY ? mx : m_ref;
          m_true = fmaxf(m_true, mx);
          over = over || mx > m_ref + kPHeadroom;
          // a query with no finite score yet keeps a finite state
          const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
          float sum = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float pe = __builtin_amdgcn_exp2f(fmaf(s[e], scale_log2, -m_use));
            s[e] = pe;
            sum += pe;
          }
          xhalf(sum, xa, xb);
          l_run += xa + xb;
          // O^T [128 x 32] += V^T [128 x 32 keys] P^T [32 keys x 32 q].  The k-slots
          // of a lane are the keys its S^T registers hold, 16 s' + 4 half +
          // {0..3, 8..11}; the permuted V^T layout stores exactly those 8 keys as
          // chunk 2 (2 a + s') + half.
#pragma unroll
          for (int sp = 0; sp < 2; ++sp) {
            bf16x8 vn[4];
            if (sp == 0) {
#pragma unroll
              for (int hb = 0; hb < 4; ++hb) vn[hb] = vfrag(a, 1, hb);
            }
            bf16x8 pf;
#pragma unroll
            for (int k = 0; k < 8; ++k) pf[k] = (__bf16)s[8 * sp + k];
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) o[hb] = mfma32(vc[hb], pf, o[hb]);
            if (sp == 0) {
#pragma unroll
              for (int hb = 0; hb < 4; ++hb) vc[hb] = vn[hb];
            }
          }
        }
        lds_barrier();  // stage st is refilled by the next step's loads
      }
      if (ballot(over) && lane == 0) sRedo = 1;
      __syncthreads();
      if (sRedo == 0) break;
      m_ref = m_true;
    }

    // O[token, h*hd + j] = O^T[j][q] / l
    if (head_ok && q < cnt) {
      const int tok = gperm[(size_t)g * T + q];
      const float inv = 1.f / l_run;
      uint16_t* dst = O + (size_t)tok * (n_kv * r * kHd) + h * kHd;
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int j = hb * 32 + 8 * q4 + 4 * half;
          const f32x16& a = o[hb];
          const uint32_t lo = pack_bf2(a[4 * q4] * inv, a[4 * q4 + 1] * inv);
          const uint32_t hi = pack_bf2(a[4 * q4 + 2] * inv, a[4 * q4 + 3] * inv);
          *reinterpret_cast<u32x2*>(dst + j) = u32x2{lo, hi};
        }
    }
  }
}

void launch_attn_prefill(const uint16_t* X, const uint16_t* Wq, const uint16_t* Wk,
                         const uint16_t* Wv, const ReorderView& rv, int T, int d, int n_kv, int r,
                         float rope_theta, uint16_t* Qc, uint16_t* Kc, uint16_t* Vt, uint16_t* O,
                         hipStream_t s) {
  const int mtiles = (T + 255) / 256;
  const int ntn = (r + 1) / 2 + 1;
  const float log2_theta = rope_theta > 0.f ? log2f(rope_theta) : 0.f;
  const int vtp = vt_pitch(T);
  {
    // compute units per group; a group has at most mtiles * ntn units and P / 2
    // extra work-groups for halves
    // Up to 64 groups: lanes shared out by units; the rounds of the 256 lanes
    // cover the units of every group at any counts (a group's lanes are at least
    // its share of 256 - n_kv, rounded down, plus one; its halves add under one
    // round).  More groups: P lanes per group, one after another.
    const int P = std::max(1, kCoreCUs / n_kv);
    const bool lanes = n_kv <= 64;
    const int units = n_kv * mtiles * ntn;
    const int grid = lanes ? kCoreCUs * ((units + kCoreCUs - n_kv - 1) / (kCoreCUs - n_kv) + 2)
                           : n_kv * (mtiles * ntn + P / 2);
    WIDE_TRACE("attn_qkv_prefill", s);
    attn_qkv_prefill<<<grid, kGemmThreads, 0, s>>>(X, Wq, Wk, Wv, rv.count, rv.perm, T, d, n_kv,
                                                   r, P, lanes, vtp, log2_theta, Qc, Kc, Vt);
  }
  // bins per group: half the most tiles a group can have, but no more than fill
  // the CUs once (256 CUs, kCoreWgPerCU work-groups each)
  const int hcs = (r + 3) / 4;
  const int npairs = ((T + kBQ - 1) / kBQ + 1) / 2;
  const int nbins = std::max(1, std::min(npairs, kCoreWgPerCU * kCoreCUs / (n_kv * hcs)));
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)kHd);
  {
    WIDE_TRACE("attn_core_prefill", s);
    attn_core_prefill<<<nbins * n_kv * hcs, 64 * kCoreWaves, 0, s>>>(
        Qc, Kc, Vt, rv.count, rv.perm, T, n_kv, r, nbins, vtp, scale_log2, O);
  }
}

}  // namespace wide
