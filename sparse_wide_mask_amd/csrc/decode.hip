// Decode (a small batch of single tokens): weight streaming over the touched
// groups only (gist.science technical summary §2.C, block-level skipping).
//
// A decode batch has at most 64 tokens, so one wave holds a group's mask column
// (lane = token) and the mask reordering is done inside the kernels that need
// it: a ballot over the column gives the kept tokens, and their ranks among the
// set bits give the stable kept-first order.  No separate reorder launch runs.
// Kernels (batch B <= 64):
//
// nmask_decode   N-masked projection (FFN gate+up, or attention q/k/v).  One
//                work-group = (group, 16 MFMA output columns); it exits at once
//                when no token keeps the group (l=0).  The tokens that keep the
//                group, in order, are the MFMA rows (16x16x32), padded to 16
//                (l=2: row blocks past the count are skipped); the 4 waves split
//                d_model and reduce through LDS.  FFN: the 16 columns are 8 gate
//                and the matching 8 up channels, so SwiGLU pairs lanes ch and
//                ch+8; epilogue writes H.  Attention: RoPE at the new token's
//                position and the q / new k,v writes (k and v straight into the
//                caches at the pair's slot: the batch's kv_len, or the
//                (sequence, group)'s own length; see DecCache).
// kmask_decode   K-masked projection (FFN down, attention out).  One work-group =
//                (128 output columns, one stretch of the batch union's K); it
//                packs the batch's mask into bit words and their union in LDS,
//                stages each unit's activation rows in LDS once for its 8 waves
//                (rows of tokens that dropped a group are not loaded, l=1), and
//                writes fp32 partial sums that kmask_decode_reduce adds.
// attn_decode_partial / attn_decode_combine
//                split-KV attention of each kept (token, group) over its cache
//                slots and the new token, 128 keys per work-group, then a
//                log-sum-exp combine of the chunks.
#include <type_traits>

#include "common.h"
#include "gemm_tile.h"
#include "internal.h"

namespace wide {

constexpr int kDecRows = 64;  // max batch of the decode kernels
constexpr int kDecRB = kDecRows / 16;
constexpr int kHdD = 128;

// Mode of nmask_decode.
enum { kNmFfn = 0, kNmQkv = 1 };

// Weight loads of this many 32-wide K steps are issued before their MFMAs, with
// the matching activation loads: W takes 4 VGPRs per step and X 4 per step and
// row block, so fewer steps are batched when the batch spans more row blocks.
template <int NRB, int NCB = 1>
constexpr int dec_unroll() {
  return NRB == 1 ? (NCB == 1 ? 16 : 8) : NRB == 2 ? (NCB == 1 ? 8 : 4) : 4;
}

// Activation operand of one 16x16x32 step: a buffer load whose offset is past the
// buffer for rows without a token, so it returns zeros and is never a branch.
WIDE_DEV bf16x8 xload(rsrc_t r, uint32_t off) {
  const u32x4 v = ldbuf16(r, off);
  return *reinterpret_cast<const bf16x8*>(&v);
}

// One MFMA output column of the N-masked decode projection: its weight row and,
// at the end, where its value for a token goes.  FFN: columns 0..7 are gate
// channels cb*8 + ch, columns 8..15 the same up channels, and SwiGLU pairs lane
// ch with lane ch + 8.  Attention: chunk cb of head hh (q heads 0..r-1, then k,
// then v) covers head dims {8c..8c+7} and {64+8c..64+8c+7}, so each RoPE pair
// (j, j + 64) is a lane pair too; rotation is at position kv_len, and k and v go
// straight into the caches at slot kv_len.
// The decode K/V caches: where a kept (sequence, group) appends the new token's
// K/V and how many earlier entries it attends to.  One length for the whole batch
// (kvl null), or one per (sequence, group) (kvl [B, n_groups]: caches in which
// tokens that skipped the group left no entry).  A length outside [0, kv_cap)
// makes the pair write nothing and output zero.  pos is the new token's RoPE
// position.
// Layout: contiguous (pt null), slot s of pair (b, g) at row (b n_groups + g)
// kv_cap + s; or paged, a pool of n_pages pages of 2^page_shift rows and a page
// table pt [B, n_groups, kv_cap >> page_shift] that maps the pair's slot s to row
// s mod 2^page_shift of page pt[b, g, s >> page_shift].  A slot on an unmapped
// page (entry outside [0, n_pages)) reads as zeros and takes no write; a pair
// whose new slot is on one takes no part, like an out-of-range length.
struct DecCache {
  const int32_t* kvl;
  int kv_len, kv_cap, pos;
  const int32_t* pt;
  int page_shift, n_pages;
  WIDE_DEV int len(int b, int g, int n_groups) const {
    return kvl ? kvl[b * n_groups + g] : kv_len;
  }
  WIDE_DEV bool ok(int l) const { return l >= 0 && l < kv_cap; }
  // cache row of slot s in [0, kv_cap) of pair (b, g); -1 on an unmapped page
  WIDE_DEV long long row(int b, int g, int n_groups, int s) const {
    const size_t pair = (size_t)b * n_groups + g;
    if (!pt) return (long long)(pair * kv_cap + s);
    const int p = pt[pair * (size_t)(kv_cap >> page_shift) + (s >> page_shift)];
    return p >= 0 && p < n_pages ? ((long long)p << page_shift) + (s & ((1 << page_shift) - 1))
                                 : -1;
  }
  // the pair takes part: its length is in range and its new slot is mapped
  WIDE_DEV bool live(int b, int g, int n_groups, int l) const {
    return ok(l) && (!pt || row(b, g, n_groups, l) >= 0);
  }
  // rows of the cache buffers
  WIDE_DEV size_t rows(int B, int n_groups) const {
    return pt ? (size_t)n_pages << page_shift : (size_t)B * n_groups * kv_cap;
  }
};

template <int MODE>
struct NmCol {
  const uint16_t* wrow;
  int hh = 0, jrow = 0;
  float sn = 0.f, cs = 1.f;
  bool rope = false;

  WIDE_DEV NmCol(int g, int cb, int ch, const uint16_t* W0, const uint16_t* W1,
                 const uint16_t* W2, int G, int d, int r, int pos, float log2_theta) {
    if (MODE == kNmFfn) {
      wrow = (ch < 8 ? W0 : W1) + (size_t)(g * G + cb * 8 + (ch & 7)) * d;
    } else {
      hh = cb / 8;
      const int c = cb % 8;
      jrow = ch < 8 ? 8 * c + ch : 64 + 8 * c + (ch - 8);
      if (hh < r)
        wrow = W0 + ((size_t)(g * r + hh) * kHdD + jrow) * d;
      else
        wrow = (hh == r ? W1 : W2) + ((size_t)g * kHdD + jrow) * d;
      rope = hh < r + 1 && log2_theta > 0.f;
      if (rope) {
        const float inv = exp2f(-(2.f * (ch < 8 ? jrow : jrow - 64) / kHdD) * log2_theta);
        sincosf((float)pos * inv, &sn, &cs);
      }
    }
  }

  // v = this lane's column value for token tok (tok < 0: no token).  Every lane
  // of the wave calls it (the pairing is a lane shuffle).
  WIDE_DEV void store(float v, int tok, int g, int cb, int ch, int G, int r, int n_groups,
                      const DecCache& dc, uint16_t* out0, uint16_t* Kc, uint16_t* Vc) const {
    const float other = __shfl_xor(v, 8);
    if (MODE == kNmFfn) {
      if (tok >= 0 && ch < 8)
        out0[(size_t)tok * (n_groups * G) + g * G + cb * 8 + ch] = f2bf(silu(v) * other);
    } else {
      float o = v;
      if (rope) o = ch < 8 ? v * cs - other * sn : v * cs + other * sn;
      if (tok < 0) return;
      const uint16_t bits = f2bf(o);
      if (hh < r) {
        out0[((size_t)tok * (n_groups * r) + g * r + hh) * kHdD + jrow] = bits;
      } else {
        const int slot = dc.len(tok, g, n_groups);
        const long long row = dc.ok(slot) ? dc.row(tok, g, n_groups, slot) : -1;
        if (row >= 0) (hh == r ? Kc : Vc)[(size_t)row * kHdD + jrow] = bits;
      }
    }
  }
};

// Batches up to this size run the N-masked decode kernel on a compacted grid.
constexpr int kDecCompactRows = 4;

// Compacted grid of the N-masked decode kernel (B <= kDecCompactRows): work-group
// row q takes the q-th group (ascending) that some token of the batch keeps, so
// the work-groups of kept groups come first and the rest (l=0) exit together at
// the end of the grid.  Exits interleaved with working groups slow the working
// ones (a read kernel of the same bytes with every other run of 16 work-groups
// empty took 27 us instead of 22 us; with the empty ones last, 22 us).  Thread
// t < n_groups reads group t's mask column; returns the group (-1: none) and
// its column's token bits.  A work-group of NW >= 4 waves, n_groups <= 256.
template <int NW>
WIDE_DEV int union_group_nth(const uint8_t* mask, int B, int n_groups, int q, int* sSel,
                             int* sWc, uint32_t* colbits_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const rsrc_t mr = make_rsrc(mask, (uint32_t)(B * n_groups));
  uint32_t col = 0;
#pragma unroll
  for (int b = 0; b < kDecCompactRows; ++b)
    col |= (ldbuf1(mr, b < B && tid < n_groups ? (uint32_t)(b * n_groups + tid) : kSkip) != 0u)
           << b;
  if (tid == 0) sSel[0] = -1;
  const uint64_t bits = ballot(col != 0u);
  if (lane == 0) sWc[wave] = popc64(bits);
  __syncthreads();
  int rank = popc64(bits & ((1ull << lane) - 1ull));
  for (int w = 0; w < wave; ++w) rank += sWc[w];
  if (col != 0u && rank == q) {
    sSel[0] = tid;
    sSel[1] = (int)col;
  }
  __syncthreads();
  *colbits_out = (uint32_t)sSel[1];
  return sSel[0];
}

// NCB: MFMA column blocks per wave (consecutive chunks of the group).  Each wave
// reads an activation fragment once for its NCB weight fragments, so a larger
// NCB reads the activation rows fewer times from L2 (they are as many bytes as
// the weights when every 16 columns read them); the grid has NCB times fewer
// work-groups.
template <int MODE, int NRB, int NCB, int NW>
__global__ void __launch_bounds__(64 * NW)
    nmask_decode(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W0,
                 const uint16_t* __restrict__ W1, const uint16_t* __restrict__ W2,
                 const uint8_t* __restrict__ mask, int B, int d, int G, int chunks, int r,
                 DecCache dc, float log2_theta, uint16_t* __restrict__ out0,
                 uint16_t* __restrict__ Kc, uint16_t* __restrict__ Vc, int n_groups) {
  constexpr int NEL = NCB * NRB * 256;  // output elements of the work-group
  __shared__ int sTok[kDecRows];
  __shared__ float sRed[NW][NEL];
  __shared__ int sSel[2], sWc[NW];

  const int cpw = chunks / NCB;  // work-groups per group
  const int q = blockIdx.x / cpw, cb0 = (blockIdx.x % cpw) * NCB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // group g and its mask column (one token per bit): kept tokens in order are the
  // MFMA rows
  int g;
  uint64_t mcol;
  if (B <= kDecCompactRows) {
    uint32_t colbits;
    g = union_group_nth<NW>(mask, B, n_groups, q, sSel, sWc, &colbits);
    if (g < 0) return;  // l=0: past the batch's union
    mcol = colbits;
  } else {
    g = q;
    const rsrc_t mr = make_rsrc(mask, (uint32_t)(B * n_groups));
    mcol = ballot(ldbuf1(mr, lane < B ? (uint32_t)(lane * n_groups + g) : kSkip) != 0u);
    if (mcol == 0) return;  // l=0: no token of the batch keeps g
  }
  const bool kept = (mcol >> lane) & 1ull;
  const int cnt = popc64(mcol);
  if (wave == 0) {
    if (kept) sTok[popc64(mcol & ((1ull << lane) - 1ull))] = lane;
    if (lane >= cnt) sTok[lane] = -1;
  }
  __syncthreads();
  const int nrb = (cnt + 15) / 16;  // l=2: row blocks past the count are skipped

  const int ch = lane & 15;
  const int koff = 8 * (lane >> 4);
  const uint16_t* wp[NCB];
#pragma unroll
  for (int j = 0; j < NCB; ++j)
    wp[j] = NmCol<MODE>(g, cb0 + j, ch, W0, W1, W2, G, d, r, dc.pos, 0.f).wrow + koff;

  f32x4 acc[NRB][NCB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int j = 0; j < NCB; ++j) acc[rb][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = d / 32;  // 32-wide K steps, split evenly over the NW waves
  const int kbeg = (wave * nsteps / NW) * 32, kend = ((wave + 1) * nsteps / NW) * 32;
  // X byte offsets of this lane's rows (k = koff); kSkip for rows without a token
  const rsrc_t xr = make_rsrc(X, (uint32_t)((size_t)B * d * 2));
  uint32_t xoff[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int tok = sTok[rb * 16 + ch];
    xoff[rb] = tok >= 0 ? (uint32_t)(((size_t)tok * d + koff) * 2) : kSkip;
  }
  // Every work-group reads the same activation rows; each starts its K walk at
  // a different batch so that they do not all hit the same L2 lines at once.
  constexpr int U = dec_unroll<NRB, NCB>();
  const int S = (kend - kbeg) / 32;
  const int nbat = S / U;
  const int rot = nbat > 0 ? (int)((blockIdx.x * 7u) % (unsigned)nbat) * U : 0;
  auto kat = [&](int j) {  // K offset of step j; a whole batch stays contiguous
    if (j >= nbat * U) return kbeg + 32 * j;
    const int s = j + rot;
    return kbeg + 32 * (s >= nbat * U ? s - nbat * U : s);
  };
  if constexpr (NRB == 1) {
    // few rows: MFMA fragments straight from global memory
#pragma unroll 1
    for (int j0 = 0; j0 < nbat * U; j0 += U) {
      bf16x8 wf[U][NCB], xf[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < NCB; ++j)
          wf[u][j] = *reinterpret_cast<const bf16x8*>(wp[j] + kat(j0 + u));
#pragma unroll
      for (int u = 0; u < U; ++u) xf[u] = xload(xr, xoff[0] + kat(j0 + u) * 2);
      __builtin_amdgcn_sched_barrier(0);  // all loads of the batch before its MFMAs
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < NCB; ++j) acc[0][j] = mfma16(xf[u], wf[u][j], acc[0][j]);
    }
  } else {
    // Many rows (used when there are too few column blocks to fill the chip
    // with nmask_decode_cols): 16-row fragment loads are slow from L2, so each
    // wave copies its batch's rows (64 U bytes per row) with contiguous loads
    // into its own LDS area (16-byte chunk c of row i at slot c ^ (i mod CPR))
    // and reads the fragments from there.
    constexpr int CPR = 4 * U;          // 16-byte chunks per row per batch
    constexpr int RPI = 64 / CPR;       // rows per load instruction
    constexpr int NI = 16 * NRB / RPI;  // load instructions per batch
    __shared__ __attribute__((aligned(16))) uint16_t sX[NW][16 * NRB * CPR * 8];
    uint16_t* myX = sX[wave];
    const int lrow = lane / CPR, lch = lane % CPR;
    uint32_t rowoff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tok = sTok[i * RPI + lrow];
      rowoff[i] = tok >= 0 ? (uint32_t)(((size_t)tok * d + lch * 8) * 2) : kSkip;
    }
#pragma unroll 1
    for (int j0 = 0; j0 < nbat * U; j0 += U) {
      const int k0 = kat(j0);
      bf16x8 wf[U][NCB];
      u32x4 xv[NI];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < NCB; ++j)
          wf[u][j] = *reinterpret_cast<const bf16x8*>(wp[j] + k0 + 32 * u);
#pragma unroll
      for (int i = 0; i < NI; ++i) xv[i] = ldbuf16(xr, rowoff[i] + k0 * 2);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int row = i * RPI + lrow;
        *reinterpret_cast<u32x4*>(myX + (row * CPR + (lch ^ (row % CPR))) * 8) = xv[i];
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          if (rb >= nrb) continue;
          const int row = rb * 16 + ch, c = 4 * u + (lane >> 4);
          const bf16x8 xf =
              *reinterpret_cast<const bf16x8*>(myX + (row * CPR + (c ^ (row % CPR))) * 8);
#pragma unroll
          for (int j = 0; j < NCB; ++j) acc[rb][j] = mfma16(xf, wf[u][j], acc[rb][j]);
        }
      __builtin_amdgcn_wave_barrier();  // fragment reads before the next batch's writes
    }
  }
  for (int j0 = nbat * U; j0 < S; ++j0) {
    const int k0 = kat(j0);
#pragma unroll
    for (int j = 0; j < NCB; ++j) {
      const bf16x8 wf = *reinterpret_cast<const bf16x8*>(wp[j] + k0);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        if (rb < nrb) acc[rb][j] = mfma16(xload(xr, xoff[rb] + k0 * 2), wf, acc[rb][j]);
    }
  }

  // reduce the NW K-stretches: every wave parks its partial sums in LDS, the
  // work-group adds them (one element per thread at a time), wave 0 stores
#pragma unroll
  for (int j = 0; j < NCB; ++j)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sRed[wave][((j * NRB + rb) * 16 + acc16_row(lane, i)) * 16 + ch] = acc[rb][j][i];
  __syncthreads();
  for (int e = tid; e < NEL; e += 64 * NW) {
    float v = sRed[0][e];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += sRed[w][e];
    sRed[0][e] = v;
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int j = 0; j < NCB; ++j) {
    const NmCol<MODE> col(g, cb0 + j, ch, W0, W1, W2, G, d, r, dc.pos, log2_theta);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      if (rb >= nrb) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rb * 16 + acc16_row(lane, i);
        const float v = sRed[0][((j * NRB + rb) * 16 + acc16_row(lane, i)) * 16 + ch];
        col.store(v, row < cnt ? sTok[row] : -1, g, cb0 + j, ch, G, r, n_groups, dc, out0,
                  Kc, Vc);
      }
    }
  }
}

// The same projection for batches over 16 tokens, where the activation rows
// (up to 64 x d) are read as often as the weights: a work-group is 4 waves x 16
// columns over the whole of K, and each batch of 8 K steps of the rows is copied
// once per work-group, with contiguous loads, into an LDS tile that all 4 waves
// read their fragments from (16-byte chunk c of row i at slot c ^ (i mod 32));
// two tiles alternate so the next batch's rows and weights load during the
// MFMAs of this one.
template <int MODE, int NRB>
__global__ void __launch_bounds__(256)
    nmask_decode_cols(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W0,
                      const uint16_t* __restrict__ W1, const uint16_t* __restrict__ W2,
                      const uint8_t* __restrict__ mask, int B, int d, int G, int chunks, int r,
                      DecCache dc, float log2_theta, uint16_t* __restrict__ out0,
                      uint16_t* __restrict__ Kc, uint16_t* __restrict__ Vc, int n_groups) {
  constexpr int U = 8;                  // 32-wide K steps per batch
  constexpr int ROWS = 16 * NRB;
  constexpr int CPR = 4 * U;            // 16-byte chunks of a row per batch
  constexpr int XL = ROWS * CPR / 256;  // 16-byte loads per thread per batch
  __shared__ int sTok[kDecRows];
  __shared__ __attribute__((aligned(16))) uint16_t sX[2][ROWS * CPR * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c4n = chunks / 4;
  const int g = blockIdx.x / c4n, cb = (blockIdx.x % c4n) * 4 + wave;
  const rsrc_t mr = make_rsrc(mask, (uint32_t)(B * n_groups));
  const bool kept = ldbuf1(mr, lane < B ? (uint32_t)(lane * n_groups + g) : kSkip) != 0u;
  const uint64_t mcol = ballot(kept);
  const int cnt = popc64(mcol);
  if (cnt == 0) return;  // l=0: no token of the batch keeps g
  if (wave == 0) {
    if (kept) sTok[popc64(mcol & ((1ull << lane) - 1ull))] = lane;
    if (lane >= cnt) sTok[lane] = -1;
  }
  __syncthreads();
  const int nrb = (cnt + 15) / 16;  // l=2: row blocks past the count are skipped
  const int ch = lane & 15, koff = 8 * (lane >> 4);
  const NmCol<MODE> col(g, cb, ch, W0, W1, W2, G, d, r, dc.pos, log2_theta);
  const uint16_t* wp = col.wrow + koff;

  // this thread's share of a batch copy: chunk q = tid + 256 i of the tile
  const rsrc_t xr = make_rsrc(X, (uint32_t)((size_t)B * d * 2));
  uint32_t xo[XL];
  int xdst[XL];
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int q = tid + 256 * i, row = q / CPR, c = q % CPR;
    const int tok = sTok[row];
    xo[i] = tok >= 0 ? (uint32_t)(((size_t)tok * d + c * 8) * 2) : kSkip;
    xdst[i] = (row * CPR + (c ^ (row % CPR))) * 8;
  }
  f32x4 acc[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nb = d / (32 * U);
  // work-groups start at different batches so they do not all read the same
  // activation lines at once
  const int rot = nb > 0 ? (int)((blockIdx.x * 7u) % (unsigned)nb) : 0;
  auto kof = [&](int b) {
    const int s = b + rot;
    return 32 * U * (s >= nb ? s - nb : s);
  };
  u32x4 xv[XL];
  bf16x8 wc[U];
  if (nb > 0) {
    const int k0 = kof(0);
#pragma unroll
    for (int i = 0; i < XL; ++i) xv[i] = ldbuf16(xr, xo[i] + k0 * 2);
#pragma unroll
    for (int u = 0; u < U; ++u) wc[u] = *reinterpret_cast<const bf16x8*>(wp + k0 + 32 * u);
#pragma unroll
    for (int i = 0; i < XL; ++i) *reinterpret_cast<u32x4*>(&sX[0][xdst[i]]) = xv[i];
    lds_barrier();
  }
#pragma unroll 1
  for (int b = 0; b < nb; ++b) {
    const bool more = b + 1 < nb;
    bf16x8 wn[U];
    if (more) {  // rows first: their LDS copy is waited for while the weights fly
      const int k1 = kof(b + 1);
#pragma unroll
      for (int i = 0; i < XL; ++i) xv[i] = ldbuf16(xr, xo[i] + k1 * 2);
#pragma unroll
      for (int u = 0; u < U; ++u) wn[u] = *reinterpret_cast<const bf16x8*>(wp + k1 + 32 * u);
    }
    const uint16_t* cx = sX[b & 1];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        if (rb >= nrb) continue;
        const int row = rb * 16 + ch, c = 4 * u + (lane >> 4);
        const bf16x8 xf = *reinterpret_cast<const bf16x8*>(cx + (row * CPR + (c ^ (row % CPR))) * 8);
        acc[rb] = mfma16(xf, wc[u], acc[rb]);
      }
    if (more) {
#pragma unroll
      for (int i = 0; i < XL; ++i) *reinterpret_cast<u32x4*>(&sX[(b + 1) & 1][xdst[i]]) = xv[i];
    }
    lds_barrier();
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) wc[u] = wn[u];
    }
  }
  // K steps past the last whole batch: fragments straight from global memory
  {
    uint32_t xof[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int tok = sTok[rb * 16 + ch];
      xof[rb] = tok >= 0 ? (uint32_t)(((size_t)tok * d + koff) * 2) : kSkip;
    }
    for (int k0 = nb * 32 * U; k0 < d; k0 += 32) {
      const bf16x8 wf = *reinterpret_cast<const bf16x8*>(wp + k0);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        if (rb < nrb) acc[rb] = mfma16(xload(xr, xof[rb] + k0 * 2), wf, acc[rb]);
    }
  }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    if (rb >= nrb) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rb * 16 + acc16_row(lane, i);
      col.store(acc[rb][i], row < cnt ? sTok[row] : -1, g, cb, ch, G, r, n_groups, dc, out0,
                Kc, Vc);
    }
  }
}

// K-masked decode projection: Y[b, c] = sum over union groups g of
// sum_j A[b, gG + j] Wp[g, c, j] over the tokens b that keep g (+ residual).
//
// One work-group = (128 output columns, one of S stretches of the union's K
// units).  A unit is (union group, UK-wide K block).  Per unit the work-group
// copies the batch's A rows of the unit (rows of tokens that dropped the group
// are not fetched, l=1) into LDS once, and each wave multiplies them by the
// weight rows of its 16 columns; weights and A rows are loaded two units ahead.
// Splitting K over work-groups is what keeps the A traffic low: every
// work-group reads only its stretch of A, so A crosses L2 d / 128 times in all
// rather than d / 16 times.  With S > 1 each work-group writes fp32 partial
// sums, and kmask_decode_reduce (the next launch) adds them and the residual.
// A device-scope handshake inside the kernel would need a release fence per
// work-group, which on this chip writes back the XCD's L2: the kernel boundary
// is the cheaper synchronisation.
constexpr int kKmWaves = 8;             // one 16-column MFMA tile per wave
constexpr int kKmCols = 16 * kKmWaves;  // output columns per work-group
constexpr int kKmThreads = 64 * kKmWaves;

int kmask_decode_col_blocks(int d) { return (d + kKmCols - 1) / kKmCols; }

// K splits: enough work-groups to fill the 256 CUs, at most kMaxDecSplits partial
// sums, and no more splits than the largest possible union has units.
constexpr int kMaxDecSplits = 16;
int kmask_decode_splits(int d, int n, int G) {
  const int units = n * (G % 128 == 0 ? G / 128 : G % 64 == 0 ? G / 64 : G / 32);
  const int ncb = kmask_decode_col_blocks(d);
  int s = (256 + ncb - 1) / ncb;
  s = s < kMaxDecSplits ? s : kMaxDecSplits;
  s = s < units ? s : units;
  return s > 1 ? s : 1;
}

template <int NRB, int KS, int USE>
__global__ void __launch_bounds__(kKmThreads)
    kmask_decode(const uint16_t* __restrict__ A, const uint16_t* __restrict__ Wp,
                 const uint8_t* __restrict__ mask, int B, int d, int F, int G, int n, int S,
                 const uint16_t* __restrict__ residual, float* __restrict__ part,
                 uint16_t* __restrict__ Y) {
  constexpr int UK = 32 * KS;   // K width of a unit
  constexpr int CPR = UK / 8;   // 16-byte chunks per A row of a unit
  constexpr int ROWS = 16 * NRB;
  constexpr int ACH = ROWS * CPR;  // chunks of a unit's A tile
  constexpr int AP = (ACH + kKmThreads - 1) / kKmThreads;
  __shared__ uint64_t sBits[kDecRows * 4];
  __shared__ uint32_t sU[8];
  __shared__ int sGroups[256];
  __shared__ int sNu;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][ROWS * UK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cb = blockIdx.x / S, sp = blockIdx.x - cb * S;
  if (tid < 8) sU[tid] = 0u;
  __syncthreads();
  // pack the batch's mask rows into bit words (ballot over 64 groups) and OR
  // them into the batch union; all of a wave's loads are issued first
  {
    constexpr int kPer = kDecRows / kKmWaves;
    const rsrc_t mr = make_rsrc(mask, (uint32_t)(B * n));
    uint32_t v[kPer][4];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int b = wave + k * kKmWaves;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int g = 64 * w + lane;
        v[k][w] = ldbuf1(mr, (b < B && g < n) ? (uint32_t)(b * n + g) : kSkip);
      }
    }
    uint64_t uni[4] = {0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int b = wave + k * kKmWaves;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint64_t word = ballot(v[k][w] != 0u);
        if (lane == 0) sBits[b * 4 + w] = word;
        uni[w] |= word;
      }
    }
    if (lane == 0)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if ((uint32_t)uni[w]) atomicOr(&sU[2 * w], (uint32_t)uni[w]);
        if ((uint32_t)(uni[w] >> 32)) atomicOr(&sU[2 * w + 1], (uint32_t)(uni[w] >> 32));
      }
  }
  __syncthreads();
  if (wave == 0) {  // ascending list of the union's groups
    int written = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint64_t u = ((uint64_t)sU[2 * w + 1] << 32) | sU[2 * w];
      if ((u >> lane) & 1ull) sGroups[written + popc64(u & ((1ull << lane) - 1ull))] = 64 * w + lane;
      written += popc64(u);
    }
    if (lane == 0) sNu = written;
  }
  __syncthreads();

  // this work-group's stretch of units; the work-groups of one stretch start at
  // different units so that they do not read the same A lines at once
  const int UPG = G / UK, NU = sNu * UPG;
  const int u0 = sp * NU / S, UW = (sp + 1) * NU / S - u0;
  const int rot = UW > 0 ? (int)((unsigned)cb % (unsigned)UW) : 0;
  const int ch = lane & 15, koff = 8 * (lane >> 4);
  const int col = cb * kKmCols + wave * 16 + ch;
  const rsrc_t ar = make_rsrc(A, (uint32_t)((size_t)B * F * 2));
  const rsrc_t wr = make_rsrc(Wp, (uint32_t)((size_t)n * d * G * 2));
  // unit j (j >= UW: padding, every load takes the kSkip offset)
  auto load = [&](int j, bf16x8 (&wf)[KS], u32x4 (&av)[AP]) {
    const bool live = j < UW;
    int u = j + rot;
    u = u0 + (u >= UW ? u - UW : u);
    const int q = live ? u / UPG : 0, k0 = live ? (u - q * UPG) * UK : 0;
    const int g = live ? sGroups[q] : 0;
    const uint32_t wo = (uint32_t)((((size_t)g * d + col) * G + k0 + koff) * 2);
    const bool wl = live && col < d;
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      const u32x4 v = ldbuf16(wr, wl ? wo + 64u * t : kSkip);
      wf[t] = *reinterpret_cast<const bf16x8*>(&v);
    }
#pragma unroll
    for (int k = 0; k < AP; ++k) {
      const int c = tid + k * kKmThreads, b = c / CPR, cc = c % CPR;
      const uint32_t kb =
          (uint32_t)(sBits[(b & (kDecRows - 1)) * 4 + (g >> 6)] >> (g & 63)) & (uint32_t)live;
      av[k] = ldbuf16(ar, (kb && c < ACH)
                              ? (uint32_t)(((size_t)b * F + (size_t)g * G + k0 + cc * 8) * 2)
                              : kSkip);
    }
  };
  f32x4 acc[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // unit j: its A rows (ac) into LDS buffer j & 1, the loads of unit j + 2 into
  // the free register set, then the MFMAs of unit j.  Row b's chunk c sits at
  // slot c ^ (b mod CPR), so the 16 rows of a fragment read spread over the banks.
  auto step = [&](int j, const bf16x8 (&wc)[KS], const u32x4 (&ac)[AP], bf16x8 (&wn)[KS],
                  u32x4 (&an)[AP]) {
    uint16_t* st = sA[j & 1];
#pragma unroll
    for (int k = 0; k < AP; ++k) {
      const int c = tid + k * kKmThreads, b = c / CPR, cc = c % CPR;
      if (ACH % kKmThreads == 0 || c < ACH)
        *reinterpret_cast<u32x4*>(st + (b * CPR + (cc ^ (b % CPR))) * 8) = ac[k];
    }
    __syncthreads();
    load(j + 2, wn, an);
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const int row = rb * 16 + ch, c = 4 * t + (lane >> 4);
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(st + (row * CPR + (c ^ (row % CPR))) * 8);
        acc[rb] = mfma16(af, wc[t], acc[rb]);
      }
  };
  if (UW > 0) {
    bf16x8 w0[KS], w1[KS], w2[KS];
    u32x4 a0[AP], a1[AP], a2[AP];
    load(0, w0, a0);
    load(1, w1, a1);
#pragma unroll 1
    for (int j = 0; j < UW; j += 3) {
      step(j, w0, a0, w2, a2);
      step(j + 1, w1, a1, w0, a0);
      step(j + 2, w2, a2, w1, a1);
    }
  }

  const uint16_t* res = residual;
  if (S == 1) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = rb * 16 + acc16_row(lane, i);
        if (b >= B || col >= d) continue;
        const size_t o = (size_t)b * d + col;
        float v = acc[rb][i];
        if (res) v += bf2f(res[o]);
        Y[o] = f2bf(v);
      }
    return;
  }
  float* mine = part + (size_t)sp * B * d;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = rb * 16 + acc16_row(lane, i);
      if (b < B && col < d) mine[(size_t)b * d + col] = acc[rb][i];
    }
}

// Y[b, c] = sum over the S partial sums (+ residual); 4 columns per thread.
__global__ void __launch_bounds__(256)
    kmask_decode_reduce(const float* __restrict__ part, int S, int B, int d,
                        const uint16_t* __restrict__ residual, uint16_t* __restrict__ Y) {
  const int i = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= B * d) return;
  const size_t plane = (size_t)B * d;
  // all S partials are requested before the first add (S <= kMaxDecSplits)
  f32x4 p[kMaxDecSplits];
#pragma unroll
  for (int s2 = 0; s2 < kMaxDecSplits; ++s2)
    if (s2 < S) p[s2] = *reinterpret_cast<const f32x4*>(part + s2 * plane + i);
  f32x4 v = p[0];
#pragma unroll
  for (int s2 = 1; s2 < kMaxDecSplits; ++s2)
    if (s2 < S) v[0] += p[s2][0], v[1] += p[s2][1], v[2] += p[s2][2], v[3] += p[s2][3];
  if (residual) {
    const u32x2 r = *reinterpret_cast<const u32x2*>(residual + i);
    v[0] += __uint_as_float(r[0] << 16), v[1] += __uint_as_float(r[0] & 0xffff0000u);
    v[2] += __uint_as_float(r[1] << 16), v[3] += __uint_as_float(r[1] & 0xffff0000u);
  }
  const uint32_t lo = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
  const uint32_t hi = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
  *reinterpret_cast<u32x2*>(Y + i) = u32x2{lo, hi};
}

// One thread per cache key of a chunk; a chunk's V rows take kKeyChunk * 256 B of
// LDS, so 128-key work-groups (32 KB) let four of them share a compute unit and
// overlap one another's loads and arithmetic.
constexpr int kKeyChunk = 128;
constexpr int kAttnWaves = kKeyChunk / 64;
constexpr int kKeyBlocks = kKeyChunk / 16 / kAttnWaves;  // 16-key MFMA blocks per wave
constexpr int kKeySlices = kKeyChunk / 32;                // 32-key slices of the P V step

// One work-group = (token b, group g, chunk of kKeyChunk cache keys).  All of the
// chunk's bytes are requested up front, every load instruction reading whole
// rows: the K rows straight into LDS by buffer->LDS loads (4 rows of 256 B per
// instruction), the V rows into registers (two rows per instruction), where the
// P V step uses them.  Loads of 16 rows x 64 B per instruction (K fragments read
// as MFMA operands from memory) held the kernel 5-7 % lower.
//   scores  S^T[key, h] = K[key, :] . Q[h, :] with v_mfma_f32_16x16x32_bf16, the
//           K fragments read from LDS: 16 keys x 16 head columns (the group's r
//           heads, the rest zero) per block, 4 blocks per wave;
//   softmax per-head max and sum over the chunk (thread t = key t);
//   P V     thread = (4 head dims, 32 keys) for all r heads, then a sum over
//           the key slices through LDS.
// Writes unnormalised partial outputs and the chunk's (max, sum) per head.
// PAGED: the cache rows come through the page table (DecCache).  Pages hold at
// least 16 slots, so a 16-key block and a 4-row group never cross a page, and a
// chunk spans at most 8 pages, whose entries lanes 0..7 load once.
template <bool PAGED>
__global__ void __launch_bounds__(kKeyChunk)
    attn_decode_partial(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kc,
                        const uint16_t* __restrict__ Vc, const uint8_t* __restrict__ mask, int B,
                        int n_kv, int r, DecCache dc, int nch, float scale_log2,
                        float* __restrict__ Opart, float* __restrict__ Mpart,
                        float* __restrict__ Lpart) {
  // K rows (256 B each; 16-byte chunk c of key k at slot c ^ (k mod 16)); reused
  // for the key-slice partial sums
  __shared__ __attribute__((aligned(16))) uint16_t sK[kKeyChunk * kHdD];
  __shared__ __attribute__((aligned(16))) float sP[8][kKeyChunk];
  __shared__ float sRed[8][kAttnWaves];
  const int c = blockIdx.x % nch, rest = blockIdx.x / nch;
  const int g = rest % n_kv, b = rest / n_kv;
  const int k0 = c * kKeyChunk;  // < kv_cap: the grid has the chunks of kv_cap slots
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // The pair's keep bit, its length (its keys are cache entries 0..len-1 and the new
  // token at slot len) and, paged, the chunk's page entries (lane l = page l of the
  // chunk) depend on none of each other: all are requested before the first test.
  int pgv = -1;
  if constexpr (PAGED) {
    const int first = k0 >> dc.page_shift, max_pages = dc.kv_cap >> dc.page_shift;
    const int npg = min(max(kKeyChunk >> dc.page_shift, 1), max_pages - first);
    if (lane < npg) pgv = dc.pt[((size_t)b * n_kv + g) * (size_t)max_pages + first + lane];
  }
  const int keep = mask[(size_t)b * n_kv + g];
  const int len = dc.len(b, g, n_kv);
  asm volatile("" ::"v"(keep), "s"(len), "v"(pgv));
  if (!keep) return;  // l=0: the token dropped this group
  // no such chunk for this pair.  (A paged pair whose new slot is unmapped still
  // runs: the combine outputs zero for it without reading these partials.)
  if (!dc.ok(len) || k0 > len) return;
  const int nkeys = min(kKeyChunk, len + 1 - k0);
  const int nq = n_kv * r;
  const uint32_t cache_bytes = (uint32_t)(dc.rows(B, n_kv) * kHdD * 2);
  const int m16 = lane & 15, q4 = lane >> 4;
  const size_t kvbase = ((size_t)b * n_kv + g) * dc.kv_cap + k0;
  // cache row of the chunk's key rel, -1 if unmapped.  UNIFORM: rel is the same
  // for the whole wave (the page entry is read with readlane), else any lane's own
  // (a lane shuffle).  Pages hold at least 16 slots, so the 16-key blocks and the
  // 4-row groups used below never cross a page.
  auto row_of = [&](int rel, auto uniform) -> long long {
    if constexpr (!PAGED) {
      return (long long)(kvbase + rel);
    } else {
      const int s = k0 + rel, i = (s >> dc.page_shift) - (k0 >> dc.page_shift);
      const int p = decltype(uniform)::value
                        ? __builtin_amdgcn_readlane(pgv, __builtin_amdgcn_readfirstlane(i))
                        : __shfl(pgv, i);
      return p >= 0 && p < dc.n_pages
                 ? ((long long)p << dc.page_shift) + (s & ((1 << dc.page_shift) - 1))
                 : -1;
    }
  };
  // K: instruction q of wave w fills the 4 whole rows from row0 = 4 (kAttnWaves q + w);
  // lane (q4, m16) loads chunk m16 ^ (row mod 16) of row row0 + q4 into slot m16
  {
    const i32x4 ksrd = make_srd(Kc, cache_bytes);
    const uint32_t klds = lds_addr(sK);
#pragma unroll
    for (int q = 0; q < kKeyChunk / (4 * kAttnWaves); ++q) {
      const int row0 = 4 * (kAttnWaves * q + wave), row = row0 + q4;
      const long long r0 = row_of(row0, std::true_type{});
      const uint32_t off = row < nkeys && r0 >= 0
                               ? (uint32_t)(((r0 + q4) * kHdD + ((m16 ^ (row & 15)) * 8)) * 2)
                               : kSkip;
      lds_dma16(ksrd, klds + row0 * kHdD * 2, off);
    }
  }
  // Q operand: column m16 = head of the group (zero past r)
  bf16x8 qf[4];
  {
    const rsrc_t qr = make_rsrc(Q + ((size_t)b * nq + g * r) * kHdD, (uint32_t)(r * kHdD * 2));
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[ks] = xload(qr, m16 < r ? (uint32_t)((m16 * kHdD + 32 * ks + 8 * q4) * 2) : kSkip);
  }
  // V into registers: thread = (dims 4 j4 .. +3, keys 32 kslice .. +31), 8 bytes of
  // each of its rows; one load of a wave reads two whole rows
  const int j4 = tid & 31, kslice = tid >> 5;
  u32x2 vr[32];
  {
    const rsrc_t vrs = make_rsrc(Vc, cache_bytes);
    const long long vb[2] = {row_of(32 * kslice, std::false_type{}),
                             row_of(32 * kslice + 16, std::false_type{})};
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int key = 32 * kslice + e;
      const long long r0 = vb[e / 16];
      vr[e] = __builtin_amdgcn_raw_buffer_load_b64(
          vrs, key < nkeys && r0 >= 0 ? (int)(((r0 + e % 16) * kHdD + 4 * j4) * 2) : (int)kSkip,
          0, 0);
    }
  }
  // K rows of every wave in LDS (and the Q operand); the V loads stay in flight
  asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kKeyBlocks; ++i) {
    const int key = 16 * (kKeyBlocks * wave + i) + m16;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 kfr = *reinterpret_cast<const bf16x8*>(
          sK + key * kHdD + (((4 * ks + q4) ^ (key & 15)) * 8));
      acc = mfma16(kfr, qf[ks], acc);
    }
    if (m16 < r) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kk = 16 * (kKeyBlocks * wave + i) + acc16_row(lane, e);
        sP[m16][kk] = kk < nkeys ? acc[e] * scale_log2 : -INFINITY;
      }
    }
  }
  __syncthreads();
  float mh[8], lh[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    if (h >= r) break;
    float m = sP[h][tid];
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) sRed[h][wave] = m;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    if (h >= r) break;
    float m = sRed[h][0];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) m = fmaxf(m, sRed[h][w]);
    mh[h] = m;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    if (h >= r) break;
    const float p = exp2f(sP[h][tid] - mh[h]);
    sP[h][tid] = p;
    float l = p;
    for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
    if (lane == 0) sRed[h][wave] = l;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    if (h >= r) break;
    float l = sRed[h][0];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) l += sRed[h][w];
    lh[h] = l;
  }
  // P V: P is zero and the V rows are zero past nkeys
  float o[8][4];
#pragma unroll
  for (int h = 0; h < 8; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) o[h][e] = 0.f;
#pragma unroll
  for (int kq = 0; kq < 32; kq += 4) {
    const int kk = 32 * kslice + kq;
    float vf[4][4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const u32x2 v2 = vr[kq + e];
      vf[e][0] = __uint_as_float(v2[0] << 16);
      vf[e][1] = __uint_as_float(v2[0] & 0xffff0000u);
      vf[e][2] = __uint_as_float(v2[1] << 16);
      vf[e][3] = __uint_as_float(v2[1] & 0xffff0000u);
    }
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      if (h >= r) break;
      const f32x4 p = *reinterpret_cast<const f32x4*>(&sP[h][kk]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int x = 0; x < 4; ++x) o[h][x] += p[e] * vf[e][x];
    }
  }
  // sK was last read before the softmax barriers
  float* sO = reinterpret_cast<float*>(sK);  // [kKeySlices][r][128]
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    if (h >= r) break;
    *reinterpret_cast<f32x4*>(sO + (kslice * r + h) * kHdD + 4 * j4) =
        f32x4{o[h][0], o[h][1], o[h][2], o[h][3]};
  }
  __syncthreads();
  const size_t obase = ((size_t)b * nq + g * r) * nch;
  for (int x = tid; x < r * kHdD; x += kKeyChunk) {
    const int h = x / kHdD, j = x % kHdD;
    float a = 0.f;
#pragma unroll
    for (int sl = 0; sl < kKeySlices; ++sl) a += sO[(sl * r + h) * kHdD + j];
    Opart[(obase + (size_t)h * nch + c) * kHdD + j] = a;
  }
  if (tid < r) {
    Mpart[obase + (size_t)tid * nch + c] = mh[tid];
    Lpart[obase + (size_t)tid * nch + c] = lh[tid];
  }
}

// (token b, query head h): O[b, h] = sum_c 2^(M_c - M) Opart_c / sum_c 2^(M_c - M) L_c,
// M = max_c M_c.  Thread = (head dim, chunk slice): the chunks are dealt to
// kCmbSlices slices so that each thread has few Opart loads to wait for, and the
// slices are added through LDS at the end.  Chunk weights are computed
// kCmbBlock at a time into LDS.
constexpr int kCmbSlices = 4;
constexpr int kCmbThreads = kHdD * kCmbSlices;
constexpr int kCmbWaves = kCmbThreads / 64;
constexpr int kCmbBlock = kCmbThreads;

__global__ void __launch_bounds__(kCmbThreads)
    attn_decode_combine(const float* __restrict__ Opart, const float* __restrict__ Mpart,
                        const float* __restrict__ Lpart, const uint8_t* __restrict__ mask,
                        int n_kv, int r, DecCache dc, int nch, uint16_t* __restrict__ O) {
  __shared__ float sW[kCmbBlock];
  __shared__ float sR[kCmbWaves];
  __shared__ float sO[kCmbSlices - 1][kHdD];
  const int nq = n_kv * r;
  const int b = blockIdx.x / nq, h = blockIdx.x % nq, g = h / r;
  if (!mask[(size_t)b * n_kv + g]) return;  // never read: the O projection skips it
  const size_t base = (size_t)b * nq * nch + (size_t)h * nch;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = tid % kHdD, sl = tid / kHdD;
  const int len = dc.len(b, g, n_kv);
  if (!dc.live(b, g, n_kv, len)) {  // a pair with an out-of-range length outputs zero
    if (sl == 0) O[((size_t)b * nq + h) * kHdD + j] = 0;
    return;
  }
  nch = (len + kKeyChunk) / kKeyChunk;  // this pair's chunks (the stride above stays)
  float m = -INFINITY;
  for (int c = tid; c < nch; c += kCmbThreads) m = fmaxf(m, Mpart[base + c]);
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) sR[wave] = m;
  __syncthreads();
  m = sR[0];
#pragma unroll
  for (int w = 1; w < kCmbWaves; ++w) m = fmaxf(m, sR[w]);
  float l = 0.f, acc = 0.f;
  for (int c0 = 0; c0 < nch; c0 += kCmbBlock) {
    const int cn = min(kCmbBlock, nch - c0);
    __syncthreads();  // the previous block's reads of sW and sR are done
    float lw = 0.f;
    if (tid < cn) {
      const float w = exp2f(Mpart[base + c0 + tid] - m);
      sW[tid] = w;
      lw = w * Lpart[base + c0 + tid];
    }
    for (int off = 32; off >= 1; off >>= 1) lw += __shfl_xor(lw, off);
    if (lane == 0) sR[wave] = lw;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kCmbWaves; ++w) l += sR[w];
#pragma unroll 8
    for (int c = sl; c < cn; c += kCmbSlices) acc += sW[c] * Opart[(base + c0 + c) * kHdD + j];
  }
  if (sl > 0) sO[sl - 1][j] = acc;
  __syncthreads();
  if (sl > 0) return;
#pragma unroll
  for (int q = 0; q < kCmbSlices - 1; ++q) acc += sO[q][j];
  O[((size_t)b * nq + h) * kHdD + j] = f2bf(acc / l);
}

// ------------------------------------------------------------------ launchers

// The column-block kernel (activation rows shared by 64 columns) once the batch
// spans several row blocks and its work-groups still fill the 256 CUs;
// otherwise the K-split kernel (16 columns per work-group, 4x the work-groups).
static bool use_cols(int nrb, int col_blocks) { return nrb > 1 && col_blocks >= 256; }

// Column blocks per wave of the attention q/k/v decode projection (batches of 1
// or 2 row blocks): 2 when the group's chunks divide and at least kDecMinWg
// work-groups remain, else 1.  (The FFN projection has enough work-groups with
// one column block per wave, and measured slower with more.)
constexpr int kDecMinWg = 192;
static int dec_ncb(int nrb, int groups, int chunks) {
  if (nrb > 2) return 1;
  for (int c : {2})
    if (chunks % c == 0 && groups * (chunks / c) >= kDecMinWg) return c;
  return 1;
}

// nmask_decode instantiation for nrb row blocks and ncb column blocks per wave
template <int MODE, int NW>
static auto nmask_pick(int nrb, int ncb) {
  if (nrb == 1) return ncb == 4 ? nmask_decode<MODE, 1, 4, NW>
                      : ncb == 2 ? nmask_decode<MODE, 1, 2, NW>
                                 : nmask_decode<MODE, 1, 1, NW>;
  if (nrb == 2) return ncb == 4 ? nmask_decode<MODE, 2, 4, 4>
                      : ncb == 2 ? nmask_decode<MODE, 2, 2, 4>
                                 : nmask_decode<MODE, 2, 1, 4>;
  return nrb == 3 ? nmask_decode<MODE, 3, 1, 4> : nmask_decode<MODE, 4, 1, 4>;
}
// waves per work-group of nmask_decode with one row block (each takes d / NW of
// K).  8 and 16 waves (fewer K steps per wave) measured 1-8 us slower on the
// 8B attention and FFN decode workloads than 4.
constexpr int kDecWaves1 = 4;
static int dec_waves(int nrb) { return nrb == 1 ? kDecWaves1 : 4; }

void launch_ffn_decode(const uint16_t* X, const uint8_t* mask, const uint16_t* Wg,
                       const uint16_t* Wu, const uint16_t* Wdp, int B, int d, int F, int n,
                       const uint16_t* residual, uint16_t* H, float* kpart, uint16_t* Y,
                       hipStream_t s) {
  const int G = F / n, chunks = G / 8;
  {
    WIDE_TRACE("ffn_up_decode", s);
    const int nrb = (B + 15) / 16;
    if (!use_cols(nrb, n * (chunks / 4))) {
      const int ncb = 1;
      nmask_pick<kNmFfn, kDecWaves1>(nrb, ncb)<<<n * (chunks / ncb), 64 * dec_waves(nrb), 0, s>>>(
          X, Wg, Wu, nullptr, mask, B, d, G, chunks, 0, DecCache{nullptr, 0, 0, 0}, 0.f, H,
          nullptr, nullptr, n);
    } else {
      auto k = nrb == 2   ? nmask_decode_cols<kNmFfn, 2>
               : nrb == 3 ? nmask_decode_cols<kNmFfn, 3>
                          : nmask_decode_cols<kNmFfn, 4>;
      k<<<n * (chunks / 4), 256, 0, s>>>(X, Wg, Wu, nullptr, mask, B, d, G, chunks, 0, DecCache{nullptr, 0, 0, 0}, 0.f, H,
                                         nullptr, nullptr, n);
    }
  }
  launch_kmask_decode(kUseFfnDown, H, Wdp, mask, B, d, F, n, residual, kpart, Y, s);
}

void launch_kmask_decode(KmUse use, const uint16_t* A, const uint16_t* Wp, const uint8_t* mask,
                         int B, int d, int F, int n, const uint16_t* residual, float* part,
                         uint16_t* Y, hipStream_t s) {
  WIDE_TRACE(use == kUseAttnO ? "attn_o_decode" : "ffn_down_decode", s);
  const int G = F / n, S = kmask_decode_splits(d, n, G), nrb = (B + 15) / 16;
  auto pick = [&](auto use_tag, auto ks_tag) {
    constexpr int U = decltype(use_tag)::value, KS = decltype(ks_tag)::value;
    return nrb == 1   ? kmask_decode<1, KS, U>
           : nrb == 2 ? kmask_decode<2, KS, U>
           : nrb == 3 ? kmask_decode<3, KS, U>
                      : kmask_decode<4, KS, U>;
  };
  using O = std::integral_constant<int, kUseAttnO>;
  using D = std::integral_constant<int, kUseFfnDown>;
  using K4 = std::integral_constant<int, 4>;
  using K2 = std::integral_constant<int, 2>;
  using K1 = std::integral_constant<int, 1>;
  auto k = use == kUseAttnO ? (G % 128 == 0 ? pick(O{}, K4{}) : pick(O{}, K2{}))
           : G % 128 == 0   ? pick(D{}, K4{})
           : G % 64 == 0    ? pick(D{}, K2{})
                            : pick(D{}, K1{});  // groups of 32: 32-wide units
  k<<<kmask_decode_col_blocks(d) * S, kKmThreads, 0, s>>>(A, Wp, mask, B, d, F, G, n, S, residual,
                                                         part, Y);
  if (S > 1) kmask_decode_reduce<<<(B * d / 4 + 255) / 256, 256, 0, s>>>(part, S, B, d, residual, Y);
}

size_t kmask_decode_part_floats(int B, int d, int n, int G) {
  const int S = kmask_decode_splits(d, n, G);
  return S > 1 ? (size_t)S * B * d : 0;
}

int attn_decode_chunks(int kv_len) { return (kv_len + 1 + kKeyChunk - 1) / kKeyChunk; }

void launch_attn_decode(const uint16_t* X, const uint8_t* mask, const uint16_t* Wq,
                        const uint16_t* Wk, const uint16_t* Wv, int B, int d,
                        int n_kv, int r, float rope_theta, uint16_t* Kc, uint16_t* Vc, int kv_len,
                        int kv_cap, const int32_t* kvl, int pos, uint16_t* Qd, float* Opart,
                        float* Mpart, float* Lpart, uint16_t* O, hipStream_t s,
                        const PagedKV* paged) {
  const int chunks = (r + 2) * 8;  // 16-row chunks of the group's q, k, v heads
  const float log2_theta = rope_theta > 0.f ? log2f(rope_theta) : 0.f;
  const DecCache dc{kvl,
                    kv_len,
                    kv_cap,
                    pos,
                    paged ? paged->table : nullptr,
                    paged ? paged->page_shift : 0,
                    paged ? paged->n_pages : 0};
  {
    WIDE_TRACE("attn_qkv_decode", s);
    const int nrb = (B + 15) / 16;
    if (!use_cols(nrb, n_kv * (chunks / 4))) {
      const int ncb = dec_ncb(nrb, n_kv, chunks);
      nmask_pick<kNmQkv, kDecWaves1>(nrb, ncb)<<<n_kv * (chunks / ncb), 64 * dec_waves(nrb), 0, s>>>(
          X, Wq, Wk, Wv, mask, B, d, kHdD, chunks, r, dc, log2_theta, Qd, Kc, Vc, n_kv);
    } else {
      auto k = nrb == 2   ? nmask_decode_cols<kNmQkv, 2>
               : nrb == 3 ? nmask_decode_cols<kNmQkv, 3>
                          : nmask_decode_cols<kNmQkv, 4>;
      k<<<n_kv * (chunks / 4), 256, 0, s>>>(X, Wq, Wk, Wv, mask, B, d, kHdD, chunks, r, dc,
                                            log2_theta, Qd, Kc, Vc, n_kv);
    }
  }
  // chunk grid for the longest possible pair: the batch's length, or with per-pair
  // lengths the last cache slot
  const int nch = attn_decode_chunks(kvl ? kv_cap - 1 : kv_len);
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)kHdD);
  {
    WIDE_TRACE("attn_core_decode", s);
    auto k = paged ? attn_decode_partial<true> : attn_decode_partial<false>;
    k<<<B * n_kv * nch, kKeyChunk, 0, s>>>(Qd, Kc, Vc, mask, B, n_kv, r, dc, nch, scale_log2, Opart,
                                           Mpart, Lpart);
  }
  {
    WIDE_TRACE("attn_combine_decode", s);
    attn_decode_combine<<<B * n_kv * r, kCmbThreads, 0, s>>>(Opart, Mpart, Lpart, mask, n_kv, r,
                                                             dc, nch, O);
  }
}

}  // namespace wide
