// Mask reordering (gist.science technical summary §2.B): per group, a stable
// partition of the tokens into "kept" (a contiguous prefix) and "dropped", plus
// the per-tile union of kept groups that block-level skipping reads (§2.C, l=0),
// the mask's packed bit words, and for few groups a token order sorted by the
// whole mask pattern.
//
// Everything for one or two masks runs in one launch of 1024-thread work-groups,
// each taking one role (no host synchronisation, no dependencies inside the
// launch: every role reads the mask bytes, or the packed words when those are the
// input; a mask of more than 4 MB is packed by a launch of its own first):
//   sort    one work-group per sorted mask: a stable counting sort of the tokens
//           by their pattern (n <= 8) and the unions of tiles of that order; with
//           more groups by the pattern of the first 8, without unions;
//   groups  one per group: chunks of 64 tokens (lane = token), a ballot per chunk,
//           a scan over the waves, then each lane places its token by mbcnt;
//   unions  one per token tile: the OR of the tile's keep bits, compacted into an
//           ascending group list, -1 padded;
//   pack    one per 128 tokens: the mask's little-endian 64-bit words by ballot;
//   norm    four token rows of the layer's first RMSNorm (a layer call folds it
//           into this launch, so the reorders run beside it on one stream).
#include "wide.h"
#include "common.h"
#include "gemm_tile.h"
#include "internal.h"
#include "norm_row.h"

#include <algorithm>

namespace wide {

constexpr int kRoThreads = 1024;
constexpr int kRoWaves = kRoThreads / kWave;
constexpr int kPackTok = 8;                          // rows per wave of a pack work-group
constexpr int kPackPerWg = kRoWaves * kPackTok;      // 128
constexpr int kNormPerWg = kRoThreads / 256;         // 4 rows per norm work-group
constexpr int kSortBins = 256;                       // key = the whole pattern (n <= 8)
constexpr int kSortMaxTiles = 256;                   // tiles ranked for tile_perm

// ------------------------------------------------------------------ roles

// Packing: one wave per token row at a time, lane j reading mask byte 64 w + j
// (64 consecutive bytes per load); the ballot of "nonzero" is word w.  The kPackTok
// rows from t0 (one wave); all loads are issued before the first ballot.
WIDE_DEV void pack_rows(const uint8_t* __restrict__ mask, int T, int n, int nw,
                        uint64_t* __restrict__ packed, int t0, int lane) {
  const rsrc_t mr = make_rsrc(mask, (uint32_t)((size_t)T * n));
  uint32_t v[kPackTok][4];
#pragma unroll
  for (int k = 0; k < kPackTok; ++k)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int t = t0 + k, g = 64 * w + lane;
      v[k][w] = ldbuf1(mr, t < T && g < n ? (uint32_t)(t * n + g) : kSkip);
    }
#pragma unroll
  for (int k = 0; k < kPackTok; ++k)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint64_t word = ballot(v[k][w] != 0u);
      if (lane == 0 && w < nw && t0 + k < T) packed[(size_t)(t0 + k) * nw + w] = word;
    }
}

// Group g's stable partition.  Wave w takes a contiguous run of 64-token chunks.
// Pass 1: the ballot of each chunk's keep bits (kept in LDS) and the wave's count;
// a scan over the waves gives each wave's kept and dropped tokens before its run.
// Pass 2: a kept lane goes to (kept before it), a dropped one to count + (dropped
// before it): mbcnt of the ballot inside the chunk, so a wave's stores of a chunk
// are two contiguous runs.  Keep bits come from the mask bytes, or from bit j of
// the packed words.
WIDE_DEV void group_partition(const MaskJob& J, int T, int g, uint64_t* sBallot, int* sWave) {
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int n = J.n, nw = J.nw, w = g >> 6, j = g & 63;
  const int nch = (T + kWave - 1) / kWave;
  const int per = (nch + kRoWaves - 1) / kRoWaves;
  const int c0 = min(nch, wave * per), c1 = min(nch, c0 + per);
  const bool bytes = J.mask != nullptr;
  const rsrc_t pr = make_rsrc(J.packed, bytes ? 0u : (uint32_t)((size_t)T * nw * 8));
  const rsrc_t mr = make_rsrc(J.mask, bytes ? (uint32_t)((size_t)T * n) : 0u);
  const int shift = bytes ? 0 : (j & 31);
  int mine = 0;
  for (int c = c0; c < c1; c += 8) {
    uint32_t v[8];  // the mask byte, or the 32-bit half of word w that holds bit j
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = (c + u) * kWave + lane;
      const bool in = c + u < c1 && t < T;
      v[u] = bytes ? ldbuf1(mr, in ? (uint32_t)(t * n + g) : kSkip)
                   : __builtin_amdgcn_raw_buffer_load_b32(
                         pr, in ? (uint32_t)((t * nw + w) * 8 + (j >> 5) * 4) : kSkip, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint64_t b = ballot(bytes ? v[u] != 0u : ((v[u] >> shift) & 1u) != 0u);
      if (c + u < c1) {
        if (lane == 0) sBallot[c + u] = b;
        mine += popc64(b);
      }
    }
  }
  if (lane == 0) sWave[wave] = mine;
  __syncthreads();
  int kept = 0, cnt = 0;
  for (int i = 0; i < kRoWaves; ++i) {
    const int x = sWave[i];
    if (i < wave) kept += x;
    cnt += x;
  }
  int dropped = c0 * kWave - kept;  // tokens before this wave's run that dropped g
  int32_t* perm = J.perm + (size_t)g * T;
  int32_t* rank = J.rank ? J.rank + (size_t)g * T : nullptr;
  for (int c = c0; c < c1; ++c) {
    const uint64_t b = sBallot[c];
    const int t = c * kWave + lane;
    const int valid = min(kWave, T - c * kWave);
    const uint64_t vm = valid == kWave ? ~0ull : ((1ull << valid) - 1ull);
    const uint64_t dmask = ~b & vm;
    if (t < T) {
      const bool k = (b >> lane) & 1ull;
      const int r = k ? kept + mbcnt(b) : cnt + dropped + mbcnt(dmask);
      perm[r] = t;
      if (rank) rank[t] = r;
    }
    kept += popc64(b);
    dropped += popc64(dmask);
  }
  if (threadIdx.x == 0) J.count[g] = cnt;
}

// The group union of tile `tile` (tile_m consecutive tokens).  From the bytes:
// wave w takes rows w, w + 16, ...; lane holds groups lane + 64 i; a ballot per
// word, OR-ed over the waves in LDS.  From the packed words: the OR of the rows'
// words.  Then wave 0 compacts the union into an ascending list, -1 padded.
WIDE_DEV void tile_union(const MaskJob& J, int T, int tile, uint32_t* sU) {
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int n = J.n, nw = J.nw;
  if (threadIdx.x < 8) sU[threadIdx.x] = 0u;
  __syncthreads();
  const int t0 = tile * J.tile_m, t1 = min(T, t0 + J.tile_m);
  if (J.mask) {
    const rsrc_t mr = make_rsrc(J.mask, (uint32_t)((size_t)T * n));
    bool any[4] = {false, false, false, false};
    for (int r0 = t0 + wave; r0 < t1; r0 += 8 * kRoWaves) {
      uint32_t v[8][4];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int t = r0 + u * kRoWaves;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int g = 64 * w + lane;
          v[u][w] = ldbuf1(mr, t < t1 && g < n ? (uint32_t)(t * n + g) : kSkip);
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) any[w] = any[w] || v[u][w] != 0u;
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint64_t word = ballot(any[w]);
      if (lane == 0 && w < nw && word) {
        if ((uint32_t)word) atomicOr(&sU[2 * w], (uint32_t)word);
        if ((uint32_t)(word >> 32)) atomicOr(&sU[2 * w + 1], (uint32_t)(word >> 32));
      }
    }
  } else {
    uint64_t uni[4] = {0, 0, 0, 0};
    for (int t = t0 + (int)threadIdx.x; t < t1; t += kRoThreads) {
#pragma unroll
      for (int w = 0; w < 4; ++w)
        if (w < nw) uni[w] |= J.packed[(size_t)t * nw + w];
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t lo = (uint32_t)uni[w], hi = (uint32_t)(uni[w] >> 32);
      for (int off = 32; off >= 1; off >>= 1) lo |= __shfl_xor(lo, off), hi |= __shfl_xor(hi, off);
      if (lane == 0 && w < nw) {
        if (lo) atomicOr(&sU[2 * w], lo);
        if (hi) atomicOr(&sU[2 * w + 1], hi);
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    int32_t* out = J.tile_groups + (size_t)tile * n;
    int written = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (w >= nw) break;
      const uint64_t u = ((uint64_t)sU[2 * w + 1] << 32) | sU[2 * w];
      const int g = 64 * w + lane;
      if (g < n && ((u >> lane) & 1ull)) out[written + popc64(u & ((1ull << lane) - 1ull))] = g;
      written += popc64(u);
    }
    for (int p = written + lane; p < n; p += kWave) out[p] = -1;
    if (lane == 0) J.tile_count[tile] = written;
  }
}

// Stable counting sort of the tokens by their whole pattern (n <= 8, pattern <
// 256; with more groups, by the pattern of the first 8), patterns taken in
// reflected Gray-code order: the key of pattern p is its
// rank k with k ^ (k >> 1) = p, so the patterns of neighbouring key ranges differ
// in few groups and a tile that spans several ranges keeps a smaller union (top-4
// of 8 groups at T = 8192: 5.66 instead of 6.16 groups per 256-token tile on
// average, at most 7 instead of 8).  Keys staged in LDS (sKey [T]).  Wave w owns
// the contiguous tokens [w c, (w+1) c) and (1) counts its keys, (2) one scan over
// (key, wave) gives each wave's first slot per key, (3) each wave places its
// tokens in order, 64 at a time; lanes with equal keys are ranked by a ballot
// match.  (4) A tile of the new order covers a run of whole key ranges, so its
// group union is the OR of the patterns whose range meets it.  (5) When tile_perm is given: the K-masked kernel's XCD x takes the
// tile slots m x .. m x + m - 1 (m = tiles / 8) whenever the tile count is a
// multiple of 32, and a tile's time grows with its union; so the tiles, largest
// union first, are dealt to the XCDs in snake order (XCD x gets ranks x, 15 - x,
// 16 + x, ...) and tile_perm[slot] names the tile of each slot (identity otherwise).
WIDE_DEV void token_sort(const MaskJob& J, int T, uint8_t* sKey, int (*sHist)[kSortBins],
                         int* sStart, int* sUnion) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int n = J.n;
  for (int i = tid; i < kRoWaves * kSortBins; i += kRoThreads) (&sHist[0][0])[i] = 0;
  // keys: bit g = (mask byte g != 0), or the low byte of the first packed word
  const rsrc_t mr = make_rsrc(J.mask, J.mask ? (uint32_t)((size_t)T * n) : 0u);
  for (int t0 = 0; t0 < T; t0 += 4 * kRoThreads) {
    uint32_t key[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + u * kRoThreads + tid;
      key[u] = 0u;
      if (J.mask && n % 8 == 0) {
        // the first 8 bytes of the row in one load (rows start 8-byte aligned)
        const uint32_t off = t < T ? (uint32_t)(t * n) : kSkip;
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b32(mr, (int)off, 0, 0);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b32(mr, (int)(off + 4u), 0, 0);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          key[u] |= (((lo >> (8 * g)) & 0xffu) != 0u ? 1u : 0u) << g;
          key[u] |= (((hi >> (8 * g)) & 0xffu) != 0u ? 1u : 0u) << (g + 4);
        }
      } else if (J.mask) {
        uint32_t b[8];
#pragma unroll
        for (int g = 0; g < 8; ++g) b[g] = ldbuf1(mr, t < T && g < n ? (uint32_t)(t * n + g) : kSkip);
#pragma unroll
        for (int g = 0; g < 8; ++g) key[u] |= (b[g] != 0u ? 1u : 0u) << g;
      } else if (t < T) {
        key[u] = (uint32_t)(J.packed[(size_t)t * J.nw] & 0xffull);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + u * kRoThreads + tid;
      uint32_t k = key[u];  // pattern -> its Gray-code rank
      k ^= k >> 1;
      k ^= k >> 2;
      k ^= k >> 4;
      if (t < T) sKey[t] = (uint8_t)k;
    }
  }
  __syncthreads();
  const int per = (T + kRoWaves - 1) / kRoWaves;
  const int c0 = min(T, wave * per), c1 = min(T, c0 + per);
  for (int t = c0 + lane; t < c1; t += kWave) atomicAdd(&sHist[wave][sKey[t]], 1);
  __syncthreads();
  // exclusive scan in (key, wave) order: thread k < 256 owns key k
  if (tid < kSortBins) {
    int run = 0;
    for (int w = 0; w < kRoWaves; ++w) {
      const int v = sHist[w][tid];
      sHist[w][tid] = run;
      run += v;
    }
    sStart[tid] = run;
  }
  __syncthreads();
  if (wave == 0) {  // scan of the per-key totals, 4 keys per lane
    int v[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = sStart[4 * lane + i], sum += v[i];
    int incl = sum;
    for (int off = 1; off < kWave; off <<= 1) {
      const int u = __shfl_up(incl, off);
      if (lane >= off) incl += u;
    }
    int base = incl - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) sStart[4 * lane + i] = base, base += v[i];
    if (lane == kWave - 1) sStart[kSortBins] = incl;
  }
  __syncthreads();
  for (int t0 = c0; t0 < c1; t0 += kWave) {
    const int t = t0 + lane;
    const bool ok = t < c1;
    const int key = ok ? sKey[t] : -1;
    uint64_t same = ballot(ok);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t ones = ballot(ok && ((key >> b) & 1));
      same &= ((key >> b) & 1) ? ones : ~ones;
    }
    if (ok) {
      const uint64_t below = same & ((1ull << lane) - 1ull);
      J.order[sStart[key] + sHist[wave][key] + popc64(below)] = t;
      // the last lane of each key bumps the wave's slot for that key
      if ((same >> lane) == 1ull) sHist[wave][key] += popc64(same);
    }
  }
  // More than 8 groups: the key is the pattern of the first 8 only, so a key range
  // does not give its tokens' union; the K-masked GEMM that runs over this order
  // ORs the mask words of its tile's rows itself (tile_count / tile_groups null).
  if (n > kSortMaxGroups || !J.tile_groups) return;
  // tile unions from the key ranges: wave w takes tiles w, w + 16, ...
  const int n_tiles = (T + J.tile_m - 1) / J.tile_m;
  for (int tile = wave; tile < n_tiles; tile += kRoWaves) {
    const int p0 = tile * J.tile_m, p1 = min(T, p0 + J.tile_m);
    uint32_t u = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = 4 * lane + i;
      const int a = sStart[k], e = sStart[k + 1];
      if (a < e && a < p1 && e > p0) u |= (uint32_t)(k ^ (k >> 1));
    }
    for (int off = 32; off >= 1; off >>= 1) u |= __shfl_xor(u, off);
    int32_t* out = J.tile_groups + (size_t)tile * n;
    const bool has = lane < n && ((u >> lane) & 1u);
    const uint64_t hb = ballot(has);
    if (has) out[popc64(hb & ((1ull << lane) - 1ull))] = lane;
    const int written = popc64(hb);
    for (int q = written + lane; q < n; q += kWave) out[q] = -1;
    if (lane == 0) {
      J.tile_count[tile] = written;
      if (tile < kSortMaxTiles) sUnion[tile] = written;
    }
  }
  if (!J.tile_perm) return;
  __syncthreads();
  const bool snake = n_tiles % 32 == 0 && n_tiles <= kSortMaxTiles;
  for (int i = tid; i < n_tiles; i += kRoThreads) {
    int slot = i;
    if (snake) {
      const int u = sUnion[i];
      int rank = 0;  // position among the tiles by union, descending (ties by index)
      for (int k = 0; k < n_tiles; ++k) {
        const int v = sUnion[k];
        rank += (v > u || (v == u && k < i)) ? 1 : 0;
      }
      const int round = rank >> 3, pos = rank & 7;
      const int x = (round & 1) ? 7 - pos : pos;
      slot = (n_tiles >> 3) * x + round;
    }
    J.tile_perm[slot] = i;
  }
}

// Norm rows 4 w .. 4 w + 3, 256 threads each.  Every thread of the work-group
// passes the same barriers, so a row past T computes on row T - 1 and does not
// store.
WIDE_DEV void norm_rows(const NormJob& nm, int T, int w, float* sRed) {
  const int quarter = threadIdx.x >> 8;
  const int row = kNormPerWg * w + quarter;
  const int rr = min(row, T - 1);
  rms_row(nm.x + (size_t)rr * nm.d, nm.gamma, nm.d, nm.eps,
          row < T ? nm.y + (size_t)rr * nm.d : nullptr, threadIdx.x & 255, sRed + 4 * quarter);
}

// ------------------------------------------------------------------ the launch

// Work-group counts of the roles, in grid order: the sorts (the longest single
// work-groups) first, then the norm rows (most of the launch's memory traffic),
// then the short group, union and pack work-groups, which fill the compute units
// as the norm rows drain.
struct RoGrid {
  int sort[2], groups[2], unions[2], pack[2], norm;  // norm: after the sorts
};

// Dynamic LDS of the launch: the largest role present.
struct RoLds {
  static constexpr size_t align16(size_t x) { return (x + 15) / 16 * 16; }
  static size_t sort(int T) {
    return align16((size_t)T) + sizeof(int) * ((size_t)kRoWaves * kSortBins + kSortBins + 1 + kSortMaxTiles) + 16;
  }
  static size_t groups(int T) { return 64 * sizeof(int) + 8 * (size_t)((T + kWave - 1) / kWave); }
};

// Runs f(r) when r falls in the next segment of `count` work-groups; else steps r
// past it.
template <class F>
WIDE_DEV bool segment(int& r, int count, F&& f) {
  if (r < count) {
    f(r);
    return true;
  }
  r -= count;
  return false;
}

// Two work-groups per compute unit (8 waves per SIMD): the norm rows need the
// memory parallelism of a full CU.
__global__ void __launch_bounds__(kRoThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
    reorder_all(MaskJob a, MaskJob b, NormJob nm, int T, RoGrid grid) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int r = blockIdx.x;
  uint8_t* sKey = smem;
  int(*sHist)[kSortBins] = reinterpret_cast<int(*)[kSortBins]>(smem + RoLds::align16(T));
  int* sStart = &sHist[kRoWaves][0];
  int* sUnion = sStart + kSortBins + 1;
  uint64_t* sBallot = reinterpret_cast<uint64_t*>(smem + 64 * sizeof(int));
  int* sWave = reinterpret_cast<int*>(smem);
  uint32_t* sU = reinterpret_cast<uint32_t*>(smem);
  const int t0p = (int)threadIdx.x / kWave * kPackTok;  // this wave's first row of a pack unit
  if (segment(r, grid.sort[0], [&](int) { token_sort(a, T, sKey, sHist, sStart, sUnion); }) ||
      segment(r, grid.sort[1], [&](int) { token_sort(b, T, sKey, sHist, sStart, sUnion); }) ||
      segment(r, grid.norm, [&](int w) { norm_rows(nm, T, w, reinterpret_cast<float*>(smem)); }) ||
      segment(r, grid.groups[0], [&](int g) { group_partition(a, T, g, sBallot, sWave); }) ||
      segment(r, grid.groups[1], [&](int g) { group_partition(b, T, g, sBallot, sWave); }) ||
      segment(r, grid.unions[0], [&](int t) { tile_union(a, T, t, sU); }) ||
      segment(r, grid.unions[1], [&](int t) { tile_union(b, T, t, sU); }) ||
      segment(r, grid.pack[0], [&](int p) {
        const int t0 = p * kPackPerWg + t0p;
        if (t0 < T) pack_rows(a.mask, T, a.n, a.nw, a.packed, t0, lane_id());
      }) ||
      segment(r, grid.pack[1], [&](int p) {
        const int t0 = p * kPackPerWg + t0p;
        if (t0 < T) pack_rows(b.mask, T, b.n, b.nw, b.packed, t0, lane_id());
      }))
    return;
}

// Masks of more bytes than this (an XCD's L2) are packed by a launch of their own
// first (see launch_reorder_jobs).
constexpr size_t kBytesMaxMask = size_t(4) << 20;

static RoGrid ro_grid(int T, const MaskJob* const (&J)[2], const NormJob* norm, bool pack_only,
                      size_t& lds) {
  RoGrid g{};
  lds = 64;
  for (int q = 0; q < 2; ++q) {
    const MaskJob* j = J[q];
    if (!j) continue;
    g.pack[q] = j->mask ? (T + kPackPerWg - 1) / kPackPerWg : 0;
    if (pack_only) continue;
    const bool sort = j->order != nullptr;
    g.sort[q] = sort ? 1 : 0;
    g.groups[q] = j->n;
    g.unions[q] = (!sort && j->tile_count) ? (T + j->tile_m - 1) / j->tile_m : 0;
    if (sort) lds = std::max(lds, RoLds::sort(T));
    lds = std::max(lds, RoLds::groups(T));
  }
  g.norm = norm && !pack_only ? (T + kNormPerWg - 1) / kNormPerWg : 0;
  return g;
}

static int ro_blocks(const RoGrid& g) {
  return g.sort[0] + g.sort[1] + g.groups[0] + g.groups[1] + g.unions[0] + g.unions[1] +
         g.pack[0] + g.pack[1] + g.norm;
}

void launch_reorder_jobs(int T, const MaskJob* a, const MaskJob* b, const NormJob* norm,
                         hipStream_t s) {
  if (T <= 0) return;
  // the sort's keys may take the whole 64 KB of tokens next to its tables
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&reorder_all), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)RoLds::sort(WIDE_MAX_TOKENS));
  (void)attr;
  // The roles read the mask bytes (or the packed words when those are the input).
  // A group's work-group reads one byte per token at a stride of n bytes, so the
  // 112 groups of the 8B FFN pull the 0.9 MB mask through L2 about 100 times,
  // which costs the launch ≈7 us beside the norm rows; packing it in a launch of
  // its own first took ≈11 us.  A mask larger than an XCD's L2 would be re-read
  // from beyond it by every group, so such a mask is still packed first and the
  // roles of the main launch read its words.
  const MaskJob none{};
  MaskJob local[2];
  const MaskJob* J[2] = {a, b};
  const MaskJob* P[2] = {nullptr, nullptr};  // jobs packed first
  for (int q = 0; q < 2; ++q)
    if (J[q] && J[q]->mask && (size_t)T * J[q]->n > kBytesMaxMask) {
      P[q] = J[q];
      local[q] = *J[q];
      local[q].mask = nullptr;  // the main launch reads the packed words
      J[q] = &local[q];
    }
  size_t lds = 0;
  if (P[0] || P[1]) {
    WIDE_TRACE("reorder_pack", s);
    const RoGrid g = ro_grid(T, P, nullptr, true, lds);
    reorder_all<<<ro_blocks(g), kRoThreads, lds, s>>>(P[0] ? *P[0] : none, P[1] ? *P[1] : none,
                                                      NormJob{}, T, g);
  }
  const RoGrid g = ro_grid(T, J, norm, false, lds);
  WIDE_TRACE(norm ? "norm_reorder" : "reorder", s);
  reorder_all<<<ro_blocks(g), kRoThreads, lds, s>>>(J[0] ? *J[0] : none, J[1] ? *J[1] : none,
                                                    norm ? *norm : NormJob{}, T, g);
}

void launch_reorder(const uint8_t* mask, int T, int n, int tile_m, uint64_t* packed,
                    int32_t* group_count, int32_t* group_perm, int32_t* group_rank,
                    int32_t* tile_count, int32_t* tile_groups, hipStream_t s) {
  const MaskJob j{mask, packed, n, (n + 63) / 64, tile_m, group_count, group_perm, group_rank,
                  tile_count, tile_groups, nullptr, nullptr};
  launch_reorder_jobs(T, &j, nullptr, nullptr, s);
}

void launch_reorder_packed(const uint64_t* packed, int T, int n, int tile_m,
                           int32_t* group_count, int32_t* group_perm, int32_t* group_rank,
                           int32_t* tile_count, int32_t* tile_groups, hipStream_t s) {
  const MaskJob j{nullptr, const_cast<uint64_t*>(packed), n, (n + 63) / 64, tile_m, group_count,
                  group_perm, group_rank, tile_count, tile_groups, nullptr, nullptr};
  launch_reorder_jobs(T, &j, nullptr, nullptr, s);
}

}  // namespace wide
