// Mask reordering (gist.science technical summary §2.B): per group, a stable
// partition of the tokens into "kept" (a contiguous prefix) and "dropped", plus
// the per-tile union of kept groups that block-level skipping reads (§2.C, l=0).
//
// No host synchronisation; one or two launches:
//   1. reorder_pack   : one wave per token row packs its mask bytes into 64-bit
//                       words by ballot.
//   2. reorder_groups : one work-group per group (chunks of 64 tokens, a ballot
//                       per chunk, a scan over the waves, then each lane places its
//                       token by mbcnt), plus one work-group per token tile for
//                       the tile's union of kept groups.
// When no tile unions are asked for, one launch does both: the group work-groups
// read the mask bytes themselves and further work-groups of the same grid pack the
// words (which later kernels read).
#include "wide.h"
#include "common.h"
#include "gemm_tile.h"
#include "internal.h"

namespace wide {

// Packing: one wave per token row at a time, lane j reading mask byte 64 w + j
// (64 consecutive bytes per load); the ballot of "nonzero" is word w.  A wave
// takes kPackTok rows and issues all of their loads before the first ballot.
constexpr int kPackThreads = 256;
constexpr int kPackWaves = kPackThreads / kWave;
constexpr int kPackTok = 8;

// The kPackTok rows from t0 (one wave).
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

__global__ void __launch_bounds__(kPackThreads)
    reorder_pack(const uint8_t* __restrict__ mask, int T, int n, int nw,
                 uint64_t* __restrict__ packed) {
  const int wave = threadIdx.x / kWave;
  const int t0 = (blockIdx.x * kPackWaves + wave) * kPackTok;
  if (t0 < T) pack_rows(mask, T, n, nw, packed, t0, lane_id());
}

constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / kWave;
constexpr int kGroupMaxChunks = WIDE_MAX_TOKENS / kWave;

// Work-groups 0..n-1: one per group.  The tokens go in chunks of 64 (lane = token);
// wave w takes a contiguous run of chunks.  Pass 1: the ballot of each chunk's
// keep bits (kept in LDS) and the wave's count; a scan over the waves gives each
// wave's kept and dropped tokens before its run.  Pass 2: a kept lane goes to
// (kept before it), a dropped one to count + (dropped before it): mbcnt of the
// ballot inside the chunk, so a wave's stores of a chunk are two contiguous runs.
// Work-groups n..: one per token tile (when tile unions are asked for): the OR of
// the tile's packed words, compacted into an ascending group list, -1 padded.
// mask != nullptr (no tile unions then): the group work-groups read the keep bits
// from the mask bytes, and the work-groups from n on pack the words, kPackTok rows
// per wave.
__global__ void __launch_bounds__(kGroupThreads)
    reorder_groups(const uint8_t* __restrict__ mask, uint64_t* __restrict__ packed, int T, int n,
                   int nw, int tile_m, int32_t* __restrict__ group_count,
                   int32_t* __restrict__ group_perm, int32_t* __restrict__ group_rank,
                   int32_t* __restrict__ tile_count, int32_t* __restrict__ tile_groups) {
  __shared__ int sWave[kGroupWaves];
  __shared__ uint32_t sU[8];
  __shared__ uint64_t sBallot[kGroupMaxChunks];
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  if (mask && (int)blockIdx.x >= n) {
    const int t0 = (((int)blockIdx.x - n) * kGroupWaves + wave) * kPackTok;
    if (t0 < T) pack_rows(mask, T, n, nw, packed, t0, lane);
    return;
  }
  if ((int)blockIdx.x >= n) {
    const int tile = blockIdx.x - n;
    if (threadIdx.x < 8) sU[threadIdx.x] = 0u;
    __syncthreads();
    const int t0 = tile * tile_m, t1 = min(T, t0 + tile_m);
    uint64_t uni[4] = {0, 0, 0, 0};
    for (int t = t0 + (int)threadIdx.x; t < t1; t += kGroupThreads) {
#pragma unroll
      for (int w = 0; w < 4; ++w)
        if (w < nw) uni[w] |= packed[(size_t)t * nw + w];
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
    __syncthreads();
    if (wave == 0) {
      int32_t* out = tile_groups + (size_t)tile * n;
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
      if (lane == 0) tile_count[tile] = written;
    }
    return;
  }
  const int g = blockIdx.x;
  const int w = g >> 6, j = g & 63;
  const int nch = (T + kWave - 1) / kWave;
  const int per = (nch + kGroupWaves - 1) / kGroupWaves;
  const int c0 = min(nch, wave * per), c1 = min(nch, c0 + per);
  const rsrc_t pr = make_rsrc(packed, mask ? 0u : (uint32_t)((size_t)T * nw * 8));
  const rsrc_t mr = make_rsrc(mask, mask ? (uint32_t)((size_t)T * n) : 0u);
  // keep bit of lane's token: bit j of the loaded half word, or the mask byte
  const int shift = mask ? 0 : (j & 31);
  int mine = 0;
  for (int c = c0; c < c1; c += 8) {
    uint32_t v[8];  // the 32-bit half of word w that holds bit j, or the mask byte
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = (c + u) * kWave + lane;
      const bool in = c + u < c1 && t < T;
      v[u] = mask ? ldbuf1(mr, in ? (uint32_t)(t * n + g) : kSkip)
                  : __builtin_amdgcn_raw_buffer_load_b32(
                        pr, in ? (uint32_t)((t * nw + w) * 8 + (j >> 5) * 4) : kSkip, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint64_t b = ballot(mask ? v[u] != 0u : ((v[u] >> shift) & 1u) != 0u);
      if (c + u < c1) {
        if (lane == 0) sBallot[c + u] = b;
        mine += popc64(b);
      }
    }
  }
  if (lane == 0) sWave[wave] = mine;
  __syncthreads();
  int kept = 0, cnt = 0;
  for (int i = 0; i < kGroupWaves; ++i) {
    const int x = sWave[i];
    if (i < wave) kept += x;
    cnt += x;
  }
  int dropped = c0 * kWave - kept;  // tokens before this wave's run that dropped g
  int32_t* perm = group_perm + (size_t)g * T;
  int32_t* rank = group_rank ? group_rank + (size_t)g * T : nullptr;
  for (int c = c0; c < c1; ++c) {
    const uint64_t b = sBallot[c];
    const int t = c * kWave + lane;
    const int valid = min(kWave, T - c * kWave);
    const uint64_t vm = valid == kWave ? ~0ull : ((1ull << valid) - 1ull);
    const uint64_t d = ~b & vm;
    if (t < T) {
      const bool k = (b >> lane) & 1ull;
      const int r = k ? kept + mbcnt(b) : cnt + dropped + mbcnt(d);
      perm[r] = t;
      if (rank) rank[t] = r;
    }
    kept += popc64(b);
    dropped += popc64(d);
  }
  if (threadIdx.x == 0) group_count[g] = cnt;
}

constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / kWave;
constexpr int kSortBins = 256;  // key = the whole mask pattern (n <= 8 groups)
constexpr int kSortMaxTiles = 256;  // tiles ranked for tile_perm (256-token tiles of 65536)

// One work-group; keys (the tokens' 8-bit patterns) are staged in LDS.  Wave w
// owns the contiguous tokens [w c, (w + 1) c) and (1) counts its keys, (2) one
// scan over (key, wave) gives each wave's first slot per key, (3) each wave
// places its tokens in order, 64 at a time; lanes with equal keys are ranked by a
// ballot match.  (4) A tile of the new order covers a run of whole key ranges,
// so its group union is the OR of the keys whose range meets it.  (5) When
// tile_perm is given: the K-masked kernel's XCD x takes the tile slots
// m x .. m x + m - 1 (m = tiles / 8) whenever the tile count is a multiple of 32,
// and a tile's time grows with its union; so the tiles, largest union first,
// are dealt to the XCDs in snake order (XCD x gets ranks x, 15 - x, 16 + x, ...)
// and tile_perm[slot] names the tile of each slot (identity otherwise).
__global__ void __launch_bounds__(kSortThreads)
    reorder_token_sort(const uint64_t* __restrict__ packed, int T, int n, int nw, int tile_m,
                       int32_t* __restrict__ order, int32_t* __restrict__ tile_count,
                       int32_t* __restrict__ tile_groups, int32_t* __restrict__ tile_perm) {
  extern __shared__ uint8_t sKey[];  // [T]
  __shared__ int sHist[kSortWaves][kSortBins];
  __shared__ int sStart[kSortBins + 1];
  __shared__ int sUnion[kSortMaxTiles];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  for (int i = tid; i < kSortWaves * kSortBins; i += kSortThreads) (&sHist[0][0])[i] = 0;
  for (int t0 = 0; t0 < T; t0 += 4 * kSortThreads) {
    uint64_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + u * kSortThreads + tid;
      v[u] = t < T ? packed[(size_t)t * nw] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + u * kSortThreads + tid;
      if (t < T) sKey[t] = (uint8_t)v[u];
    }
  }
  __syncthreads();
  const int per = (T + kSortWaves - 1) / kSortWaves;
  const int c0 = min(T, wave * per), c1 = min(T, c0 + per);
  for (int t = c0 + lane; t < c1; t += kWave) atomicAdd(&sHist[wave][sKey[t]], 1);
  __syncthreads();
  // exclusive scan in (key, wave) order: thread k < 256 owns key k
  if (tid < kSortBins) {
    int run = 0;
    for (int w = 0; w < kSortWaves; ++w) {
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
      order[sStart[key] + sHist[wave][key] + popc64(below)] = t;
      // the last lane of each key bumps the wave's slot for that key
      if ((same >> lane) == 1ull) sHist[wave][key] += popc64(same);
    }
  }
  // tile unions from the key ranges: wave w takes tiles w, w + 16, ...
  const int n_tiles = (T + tile_m - 1) / tile_m;
  for (int tile = wave; tile < n_tiles; tile += kSortWaves) {
    const int p0 = tile * tile_m, p1 = min(T, p0 + tile_m);
    uint32_t u = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = 4 * lane + i;
      const int a = sStart[k], e = sStart[k + 1];
      if (a < e && a < p1 && e > p0) u |= (uint32_t)k;
    }
    for (int off = 32; off >= 1; off >>= 1) u |= __shfl_xor(u, off);
    int32_t* out = tile_groups + (size_t)tile * n;
    const bool has = lane < n && ((u >> lane) & 1u);
    const uint64_t hb = ballot(has);
    if (has) out[popc64(hb & ((1ull << lane) - 1ull))] = lane;
    const int written = popc64(hb);
    for (int q = written + lane; q < n; q += kWave) out[q] = -1;
    if (lane == 0) {
      tile_count[tile] = written;
      if (tile < kSortMaxTiles) sUnion[tile] = written;
    }
  }
  if (!tile_perm) return;
  __syncthreads();
  const bool snake = n_tiles % 32 == 0 && n_tiles <= kSortMaxTiles;
  for (int i = tid; i < n_tiles; i += kSortThreads) {
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
    tile_perm[slot] = i;
  }
}

void launch_token_sort(const uint64_t* packed, int T, int n, int tile_m, int32_t* order,
                       int32_t* tile_count, int32_t* tile_groups, int32_t* tile_perm,
                       hipStream_t s) {
  // the key array may take the whole 64 KB of dynamic LDS next to the static part
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&reorder_token_sort),
      hipFuncAttributeMaxDynamicSharedMemorySize, WIDE_MAX_TOKENS);
  (void)attr;
  WIDE_TRACE("reorder_token_sort", s);
  reorder_token_sort<<<1, kSortThreads, (size_t)T, s>>>(packed, T, n, (n + 63) / 64, tile_m,
                                                        order, tile_count, tile_groups,
                                                        tile_perm);
}

void launch_reorder_packed(const uint64_t* packed, int T, int n, int tile_m,
                           int32_t* group_count, int32_t* group_perm, int32_t* group_rank,
                           int32_t* tile_count, int32_t* tile_groups, hipStream_t s) {
  const int nw = (n + 63) / 64;
  const int n_tiles = tile_count ? (T + tile_m - 1) / tile_m : 0;
  WIDE_TRACE("reorder_groups", s);
  reorder_groups<<<n + n_tiles, kGroupThreads, 0, s>>>(nullptr, const_cast<uint64_t*>(packed), T,
                                                        n, nw, tile_m, group_count, group_perm,
                                                        group_rank, tile_count, tile_groups);
}

void launch_reorder(const uint8_t* mask, int T, int n, int tile_m, uint64_t* packed,
                    int32_t* group_count, int32_t* group_perm, int32_t* group_rank,
                    int32_t* tile_count, int32_t* tile_groups, hipStream_t s) {
  const int nw = (n + 63) / 64;
  if (!tile_count) {  // one launch: groups from the mask bytes, packing beside them
    const int per_block = kGroupWaves * kPackTok;
    WIDE_TRACE("reorder_groups", s);
    reorder_groups<<<n + (T + per_block - 1) / per_block, kGroupThreads, 0, s>>>(
        mask, packed, T, n, nw, tile_m, group_count, group_perm, group_rank, nullptr, nullptr);
    return;
  }
  {
    WIDE_TRACE("reorder_pack", s);
    const int per_block = kPackWaves * kPackTok;
    reorder_pack<<<(T + per_block - 1) / per_block, kPackThreads, 0, s>>>(mask, T, n, nw, packed);
  }
  launch_reorder_packed(packed, T, n, tile_m, group_count, group_perm, group_rank, tile_count,
                        tile_groups, s);
}

}  // namespace wide
