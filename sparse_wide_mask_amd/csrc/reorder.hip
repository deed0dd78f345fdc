// Mask reordering (gist.science technical summary §2.B): per group, a stable
// partition of the tokens into "kept" (a contiguous prefix) and "dropped", plus
// the per-tile union of kept groups that block-level skipping reads (§2.C, l=0).
//
// Two launches, no host synchronisation:
//   1. reorder_pack   : one thread per token packs its mask row into 64-bit words.
//   2. reorder_groups : one work-group per group (each thread owns a run of
//                       consecutive tokens; a wave shuffle scan plus one LDS pass
//                       over the waves gives the kept tokens before each run, and
//                       the thread places its tokens), plus one work-group per
//                       token tile for the tile's union of kept groups.
#include "wide.h"
#include "common.h"
#include "gemm_tile.h"
#include "internal.h"

namespace wide {

// One thread per token: it reads its mask row with 4-byte loads (all issued
// before any is used) and packs the nonzero bytes into 64-bit words.
constexpr int kPackThreads = 256;

template <bool ALIGNED4>
__global__ void __launch_bounds__(kPackThreads)
    reorder_pack(const uint8_t* __restrict__ mask, int T, int n, int nw,
                 uint64_t* __restrict__ packed) {
  const int t = blockIdx.x * kPackThreads + threadIdx.x;
  if (t >= T) return;
  const rsrc_t mr = make_rsrc(mask, (uint32_t)((size_t)T * n));
  const uint32_t row = (uint32_t)((size_t)t * n);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w >= nw) break;
    uint64_t word = 0;
    if (ALIGNED4) {
      uint32_t v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int b = 64 * w + 4 * u;
        v[u] = b < n ? __builtin_amdgcn_raw_buffer_load_b32(mr, (int)(row + b), 0, 0) : 0u;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          word |= (uint64_t)(((v[u] >> (8 * k)) & 0xffu) != 0u) << (4 * u + k);
    } else {
      uint32_t v[64];
#pragma unroll
      for (int u = 0; u < 64; ++u) {
        const int b = 64 * w + u;
        v[u] = b < n ? ldbuf1(mr, row + b) : 0u;
      }
#pragma unroll
      for (int u = 0; u < 64; ++u) word |= (uint64_t)(v[u] != 0u) << u;
    }
    packed[(size_t)t * nw + w] = word;
  }
}

constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / kWave;

// Work-groups 0..n-1: one per group.  Thread i owns the contiguous tokens
// [i*per, (i+1)*per), per <= 64: it loads their mask bits once into a register
// bitmask, one work-group exclusive scan of the kept counts gives the number
// kept before its run, and it places its tokens: kept ones at (#kept before t),
// dropped ones at cnt + (#dropped before t).
// Work-groups n..: one per token tile (when tile unions are asked for): the OR of
// the tile's packed words, compacted into an ascending group list, -1 padded.
__global__ void __launch_bounds__(kGroupThreads)
    reorder_groups(const uint64_t* __restrict__ packed, int T, int n, int nw, int tile_m,
                   int32_t* __restrict__ group_count, int32_t* __restrict__ group_perm,
                   int32_t* __restrict__ group_rank, int32_t* __restrict__ tile_count,
                   int32_t* __restrict__ tile_groups) {
  __shared__ int sWave[kGroupWaves];
  __shared__ uint32_t sU[8];
  const int lane = lane_id(), wave = threadIdx.x / kWave;
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
  const int per = (T + kGroupThreads - 1) / kGroupThreads;
  const int t0 = min(T, (int)threadIdx.x * per), t1 = min(T, t0 + per);
  uint64_t bits = 0;
  for (int c = 0; c < t1 - t0; c += 8) {
    uint64_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = t0 + c + u;
      v[u] = t < t1 ? packed[(size_t)t * nw + w] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) bits |= ((v[u] >> j) & 1ull) << (c + u);
  }
  const int mine = popc64(bits);
  // inclusive scan inside the wave, then across the 16 waves
  int incl = mine;
  for (int off = 1; off < kWave; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == kWave - 1) sWave[wave] = incl;
  __syncthreads();
  int before = incl - mine, cnt = 0;
  for (int i = 0; i < kGroupWaves; ++i) {
    const int v = sWave[i];
    if (i < wave) before += v;
    cnt += v;
  }
  int32_t* perm = group_perm + (size_t)g * T;
  int32_t* rank = group_rank ? group_rank + (size_t)g * T : nullptr;
  for (int i = 0; i < t1 - t0; ++i) {
    const int t = t0 + i;
    const bool bit = (bits >> i) & 1ull;
    const int r = bit ? before : cnt + (t - before);
    before += bit;
    if (rank) rank[t] = r;
    perm[r] = t;
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

void launch_reorder(const uint8_t* mask, int T, int n, int tile_m, uint64_t* packed,
                    int32_t* group_count, int32_t* group_perm, int32_t* group_rank,
                    int32_t* tile_count, int32_t* tile_groups, hipStream_t s) {
  const int nw = (n + 63) / 64;
  const int n_tiles = tile_count ? (T + tile_m - 1) / tile_m : 0;
  {
    WIDE_TRACE("reorder_pack", s);
    const int grid = (T + kPackThreads - 1) / kPackThreads;
    if (n % 4 == 0)
      reorder_pack<true><<<grid, kPackThreads, 0, s>>>(mask, T, n, nw, packed);
    else
      reorder_pack<false><<<grid, kPackThreads, 0, s>>>(mask, T, n, nw, packed);
  }
  {
    WIDE_TRACE("reorder_groups", s);
    reorder_groups<<<n + n_tiles, kGroupThreads, 0, s>>>(packed, T, n, nw, tile_m, group_count,
                                                          group_perm, group_rank, tile_count,
                                                          tile_groups);
  }
}

}  // namespace wide
