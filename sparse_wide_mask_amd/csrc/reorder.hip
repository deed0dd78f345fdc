// Mask reordering (gist.science technical summary §2.B): per group, a stable
// partition of the tokens into "kept" (a contiguous prefix) and "dropped", plus
// the per-tile union of kept groups that block-level skipping reads (§2.C, l=0).
//
// Three launches, no host synchronisation:
//   1. reorder_pack   : one thread per token packs its mask row into 64-bit words.
//   2. reorder_groups : one workgroup per group; a wave ballot gives each token's
//                       kept bit, mbcnt its rank inside the wave, an LDS scan over
//                       the waves the rank inside the workgroup; a running carry
//                       walks the token axis.  Two passes: count, then place.
//   3. reorder_tiles  : one wave per token tile ORs the packed rows and compacts
//                       the set bits into an ascending group list.
#include "common.h"
#include "internal.h"

namespace wide {

__global__ void __launch_bounds__(256) reorder_pack(const uint8_t* __restrict__ mask, int T, int n,
                                                    int nw, uint64_t* __restrict__ packed) {
  int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const uint8_t* row = mask + (size_t)t * n;
  for (int w = 0; w < nw; ++w) {
    uint64_t word = 0;
    int gend = min(n, 64 * w + 64);
    for (int g = 64 * w; g < gend; ++g) word |= (uint64_t)(row[g] != 0) << (g - 64 * w);
    packed[(size_t)t * nw + w] = word;
  }
}

constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / kWave;

// Exclusive scan of one int per wave (up to 16 waves); returns this wave's offset
// and writes the total to *total.  All threads must call it.
__device__ int wave_offsets(int wave_count, int* s_scan, int* total) {
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  if (lane == 0) s_scan[wave] = wave_count;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < kGroupWaves; ++w) {
      int c = s_scan[w];
      s_scan[w] = acc;
      acc += c;
    }
    s_scan[kGroupWaves] = acc;
  }
  __syncthreads();
  int off = s_scan[wave];
  *total = s_scan[kGroupWaves];
  __syncthreads();
  return off;
}

__global__ void __launch_bounds__(kGroupThreads)
    reorder_groups(const uint64_t* __restrict__ packed, int T, int n, int nw,
                   int32_t* __restrict__ group_count, int32_t* __restrict__ group_perm,
                   int32_t* __restrict__ group_rank) {
  __shared__ int s_scan[kGroupWaves + 1];
  const int g = blockIdx.x;
  const int w = g >> 6, j = g & 63;
  const int lane = lane_id();

  // pass 1: number of tokens that keep g
  int cnt = 0;
  for (int base = 0; base < T; base += kGroupThreads) {
    int t = base + threadIdx.x;
    bool bit = t < T && ((packed[(size_t)t * nw + w] >> j) & 1ull);
    int wc = popc64(ballot(bit));
    int tot;
    wave_offsets(wc, s_scan, &tot);
    cnt += tot;
  }

  // pass 2: kept tokens go to position (#kept before t); dropped ones to
  // cnt + (#dropped before t) = cnt + t - (#kept before t).
  int carry = 0;
  int32_t* perm = group_perm + (size_t)g * T;
  int32_t* rank = group_rank ? group_rank + (size_t)g * T : nullptr;
  for (int base = 0; base < T; base += kGroupThreads) {
    int t = base + threadIdx.x;
    bool bit = t < T && ((packed[(size_t)t * nw + w] >> j) & 1ull);
    uint64_t word = ballot(bit);
    int tot;
    int woff = wave_offsets(popc64(word), s_scan, &tot);
    if (t < T) {
      int before = carry + woff + mbcnt(word);
      int r = bit ? before : cnt + (t - before);
      if (group_rank) rank[t] = r;
      perm[r] = t;
    }
    carry += tot;
  }
  if (threadIdx.x == 0) group_count[g] = cnt;
  (void)lane;
}

__global__ void __launch_bounds__(256) reorder_tiles(const uint64_t* __restrict__ packed, int T,
                                                     int n, int nw, int tile_m, int n_tiles,
                                                     int32_t* __restrict__ tile_count,
                                                     int32_t* __restrict__ tile_groups) {
  const int tile = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (tile >= n_tiles) return;
  const int lane = lane_id();
  const int t0 = tile * tile_m, t1 = min(T, t0 + tile_m);
  int32_t* out = tile_groups + (size_t)tile * n;
  int written = 0;
  for (int w = 0; w < nw; ++w) {
    uint64_t u = 0;
    for (int t = t0 + lane; t < t1; t += kWave) u |= packed[(size_t)t * nw + w];
    // OR-reduce the 64-bit word across the wave
    uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
    for (int off = 32; off >= 1; off >>= 1) {
      lo |= __shfl_xor(lo, off);
      hi |= __shfl_xor(hi, off);
    }
    u = ((uint64_t)hi << 32) | lo;
    int g = 64 * w + lane;
    if (g < n && ((u >> lane) & 1ull)) {
      uint64_t below = lane ? (u & ((1ull << lane) - 1ull)) : 0ull;
      out[written + popc64(below)] = g;
    }
    written += popc64(u);
  }
  for (int p = written + lane; p < n; p += kWave) out[p] = -1;
  if (lane == 0) tile_count[tile] = written;
}

void launch_reorder(const uint8_t* mask, int T, int n, int tile_m, uint64_t* packed,
                    int32_t* group_count, int32_t* group_perm, int32_t* group_rank,
                    int32_t* tile_count, int32_t* tile_groups, hipStream_t s) {
  const int nw = (n + 63) / 64;
  {
    WIDE_TRACE("reorder_pack", s);
    reorder_pack<<<(T + 255) / 256, 256, 0, s>>>(mask, T, n, nw, packed);
  }
  {
    WIDE_TRACE("reorder_groups", s);
    reorder_groups<<<n, kGroupThreads, 0, s>>>(packed, T, n, nw, group_count, group_perm,
                                                group_rank);
  }
  if (tile_count && tile_groups) {
    const int n_tiles = (T + tile_m - 1) / tile_m;
    {
      WIDE_TRACE("reorder_tiles", s);
      reorder_tiles<<<(n_tiles + 3) / 4, 256, 0, s>>>(packed, T, n, nw, tile_m, n_tiles,
                                                      tile_count, tile_groups);
    }
  }
}

}  // namespace wide
