// Block-tile bf16 MFMA engine shared by the prefill GEMMs.
//
// A workgroup of 256 threads (4 waves, 2 x 2) owns a BM x BN output tile and
// walks K in steps of BK = 64.  Both operands are K-contiguous in global memory
// (activations row-major over d_model, weights as nn.Linear rows or as packed
// K-major group blocks), so each lane moves 16-byte chunks and each wave feeds
// v_mfma_f32_32x32x16_bf16 from padded LDS rows with 16-byte reads.
//
// Global operands are read with raw buffer loads: a lane whose offset lies past
// the buffer's num_records gets zeros without touching memory.  That is how rows
// of tokens that dropped a group are skipped at load time (intra-block skipping
// at the load stage) without a branch.  LDS is double-buffered: the loads of
// step k+1 are issued before the MFMAs of step k and land in the other buffer,
// so each K step needs one barrier.
#pragma once

#include "common.h"

namespace wide {

constexpr int kBK = 64;
constexpr int kLdsLd = kBK + 8;  // LDS row pitch in bf16 (144 bytes: 16-byte aligned, skewed banks)
constexpr int kSkip = 0x7fffff00;  // buffer offset past any num_records: load returns zeros

typedef __amdgpu_buffer_rsrc_t rsrc_t;

WIDE_DEV rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
WIDE_DEV u32x4 ldbuf16(rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}
WIDE_DEV u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
WIDE_DEV void st16(uint16_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
WIDE_DEV bf16x8 lds_frag(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Block rasterisation of a rows x cols tile grid: stripes of MB tile rows; inside
// a stripe, blocks of CBk tile columns with the row index fastest.  Consecutive
// l form an MB x CBk block whose A rows and B columns are shared, so the ~32
// work-groups an XCD runs at once read each operand slice from its L2 once.
WIDE_DEV void block_raster(int l, int rows, int cols, int MB, int CBk, int& r, int& c) {
  const int per_stripe = MB * cols;
  const int s = l / per_stripe;
  const int r0 = s * MB, mh = min(MB, rows - r0);
  const int rem = l - s * per_stripe;
  const int cb = rem / (mh * CBk);
  const int r2 = rem - cb * mh * CBk;
  r = r0 + r2 % mh;
  c = cb * CBk + r2 / mh;
}

template <int BM, int BN>
struct TileCfg {
  static constexpr int kThreads = 256;
  static constexpr int WM = BM / 2, WN = BN / 2;   // per-wave tile
  static constexpr int RB = WM / 32, CB = WN / 32; // 32x32 MFMA blocks per wave
  static constexpr int A_CHUNKS = BM * kBK / 8 / kThreads;
  static constexpr int B_CHUNKS = BN * kBK / 8 / kThreads;
  static constexpr int LDS_A = BM * kLdsLd;
  static constexpr int LDS_B = BN * kLdsLd;
  static constexpr uint32_t kAllRows = (1u << RB) - 1u;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be whole 32x32 blocks");
  static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1, "tile too small for 256 threads");
};

// Accumulators of one wave and the MFMA sweep over one BK slice held in LDS.
template <int BM, int BN>
struct WaveAcc {
  using C = TileCfg<BM, BN>;
  f32x16 acc[C::RB][C::CB];

  WIDE_DEV void zero() {
#pragma unroll
    for (int i = 0; i < C::RB; ++i)
#pragma unroll
      for (int j = 0; j < C::CB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  }

  // Every row block live: fragments of slice ks+1 are read while slice ks multiplies.
  WIDE_DEV void sweep_full(const uint16_t* sA, const uint16_t* sB, int wm, int wn, int lane) {
    const int r = lane & 31, kh = (lane >> 5) * 8;
    const uint16_t* pa = sA + (wm * C::WM + r) * kLdsLd + kh;
    const uint16_t* pb = sB + (wn * C::WN + r) * kLdsLd + kh;
    bf16x8 a[2][C::RB], b[2][C::CB];
#pragma unroll
    for (int i = 0; i < C::RB; ++i) a[0][i] = lds_frag(pa + i * 32 * kLdsLd);
#pragma unroll
    for (int j = 0; j < C::CB; ++j) b[0][j] = lds_frag(pb + j * 32 * kLdsLd);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int cur = ks & 1, nxt = cur ^ 1;
      if (ks + 1 < kBK / 16) {
#pragma unroll
        for (int i = 0; i < C::RB; ++i) a[nxt][i] = lds_frag(pa + i * 32 * kLdsLd + (ks + 1) * 16);
#pragma unroll
        for (int j = 0; j < C::CB; ++j) b[nxt][j] = lds_frag(pb + j * 32 * kLdsLd + (ks + 1) * 16);
      }
      // keep the reads of slice ks+1 ahead of the MFMAs of slice ks
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < C::RB; ++i)
#pragma unroll
        for (int j = 0; j < C::CB; ++j) acc[i][j] = mfma32(a[cur][i], b[cur][j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Some row blocks may hold no live row: their MFMAs are skipped (intra-block
  // skipping at the MMA stage).  rb_live bit i = row block i has work.  Fragments
  // of slice ks+1 are read before the MFMAs of slice ks, as in sweep_full.
  WIDE_DEV void sweep_masked(const uint16_t* sA, const uint16_t* sB, int wm, int wn, int lane,
                             uint32_t rb_live) {
    const int r = lane & 31, kh = (lane >> 5) * 8;
    const uint16_t* pa = sA + (wm * C::WM + r) * kLdsLd + kh;
    const uint16_t* pb = sB + (wn * C::WN + r) * kLdsLd + kh;
    bf16x8 a[2][C::RB], b[2][C::CB];
#pragma unroll
    for (int i = 0; i < C::RB; ++i) a[0][i] = lds_frag(pa + i * 32 * kLdsLd);
#pragma unroll
    for (int j = 0; j < C::CB; ++j) b[0][j] = lds_frag(pb + j * 32 * kLdsLd);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int cur = ks & 1, nxt = cur ^ 1;
      if (ks + 1 < kBK / 16) {
#pragma unroll
        for (int i = 0; i < C::RB; ++i) a[nxt][i] = lds_frag(pa + i * 32 * kLdsLd + (ks + 1) * 16);
#pragma unroll
        for (int j = 0; j < C::CB; ++j) b[nxt][j] = lds_frag(pb + j * 32 * kLdsLd + (ks + 1) * 16);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < C::RB; ++i) {
        if (!((rb_live >> i) & 1u)) continue;
#pragma unroll
        for (int j = 0; j < C::CB; ++j) acc[i][j] = mfma32(a[cur][i], b[cur][j], acc[i][j]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

};

}  // namespace wide
