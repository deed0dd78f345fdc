// Block-tile bf16 MFMA engine shared by the prefill GEMMs.
//
// A workgroup of 256 threads (4 waves, 2 x 2) owns a BM x BN output tile and
// walks K in steps of BK = 64.  Both operands are K-contiguous in global memory
// (activations row-major over d_model, weights as nn.Linear rows or as packed
// K-major group blocks), so each lane moves 16-byte chunks and each wave feeds
// v_mfma_f32_32x32x16_bf16 from padded LDS rows with 16-byte reads.  Global
// loads for step k+1 are issued into registers before the MFMAs of step k.
#pragma once

#include "common.h"

namespace wide {

constexpr int kBK = 64;
constexpr int kLdsLd = kBK + 8;  // LDS row pitch in bf16 (144 bytes: 16-byte aligned, skewed banks)

WIDE_DEV u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
WIDE_DEV void st16(uint16_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
WIDE_DEV bf16x8 lds_frag(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

template <int BM, int BN>
struct TileCfg {
  static constexpr int kThreads = 256;
  static constexpr int WM = BM / 2, WN = BN / 2;   // per-wave tile
  static constexpr int RB = WM / 32, CB = WN / 32; // 32x32 MFMA blocks per wave
  static constexpr int A_CHUNKS = BM * kBK / 8 / kThreads;
  static constexpr int B_CHUNKS = BN * kBK / 8 / kThreads;
  static constexpr int LDS_A = BM * kLdsLd;
  static constexpr int LDS_B = BN * kLdsLd;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be whole 32x32 blocks");
  static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1, "tile too small for 256 threads");
};

// Accumulators of one wave and the MFMA sweep over one BK slice held in LDS.
// Row blocks starting at or beyond `row_limit` (tile-relative) are skipped: their
// A rows are known to be empty (intra-block MMA skipping).
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

  // rb_live: bit rb set when row block rb of this wave has work.
  WIDE_DEV void sweep(const uint16_t* sA, const uint16_t* sB, int wm, int wn, int lane,
                      uint32_t rb_live) {
    const int r = lane & 31, kh = (lane >> 5) * 8;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8 a[C::RB], b[C::CB];
#pragma unroll
      for (int i = 0; i < C::RB; ++i)
        a[i] = lds_frag(sA + (wm * C::WM + i * 32 + r) * kLdsLd + ks * 16 + kh);
#pragma unroll
      for (int j = 0; j < C::CB; ++j)
        b[j] = lds_frag(sB + (wn * C::WN + j * 32 + r) * kLdsLd + ks * 16 + kh);
#pragma unroll
      for (int i = 0; i < C::RB; ++i) {
        if (!((rb_live >> i) & 1u)) continue;
#pragma unroll
        for (int j = 0; j < C::CB; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
      }
    }
  }
};

}  // namespace wide
