// Block-tile bf16 MFMA engine shared by the prefill GEMMs.
//
// A work-group of 512 threads (8 waves, 4 x 2, two per SIMD) owns a BM x BN
// output tile and walks K in slices of BK = 64; each wave holds a 64 x 128
// accumulator and issues v_mfma_f32_32x32x16_bf16.  Two waves per SIMD let one
// wave's LDS reads and waits overlap the other's MFMAs.
//
// Global -> LDS uses buffer loads that write LDS directly (no VGPR staging).  Two
// LDS stages: slice kt+1 loads while slice kt computes (variants: three stages for
// tiles that leave room, and two A stages with three B stages).  One load instruction of
// a wave fills 8 rows of 128 bytes (a whole cache line per row); 16 rows of 64
// bytes per instruction, as 32-wide slices give, is about 3x slower from L2.  A
// lane whose buffer offset is past num_records reads zeros without touching
// memory: that is how rows of tokens that dropped a group are skipped at the load
// stage.  Before a stage is read, every wave waits for its own loads (vmcnt) and
// then meets the others at a barrier.
//
// Measured on a dense 8192 x 8192 x 4096 GEMM: 1.60-1.65 PFLOP/s (4 waves of
// 128 x 128 with 32-wide slices and 4 stages: 1.25-1.31).
//
// LDS layout of a slice: rows of 64 bf16 (128 bytes = 8 chunks of 16 bytes);
// chunk c of row r sits in slot c ^ swz(r), swz(r) = (r mod 8) ^ ((r >> 3) mod 4),
// which keeps the 16-byte fragment reads of consecutive rows free of bank
// conflicts for both 32- and 64-bank LDS organisations.
#pragma once

#include "common.h"

namespace wide {

constexpr int kBK = 64;
constexpr int kStages = 2;
constexpr uint32_t kSkip = 0x7fffff00u;  // buffer offset past any num_records: zeros
// Cache policy of the large outputs' buffer stores: non-temporal (the next
// kernel reads them back from memory anyway).  Fewer dirty L2 lines are left
// to write back when a kernel ends: about 24 us less per 8B layer prefill step.
constexpr int kNtStore = 2;

typedef __amdgpu_buffer_rsrc_t rsrc_t;

WIDE_DEV rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
WIDE_DEV u32x4 ldbuf16(rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0);
}
// One byte; an offset past num_records reads 0.
WIDE_DEV uint32_t ldbuf1(rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)byte_off, 0, 0);
}
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint16_t lds_u16;

// Buffer descriptor as four scalar dwords (base, stride 0, num_records, format).
WIDE_DEV i32x4 make_srd(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return i32x4{(int32_t)(uint32_t)p, (int32_t)(uint32_t)(p >> 32), (int32_t)bytes, 0x00020000};
}
// LDS byte address of a pointer into __shared__ memory.
WIDE_DEV uint32_t lds_addr(const uint16_t* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((lds_u16*)(p));
}
// 16 bytes per lane from the buffer straight into LDS: lane l lands at
// lds + 16 l (lds is wave-uniform).  Written as asm so the compiler does not
// track the LDS write: the K loop orders it explicitly (vmcnt wait + barrier
// before a stage is read, barrier before a stage is refilled).
WIDE_DEV void lds_dma16(i32x4 srd, uint32_t lds, uint32_t byte_off) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(byte_off), "s"(srd)
               : "memory", "m0");
}
// depends on row mod 32 only, so a fragment read can use its row inside a 32-row block
WIDE_DEV int swz(int row) { return (row & 7) ^ ((row >> 3) & 3); }
WIDE_DEV bf16x8 lds_frag(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Wait until at most N of this wave's buffer loads are in flight (and its LDS
// reads are done), then barrier.
template <int N>
WIDE_DEV void stage_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Barrier once this wave's LDS reads are done (buffer loads may stay in flight).
WIDE_DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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

constexpr int kGemmWM = 4, kGemmWN = 2;  // waves along M and N
constexpr int kGemmThreads = 64 * kGemmWM * kGemmWN;

template <int BM, int BN, int NWM = kGemmWM, int NWN = kGemmWN>
struct TileCfg {
  static constexpr int kWaves = NWM * NWN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int WM = BM / NWM, WN = BN / NWN;   // per-wave tile
  static constexpr int RB = WM / 32, CB = WN / 32; // 32x32 MFMA blocks per wave
  // buffer->LDS instructions per thread and slice: one instruction of a wave
  // fills 16 rows (1 KB); the 4 waves share the rows of the tile.
  static constexpr int A_INST = BM / (8 * kWaves);
  static constexpr int B_INST = BN / (8 * kWaves);
  static constexpr int LOADS = A_INST + B_INST;
  static constexpr int SA = BM * kBK;  // elements per stage
  static constexpr int SB = BN * kBK;
  static constexpr uint32_t kAllRows = (1u << RB) - 1u;
  static_assert(WM % 32 == 0 && WN % 32 == 0 && BM % (8 * kWaves) == 0 && BN % (8 * kWaves) == 0, "tile shape");
};

// Row of the tile filled by lane `lane` of wave `wave` in its instruction q, and
// the logical 16-byte chunk that lane fetches for the swizzled layout.
template <int NW = kGemmWM * kGemmWN>
WIDE_DEV int dma_row(int wave, int q, int lane) { return 8 * (NW * q + wave) + (lane >> 3); }
// the logical chunk fetched by `lane` for tile row `row` (its slot is lane & 7)
WIDE_DEV int dma_chunk(int row, int lane) { return (lane & 7) ^ swz(row); }
template <int NW = kGemmWM * kGemmWN>
WIDE_DEV uint32_t dma_dst(uint32_t stage_addr, int wave, int q) {
  return stage_addr + 8 * (NW * q + wave) * kBK * 2;
}

// Accumulators of one wave and its pipelined K loop.
template <int BM, int BN, int NWM = kGemmWM, int NWN = kGemmWN>
struct WaveAcc {
  using C = TileCfg<BM, BN, NWM, NWN>;
  f32x16 acc[C::RB][C::CB];

  // fragments of one 16-wide K step: RB A blocks and CB B blocks
  struct Frags {
    bf16x8 a[C::RB], b[C::CB];
  };

  WIDE_DEV void zero() {
#pragma unroll
    for (int i = 0; i < C::RB; ++i)
#pragma unroll
      for (int j = 0; j < C::CB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  }

  WIDE_DEV static void read(Frags& f, const uint16_t* sA, const uint16_t* sB, int wm, int wn,
                            int lane, int ks) {
    const int r = lane & 31, slot = ((2 * ks + (lane >> 5)) ^ swz(r)) * 8;
    const uint16_t* pa = sA + (wm * C::WM + r) * kBK + slot;
    const uint16_t* pb = sB + (wn * C::WN + r) * kBK + slot;
#pragma unroll
    for (int i = 0; i < C::RB; ++i) f.a[i] = lds_frag(pa + i * 32 * kBK);
#pragma unroll
    for (int j = 0; j < C::CB; ++j) f.b[j] = lds_frag(pb + j * 32 * kBK);
  }

  // rb_live bit i = row block i of this wave has live rows; the other blocks skip
  // their MFMAs (intra-block skipping at the MMA stage).
  template <bool ALL>
  WIDE_DEV void mma(const Frags& f, uint32_t rb_live) {
#pragma unroll
    for (int i = 0; i < C::RB; ++i) {
      if (!ALL && !((rb_live >> i) & 1u)) continue;
#pragma unroll
      for (int j = 0; j < C::CB; ++j) acc[i][j] = mfma32(f.a[i], f.b[j], acc[i][j]);
    }
  }

  // Two stages of 64-wide slices: slice kt+1 loads while slice kt computes.
  template <bool ALL, int LOADS, class Issue, class Live>
  WIDE_DEV void run(int nk, const uint16_t* sA, const uint16_t* sB, int wm, int wn, int lane,
                    Issue&& issue, Live&& live) {
    if (nk <= 0) return;
    issue(0, 0);
    stage_barrier<0>();
    Frags lo, hi;
    read(lo, sA, sB, wm, wn, lane, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const int st = kt & 1;
      const uint32_t lv = ALL ? C::kAllRows : live(kt);
      const uint16_t* cA = sA + st * C::SA;
      const uint16_t* cB = sB + st * C::SB;
      if (kt + 1 < nk) issue(kt + 1, st ^ 1);
      read(hi, cA, cB, wm, wn, lane, 1);
      __builtin_amdgcn_sched_barrier(0);
      mma<ALL>(lo, lv);
      __builtin_amdgcn_sched_barrier(0);
      read(lo, cA, cB, wm, wn, lane, 2);
      __builtin_amdgcn_sched_barrier(0);
      mma<ALL>(hi, lv);
      __builtin_amdgcn_sched_barrier(0);
      read(hi, cA, cB, wm, wn, lane, 3);
      __builtin_amdgcn_sched_barrier(0);
      mma<ALL>(lo, lv);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 1 < nk) {
        stage_barrier<0>();
        read(lo, sA + (st ^ 1) * C::SA, sB + (st ^ 1) * C::SB, wm, wn, lane, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      mma<ALL>(hi, lv);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Two A stages and three B stages (at 256 x 256 exactly the 160 KB of LDS):
  // slice kt+1's A rows and slice kt+2's B rows load while slice kt computes, so
  // the B stream has two slices of lead.  A stage of slice kt = kt mod 2, B stage
  // = kt mod 3; both refill stages that slice kt-1 used.  Per slice a wave issues
  // its A loads before its B loads, so waiting for vmcnt <= BLOADS before slice
  // kt+1 leaves only slice kt+2's B loads in flight.
  template <bool ALL, int BLOADS, class IssueA, class IssueB, class Live>
  WIDE_DEV void run_a2b3(int nk, const uint16_t* sA, const uint16_t* sB, int wm, int wn,
                         int lane, IssueA&& issueA, IssueB&& issueB, Live&& live) {
    if (nk <= 0) return;
    issueA(0, 0);
    issueB(0, 0);
    if (nk > 1) {
      issueB(1, 1);
      stage_barrier<BLOADS>();
    } else {
      stage_barrier<0>();
    }
    Frags lo, hi;
    read(lo, sA, sB, wm, wn, lane, 0);
    int sb = 0;
    for (int kt = 0; kt < nk; ++kt) {
      const int sa = kt & 1;
      const uint32_t lv = ALL ? C::kAllRows : live(kt);
      const uint16_t* cA = sA + sa * C::SA;
      const uint16_t* cB = sB + sb * C::SB;
      const int sb1 = sb == 2 ? 0 : sb + 1, sb2 = sb1 == 2 ? 0 : sb1 + 1;
      if (kt + 1 < nk) issueA(kt + 1, sa ^ 1);
      if (kt + 2 < nk) issueB(kt + 2, sb2);
      read(hi, cA, cB, wm, wn, lane, 1);
      __builtin_amdgcn_sched_barrier(0);
      mma<ALL>(lo, lv);
      __builtin_amdgcn_sched_barrier(0);
      read(lo, cA, cB, wm, wn, lane, 2);
      __builtin_amdgcn_sched_barrier(0);
      mma<ALL>(hi, lv);
      __builtin_amdgcn_sched_barrier(0);
      read(hi, cA, cB, wm, wn, lane, 3);
      __builtin_amdgcn_sched_barrier(0);
      mma<ALL>(lo, lv);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 1 < nk) {
        if (kt + 2 < nk)
          stage_barrier<BLOADS>();
        else
          stage_barrier<0>();
        read(lo, sA + (sa ^ 1) * C::SA, sB + sb1 * C::SB, wm, wn, lane, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      mma<ALL>(hi, lv);
      __builtin_amdgcn_sched_barrier(0);
      sb = sb1;
    }
  }

  // Three stages: slices kt+1 and kt+2 load while slice kt computes (for tiles
  // whose few rows leave room in LDS, so that streaming B has more loads in
  // flight).  Stage of slice kt = kt mod 3; slice kt+2 refills the stage that
  // slice kt-1 used, whose reads all waves finished before the last barrier.
  template <bool ALL, int LOADS, class Issue, class Live>
  WIDE_DEV void run3(int nk, const uint16_t* sA, const uint16_t* sB, int wm, int wn, int lane,
                     Issue&& issue, Live&& live) {
    if (nk <= 0) return;
    issue(0, 0);
    if (nk > 1) {
      issue(1, 1);
      stage_barrier<LOADS>();
    } else {
      stage_barrier<0>();
    }
    Frags lo, hi;
    read(lo, sA, sB, wm, wn, lane, 0);
    int st = 0;
    for (int kt = 0; kt < nk; ++kt) {
      const uint32_t lv = ALL ? C::kAllRows : live(kt);
      const uint16_t* cA = sA + st * C::SA;
      const uint16_t* cB = sB + st * C::SB;
      const int st1 = st == 2 ? 0 : st + 1, st2 = st1 == 2 ? 0 : st1 + 1;
      if (kt + 2 < nk) issue(kt + 2, st2);
      read(hi, cA, cB, wm, wn, lane, 1);
      __builtin_amdgcn_sched_barrier(0);
      mma<ALL>(lo, lv);
      __builtin_amdgcn_sched_barrier(0);
      read(lo, cA, cB, wm, wn, lane, 2);
      __builtin_amdgcn_sched_barrier(0);
      mma<ALL>(hi, lv);
      __builtin_amdgcn_sched_barrier(0);
      read(hi, cA, cB, wm, wn, lane, 3);
      __builtin_amdgcn_sched_barrier(0);
      mma<ALL>(lo, lv);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 1 < nk) {
        // slice kt+1 has landed (slice kt+2 may stay in flight)
        if (kt + 2 < nk)
          stage_barrier<LOADS>();
        else
          stage_barrier<0>();
        read(lo, sA + st1 * C::SA, sB + st1 * C::SB, wm, wn, lane, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      mma<ALL>(hi, lv);
      __builtin_amdgcn_sched_barrier(0);
      st = st1;
    }
  }
};

}  // namespace wide
