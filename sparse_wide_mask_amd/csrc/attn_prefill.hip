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
//                   Vt [n_kv][hd][T] (row i = i-th kept token of the group).
// attn_core_prefill one work-group = (group, 64 compacted queries), one wave per
//                   query head.  S^T = K Q^T puts a query in each lane's column,
//                   so the online softmax is per lane (+ one cross-half swap) and
//                   P stays in registers as the B operand of O^T = V^T P^T; V is
//                   read in the key order the S^T accumulator layout gives.
//                   Output O is written token-major [T, n_q*hd] at the kept
//                   (token, group) blocks only.
// The O projection is the K-masked GEMM of the FFN down projection with group
// depth r*hd (see ffn_prefill.hip).
#include "common.h"
#include "gemm_tile.h"
#include "internal.h"

namespace wide {

constexpr int kHd = 128;

// ------------------------------------------------------------- QKV projection

__global__ void __launch_bounds__(256, 1)
    attn_qkv_prefill(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wq,
                     const uint16_t* __restrict__ Wk, const uint16_t* __restrict__ Wv,
                     const int32_t* __restrict__ gcount, const int32_t* __restrict__ gperm, int T,
                     int d, int n_kv, int r, int mtiles, int vtp, float log2_theta,
                     uint16_t* __restrict__ Qc, uint16_t* __restrict__ Kc,
                     uint16_t* __restrict__ Vt) {
  constexpr int BM = 256, BN = 256;
  using C = TileCfg<BM, BN>;
  __shared__ __attribute__((aligned(16))) uint16_t sA[kStages * C::SA];
  __shared__ __attribute__((aligned(16))) uint16_t sB[kStages * C::SB];
  const uint32_t ldsA = lds_addr(sA), ldsB = lds_addr(sB);
  __shared__ int sTok[BM];

  const int ntn = (r + 1) / 2 + 1;  // q tiles (2 heads each) + one k|v tile
  int g, mt, nt;
  {
    int c;
    if ((n_kv & 7) == 0) {
      block_raster(blockIdx.x >> 3, mtiles, (n_kv >> 3) * ntn, 4, 8, mt, c);
      g = (blockIdx.x & 7) + 8 * (c / ntn);
    } else {
      block_raster(blockIdx.x, mtiles, n_kv * ntn, 4, 8, mt, c);
      g = c / ntn;
    }
    nt = c % ntn;
  }
  const int cnt = gcount[g];
  const int row0 = mt * BM;
  if (row0 >= cnt) return;  // l=0
  const int rows = min(BM, cnt - row0);
  const bool kv_tile = nt == ntn - 1;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  for (int i = tid; i < BM; i += C::kThreads) sTok[i] = i < rows ? gperm[(size_t)g * T + row0 + i] : -1;
  __syncthreads();

  const int chunk8 = dma_chunk(lane) * 8;
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
  // B row of the tile: q tile -> Wq row g*r*hd + nt*256 + row; k|v tile -> Wk row
  // g*hd + row (row < 128: instructions q = 0, 1) or Wv row g*hd + row - 128.
  uint32_t bOff[C::B_INST];
#pragma unroll
  for (int q = 0; q < C::B_INST; ++q) {
    const int row = dma_row(wave, q, lane);
    const int wrow = kv_tile ? g * kHd + (row & (kHd - 1)) : g * r * kHd + nt * BN + row;
    bOff[q] = (uint32_t)(wrow * d + chunk8) * 2u;
  }
  auto issue = [&](int kt, int st) {
    const uint32_t a = ldsA + st * C::SA * 2, b = ldsB + st * C::SB * 2;
    const uint32_t kb = (uint32_t)kt * kBK * 2u;
#pragma unroll
    for (int q = 0; q < C::A_INST; ++q) lds_dma16(rX, dma_dst(a, wave, q), aOff[q] + kb);
    if (kv_tile) {
#pragma unroll
      for (int q = 0; q < C::B_INST; ++q)
        lds_dma16(q < C::B_INST / 2 ? rK : rV, dma_dst(b, wave, q), bOff[q] + kb);
    } else {
#pragma unroll
      for (int q = 0; q < C::B_INST; ++q) lds_dma16(rQ, dma_dst(b, wave, q), bOff[q] + kb);
    }
  };
  uint32_t rb_live = 0;
#pragma unroll
  for (int i = 0; i < C::RB; ++i)
    if (wm * C::WM + i * 32 < rows) rb_live |= 1u << i;

  WaveAcc<BM, BN> acc;
  acc.zero();
  const int nk = d / kBK;
  auto live = [&](int) { return rb_live; };
  if (rb_live == C::kAllRows)
    acc.template run<true, C::LOADS>(nk, sA, sB, wm, wn, lane, issue, live);
  else
    acc.template run<false, C::LOADS>(nk, sA, sB, wm, wn, lane, issue, live);

  // epilogue.  This wave's 128 columns are one head: q head 2*nt + wn, or k / v.
  // (With an odd head ratio the last q tile's second half reads zeros or the next
  // group's rows and is not written.)
  if (!kv_tile && 2 * nt + wn >= r) return;
  const bool is_v = kv_tile && wn == 1;
  const bool rope = log2_theta > 0.f && !is_v;
  const int c0 = lane & 31;
  float inv0 = 0.f, inv1 = 0.f;  // theta^(-2j/hd) for j = c0 and c0 + 32
  if (rope) {
    inv0 = exp2f(-(2.f * c0 / kHd) * log2_theta);
    inv1 = exp2f(-(2.f * (c0 + 32) / kHd) * log2_theta);
  }
  uint16_t* qdst = Qc + ((size_t)(g * r + 2 * nt + wn) * T) * kHd;
  uint16_t* kdst = Kc + (size_t)g * T * kHd;
  uint16_t* vdst = Vt + (size_t)g * kHd * vtp;
#pragma unroll
  for (int i = 0; i < C::RB; ++i) {
    if (!((rb_live >> i) & 1u)) continue;
    if (is_v) {
      // V^T: lane holds hd column cb*32 + c0 and rows 4 (l/32) + 8 q + {0..3}
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int rr = wm * C::WM + i * 32 + 8 * q4 + 4 * (lane >> 5);
          const f32x16& a = acc.acc[i][cb];
          const uint32_t lo = pack_bf2(a[4 * q4], a[4 * q4 + 1]);
          const uint32_t hi = pack_bf2(a[4 * q4 + 2], a[4 * q4 + 3]);
          uint16_t* p = vdst + (size_t)(cb * 32 + c0) * vtp + row0 + rr;
          if (rr + 3 < rows) {
            *reinterpret_cast<u32x2*>(p) = u32x2{lo, hi};
          } else {
            const uint16_t v4[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi,
                                    (uint16_t)(hi >> 16)};
            for (int k = 0; k < 4; ++k)
              if (rr + k < rows) p[k] = v4[k];
          }
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
        const float pos = (float)sTok[row];
        float s0, co0, s1, co1;
        sincosf(pos * inv0, &s0, &co0);
        sincosf(pos * inv1, &s1, &co1);
        const float r0 = v0 * co0 - v2 * s0, r2 = v2 * co0 + v0 * s0;
        const float r1 = v1 * co1 - v3 * s1, r3 = v3 * co1 + v1 * s1;
        v0 = r0, v1 = r1, v2 = r2, v3 = r3;
      }
      uint16_t* p = (kv_tile ? kdst : qdst) + (size_t)(row0 + row) * kHd + c0;
      p[0] = f2bf(v0);
      p[32] = f2bf(v1);
      p[64] = f2bf(v2);
      p[96] = f2bf(v3);
    }
  }
}

// ---------------------------------------------------------- attention core

constexpr int kBQ = 64;     // queries per work-group (per wave: one head, 64 queries)
constexpr int kBKey = 64;   // keys per step
constexpr int kKPitch = kHd + 8;    // LDS pitch of K rows   (bf16)
constexpr int kVPitch = kBKey + 8;  // LDS pitch of V^T rows (bf16)

WIDE_DEV bf16x8 lds8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
WIDE_DEV bf16x4 lds4(const uint16_t* p) { return *reinterpret_cast<const bf16x4*>(p); }

__global__ void __launch_bounds__(256, 1)
    attn_core_prefill(const uint16_t* __restrict__ Qc, const uint16_t* __restrict__ Kc,
                      const uint16_t* __restrict__ Vt, const int32_t* __restrict__ gcount,
                      const int32_t* __restrict__ gperm, int T, int n_kv, int r, int qtiles,
                      int vtp, float scale_log2, uint16_t* __restrict__ O) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[kBKey * kKPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kHd * kVPitch];

  // work-group -> (group, query tile, chunk of 4 query heads); late (heavy) query
  // tiles first
  const int g = blockIdx.x % n_kv;
  const int rest = blockIdx.x / n_kv;
  const int qt = qtiles - 1 - rest % qtiles;
  const int hc = rest / qtiles;
  const int cnt = gcount[g];
  const int q0 = qt * kBQ;
  if (q0 >= cnt) return;  // l=0
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool head_ok = hc * 4 + wave < r;  // waves past the group's heads only help load
  const int h = g * r + min(hc * 4 + wave, r - 1);
  const int c0 = lane & 31, half = lane >> 5;

  // Q^T fragments as B operands: lane holds query q0 + qb*32 + c0, hd 16 ks + 8 half.
  bf16x8 qf[2][8];
  const uint16_t* qbase = Qc + (size_t)h * T * kHd;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int q = q0 + qb * 32 + c0;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (q < cnt)
        qf[qb][ks] = *reinterpret_cast<const bf16x8*>(qbase + (size_t)q * kHd + ks * 16 + half * 8);
      else
        qf[qb][ks] = bf16x8{};
    }
  }
  f32x16 o[4][2];  // O^T: 4 hd blocks x 2 query blocks
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[a][b][e] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  const uint16_t* kbase = Kc + (size_t)g * T * kHd;
  const uint16_t* vbase = Vt + (size_t)g * kHd * vtp;
  const int q_last = min(cnt, q0 + kBQ) - 1;
  const int nkb = q_last / kBKey + 1;
  for (int kb = 0; kb < nkb; ++kb) {
    const int k0 = kb * kBKey;
    __syncthreads();
    // K block [64 keys][128]: 1024 16-byte chunks, 4 per thread
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + 256 * i, row = ch >> 4, col = (ch & 15) * 8;
      u32x4 v = {0, 0, 0, 0};
      if (k0 + row < cnt) v = *reinterpret_cast<const u32x4*>(kbase + (size_t)(k0 + row) * kHd + col);
      *reinterpret_cast<u32x4*>(sK + row * kKPitch + col) = v;
    }
    // V^T block [128 hd][64 keys]: 1024 chunks of 8 keys, keys >= cnt zeroed
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + 256 * i, row = ch >> 3, col = (ch & 7) * 8;
      u32x4 v = {0, 0, 0, 0};
      const int key = k0 + col;
      if (key < cnt) {
        v = *reinterpret_cast<const u32x4*>(vbase + (size_t)row * vtp + key);
        if (key + 8 > cnt) {
          uint16_t* e = reinterpret_cast<uint16_t*>(&v);
          for (int k = cnt - key; k < 8; ++k) e[k] = 0;
        }
      }
      *reinterpret_cast<u32x4*>(sV + row * kVPitch + col) = v;
    }
    __syncthreads();

    // S^T [64 keys x 64 queries] = K Q^T
    f32x16 s[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[a][b][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const bf16x8 kf = lds8(sK + (a * 32 + c0) * kKPitch + ks * 16 + half * 8);
#pragma unroll
        for (int b = 0; b < 2; ++b) s[a][b] = mfma32(kf, qf[b][ks], s[a][b]);
      }
    }
    // mask (causal in compacted order, keys past the count) and online softmax
    const bool diag = k0 + kBKey > q0;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int q = q0 + b * 32 + c0;
      float mx = -INFINITY;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + a * 32 + acc32_row(lane, e);
          float v = s[a][b][e] * scale_log2;
          if (diag && key > q) v = -INFINITY;
          if (key >= cnt) v = -INFINITY;
          s[a][b][e] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[b], mx);
      // a query past the count has no finite score; keep its state finite
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float corr = exp2f(m_run[b] - m_use);
      float sum = 0.f;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = exp2f(s[a][b][e] - m_use);
          s[a][b][e] = p;
          sum += p;
        }
      sum += __shfl_xor(sum, 32);
      l_run[b] = l_run[b] * corr + sum;
      m_run[b] = m_new;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[a][b][e] *= corr;
    }
    // O^T [128 x 64] += V^T [128 x 64 keys] P^T [64 keys x 64 q]; the k-slots of a
    // lane are the keys its S^T registers hold: 16 s' + 4 half + {0..3, 8..11}.
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        bf16x8 pf[2];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int k = 0; k < 8; ++k) pf[b][k] = (__bf16)s[a][b][8 * sp + k];
        const int key0 = a * 32 + 16 * sp + 4 * half;
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
          const uint16_t* vp = sV + (hb * 32 + c0) * kVPitch + key0;
          const bf16x4 lo = lds4(vp), hi = lds4(vp + 8);
          const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int b = 0; b < 2; ++b) o[hb][b] = mfma32(vf, pf[b], o[hb][b]);
        }
      }
  }

  // O[token, h*hd + j] = O^T[j][q] / l
  if (!head_ok) return;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int q = q0 + b * 32 + c0;
    if (q >= cnt) continue;
    const int tok = gperm[(size_t)g * T + q];
    const float inv = 1.f / l_run[b];
    uint16_t* dst = O + (size_t)tok * (n_kv * r * kHd) + h * kHd;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int j = hb * 32 + 8 * q4 + 4 * half;
        const f32x16& a = o[hb][b];
        const uint32_t lo = pack_bf2(a[4 * q4] * inv, a[4 * q4 + 1] * inv);
        const uint32_t hi = pack_bf2(a[4 * q4 + 2] * inv, a[4 * q4 + 3] * inv);
        *reinterpret_cast<u32x2*>(dst + j) = u32x2{lo, hi};
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
    WIDE_TRACE("attn_qkv_prefill", s);
    attn_qkv_prefill<<<n_kv * mtiles * ntn, 256, 0, s>>>(X, Wq, Wk, Wv, rv.count, rv.perm, T, d, n_kv,
                                                         r, mtiles, vtp, log2_theta, Qc, Kc, Vt);
  }
  const int qtiles = (T + kBQ - 1) / kBQ;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)kHd);
  {
    WIDE_TRACE("attn_core_prefill", s);
    attn_core_prefill<<<qtiles * n_kv * ((r + 3) / 4), 256, 0, s>>>(
        Qc, Kc, Vt, rv.count, rv.perm, T, n_kv, r, qtiles, vtp, scale_log2, O);
  }
}

}  // namespace wide
