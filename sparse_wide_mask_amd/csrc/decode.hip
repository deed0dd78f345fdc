// Decode (a small batch of single tokens): weight streaming over the touched
// groups only (gist.science technical summary §2.C, block-level skipping).
//
// The mask reordering runs with one tile spanning the batch, so tile_groups[0]
// is the union of the groups any token of the batch keeps; a weight block
// outside it is never read.  Kernels (batch B <= 64):
//
// nmask_decode   N-masked projection (FFN gate+up, or attention q/k/v).  One
//                work-group = (group, 16 output rows); it exits at once when no
//                token keeps the group (l=0).  The rows of the tokens that keep
//                the group (group_perm prefix) are the MFMA rows (16x16x32),
//                padded to 16 (l=2: row blocks past the count are skipped); the
//                4 waves split d_model and reduce through LDS.  Epilogue: SwiGLU
//                into H, or RoPE at position kv_len and the q / new k,v writes
//                (k and v straight into the caches at slot kv_len).
// kmask_decode   K-masked projection (FFN down, attention out).  One work-group =
//                16 output columns; the waves split the union groups; rows of
//                tokens that dropped a group are not loaded (l=1).
// attn_decode_partial / attn_decode_combine
//                split-KV attention of each kept (token, group) over cache slots
//                0..kv_len (the new token included), 256 keys per work-group,
//                then a log-sum-exp combine of the chunks.
#include "common.h"
#include "internal.h"

namespace wide {

constexpr int kDecRows = 64;  // max batch of the decode kernels
constexpr int kDecRB = kDecRows / 16;
constexpr int kHdD = 128;

// Mode of nmask_decode.
enum { kNmFfn = 0, kNmQkv = 1 };

template <int MODE>
__global__ void __launch_bounds__(256)
    nmask_decode(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W0,
                 const uint16_t* __restrict__ W1, const uint16_t* __restrict__ W2,
                 const int32_t* __restrict__ gcount, const int32_t* __restrict__ gperm, int B,
                 int d, int G, int chunks, int r, int kv_len, int kv_cap, float log2_theta,
                 uint16_t* __restrict__ out0, uint16_t* __restrict__ Kc, uint16_t* __restrict__ Vc,
                 int n_groups) {
  constexpr int NM = MODE == kNmFfn ? 2 : 1;  // matrices per work-group
  __shared__ int sTok[kDecRows];
  __shared__ float sRed[3][kDecRows][16 * NM];

  const int g = blockIdx.x / chunks, cb = blockIdx.x % chunks;
  const int cnt = gcount[g];
  if (cnt == 0) return;  // l=0: no token of the batch keeps g
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kDecRows; i += 256) sTok[i] = i < cnt ? gperm[(size_t)g * B + i] : -1;
  __syncthreads();
  const int nrb = (cnt + 15) / 16;

  // output row (16 per work-group) -> weight row
  const int ch = lane & 15;
  const uint16_t* wrow[NM];
  int hh = 0, jrow = 0;
  if (MODE == kNmFfn) {
    wrow[0] = W0 + (size_t)(g * G + cb * 16 + ch) * d;
    wrow[NM - 1] = W1 + (size_t)(g * G + cb * 16 + ch) * d;
  } else {
    // chunk cb of head hh (q heads 0..r-1, then k, then v) covers head dims
    // {8c..8c+7} and {64+8c..64+8c+7}, so each RoPE pair stays in the work-group
    hh = cb / 8;
    const int c = cb % 8;
    jrow = ch < 8 ? 8 * c + ch : 64 + 8 * c + (ch - 8);
    if (hh < r)
      wrow[0] = W0 + ((size_t)(g * r + hh) * kHdD + jrow) * d;
    else
      wrow[0] = (hh == r ? W1 : W2) + ((size_t)g * kHdD + jrow) * d;
  }

  f32x4 acc[NM][kDecRB];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int rb = 0; rb < kDecRB; ++rb) acc[m][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = d / 32;  // 32-wide K steps, split evenly over the 4 waves
  const int kbeg = (wave * nsteps / 4) * 32, kend = ((wave + 1) * nsteps / 4) * 32;
  const int koff = 8 * (lane >> 4);
  int xrow[kDecRB];
#pragma unroll
  for (int rb = 0; rb < kDecRB; ++rb) xrow[rb] = sTok[min(rb * 16 + ch, kDecRows - 1)];
#pragma unroll 4
  for (int k0 = kbeg; k0 < kend; k0 += 32) {
    bf16x8 wf[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) wf[m] = *reinterpret_cast<const bf16x8*>(wrow[m] + k0 + koff);
#pragma unroll
    for (int rb = 0; rb < kDecRB; ++rb) {
      if (rb >= nrb) break;  // l=2
      bf16x8 xf = {};
      if (xrow[rb] >= 0) xf = *reinterpret_cast<const bf16x8*>(X + (size_t)xrow[rb] * d + k0 + koff);
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[m][rb] = mfma16(xf, wf[m], acc[m][rb]);
    }
  }

  // reduce the 4 K-quarters: waves 1..3 park partials in LDS, wave 0 adds
  if (wave > 0) {
#pragma unroll
    for (int rb = 0; rb < kDecRB; ++rb) {
      if (rb >= nrb) break;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < NM; ++m)
          sRed[wave - 1][rb * 16 + acc16_row(lane, i)][m * 16 + ch] = acc[m][rb][i];
    }
  }
  __syncthreads();
  if (wave > 0) return;
  const float theta_inv = (MODE == kNmQkv && hh < r + 1 && log2_theta > 0.f)
                              ? exp2f(-(2.f * (ch < 8 ? jrow : jrow - 64) / kHdD) * log2_theta)
                              : 0.f;
  float sn = 0.f, cs = 1.f;
  if (theta_inv != 0.f) sincosf((float)kv_len * theta_inv, &sn, &cs);
#pragma unroll
  for (int rb = 0; rb < kDecRB; ++rb) {
    if (rb >= nrb) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rb * 16 + acc16_row(lane, i);
      float v[NM];
#pragma unroll
      for (int m = 0; m < NM; ++m)
        v[m] = acc[m][rb][i] + sRed[0][row][m * 16 + ch] + sRed[1][row][m * 16 + ch] +
               sRed[2][row][m * 16 + ch];
      const int tok = row < cnt ? sTok[row] : -1;
      if (MODE == kNmFfn) {
        if (tok >= 0) out0[(size_t)tok * (n_groups * G) + g * G + cb * 16 + ch] = f2bf(silu(v[0]) * v[NM - 1]);
      } else {
        // RoPE pair partner: channel ch^8 of the same row, held by lane ^ 8
        const float other = __shfl_xor(v[0], 8);
        float o = v[0];
        if (theta_inv != 0.f) o = ch < 8 ? v[0] * cs - other * sn : v[0] * cs + other * sn;
        if (tok < 0) continue;
        const uint16_t bits = f2bf(o);
        if (hh < r)
          out0[((size_t)tok * (n_groups * r) + g * r + hh) * kHdD + jrow] = bits;
        else
          (hh == r ? Kc : Vc)[(((size_t)tok * n_groups + g) * kv_cap + kv_len) * kHdD + jrow] = bits;
      }
    }
  }
}

// K-masked decode projection: Y[b, n] = sum over union groups g of
// sum_j A[b, gG + j] Wp[g, n, j] over the tokens b that keep g (+ residual).
__global__ void __launch_bounds__(256)
    kmask_decode(const uint16_t* __restrict__ A, const uint16_t* __restrict__ Wp,
                 const uint64_t* __restrict__ packed, const int32_t* __restrict__ ucount,
                 const int32_t* __restrict__ ugroups, int B, int d, int F, int G, int nw,
                 const uint16_t* __restrict__ residual, uint16_t* __restrict__ Y) {
  __shared__ uint64_t sBits[kDecRows * 4];
  __shared__ float sRed[3][kDecRows][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16;
  for (int i = tid; i < kDecRows * nw; i += 256) {
    const int b = i / nw, w = i % nw;
    sBits[b * 4 + w] = b < B ? packed[(size_t)b * nw + w] : 0ull;
  }
  __syncthreads();
  const int nu = ucount[0];
  const int nrb = (B + 15) / 16;
  const int ch = lane & 15, koff = 8 * (lane >> 4);
  f32x4 acc[kDecRB];
#pragma unroll
  for (int rb = 0; rb < kDecRB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int u = wave; u < nu; u += 4) {
    const int g = ugroups[u];
    const uint64_t sel = 1ull << (g & 63);
    const int w = g >> 6;
    bool keep[kDecRB];
#pragma unroll
    for (int rb = 0; rb < kDecRB; ++rb) {
      const int b = rb * 16 + ch;
      keep[rb] = b < B && (sBits[b * 4 + w] & sel);
    }
    const uint16_t* wrow = Wp + ((size_t)g * d + n0 + ch) * G + koff;
    const uint16_t* arow = A + (size_t)g * G + koff;
#pragma unroll 4
    for (int j0 = 0; j0 < G; j0 += 32) {
      const bf16x8 wf = *reinterpret_cast<const bf16x8*>(wrow + j0);
#pragma unroll
      for (int rb = 0; rb < kDecRB; ++rb) {
        if (rb >= nrb) break;
        bf16x8 af = {};
        if (keep[rb]) af = *reinterpret_cast<const bf16x8*>(arow + (size_t)(rb * 16 + ch) * F + j0);
        acc[rb] = mfma16(af, wf, acc[rb]);
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int rb = 0; rb < kDecRB; ++rb) {
      if (rb >= nrb) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) sRed[wave - 1][rb * 16 + acc16_row(lane, i)][ch] = acc[rb][i];
    }
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int rb = 0; rb < kDecRB; ++rb) {
    if (rb >= nrb) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = rb * 16 + acc16_row(lane, i);
      if (b >= B) continue;
      float v = acc[rb][i] + sRed[0][b][ch] + sRed[1][b][ch] + sRed[2][b][ch];
      const size_t o = (size_t)b * d + n0 + ch;
      if (residual) v += bf2f(residual[o]);
      Y[o] = f2bf(v);
    }
  }
}

constexpr int kKeyChunk = 256;

// One work-group = (token b, group g, chunk of 256 cache keys).  Scores with 16
// lanes per key (8 head dims each), then per-head softmax statistics of the
// chunk, then P V with 64 threads per head.  Writes unnormalised partial outputs.
__global__ void __launch_bounds__(256)
    attn_decode_partial(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kc,
                        const uint16_t* __restrict__ Vc, const uint8_t* __restrict__ mask, int B,
                        int n_kv, int r, int kv_len, int kv_cap, int nch, float scale_log2,
                        float* __restrict__ Opart, float* __restrict__ Mpart,
                        float* __restrict__ Lpart) {
  __shared__ float sQ[8][kHdD];
  __shared__ float sP[8][kKeyChunk];
  __shared__ float sRed[8][4];
  const int c = blockIdx.x % nch, rest = blockIdx.x / nch;
  const int g = rest % n_kv, b = rest / n_kv;
  if (!mask[(size_t)b * n_kv + g]) return;  // l=0: the token dropped this group
  const int k0 = c * kKeyChunk;
  const int nkeys = min(kKeyChunk, kv_len + 1 - k0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nq = n_kv * r;
  for (int i = tid; i < r * kHdD; i += 256)
    sQ[i / kHdD][i % kHdD] = bf2f(Q[((size_t)b * nq + g * r) * kHdD + i]);
  __syncthreads();

  const size_t kvbase = ((size_t)b * n_kv + g) * kv_cap;
  // scores: each wave takes 4 keys per pass (16 lanes per key)
  const int sub = lane >> 4, part = lane & 15;
  for (int base = wave * 4; base < kKeyChunk; base += 16) {
    const int kk = base + sub;
    float s[8];
    bool ok = kk < nkeys;
    u32x4 kv = {0, 0, 0, 0};
    if (ok) kv = *reinterpret_cast<const u32x4*>(Kc + (kvbase + k0 + kk) * kHdD + part * 8);
    float kf[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kf[2 * e] = __uint_as_float(kv[e] << 16);
      kf[2 * e + 1] = __uint_as_float(kv[e] & 0xffff0000u);
    }
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      float a = 0.f;
      if (h < r)
#pragma unroll
        for (int e = 0; e < 8; ++e) a += kf[e] * sQ[h][part * 8 + e];
      a += __shfl_xor(a, 8);
      a += __shfl_xor(a, 4);
      a += __shfl_xor(a, 2);
      a += __shfl_xor(a, 1);
      s[h] = a;
    }
    if (part == 0) {
#pragma unroll
      for (int h = 0; h < 8; ++h)
        if (h < r) sP[h][kk] = ok ? s[h] * scale_log2 : -INFINITY;
    }
  }
  __syncthreads();
  // per-head max and sum over the chunk (thread t = key t)
  float mh[8], lh[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    if (h >= r) break;
    float v = sP[h][tid];
    float m = v;
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) sRed[h][wave] = m;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    if (h >= r) break;
    mh[h] = fmaxf(fmaxf(sRed[h][0], sRed[h][1]), fmaxf(sRed[h][2], sRed[h][3]));
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
    lh[h] = sRed[h][0] + sRed[h][1] + sRed[h][2] + sRed[h][3];
  }
  // P V: thread -> (head, pair of dims); V rows read 256 bytes per 64 threads
  const size_t obase = ((size_t)b * nq + g * r) * nch;
  for (int o = tid; o < r * 64; o += 256) {
    const int h = o >> 6, jp = (o & 63) * 2;
    float a0 = 0.f, a1 = 0.f;
    const uint16_t* vp = Vc + (kvbase + k0) * kHdD + jp;
    for (int kk = 0; kk < nkeys; ++kk) {
      const uint32_t v2 = *reinterpret_cast<const uint32_t*>(vp + (size_t)kk * kHdD);
      const float p = sP[h][kk];
      a0 += p * __uint_as_float(v2 << 16);
      a1 += p * __uint_as_float(v2 & 0xffff0000u);
    }
    float* op = Opart + ((obase + (size_t)h * nch + c) * kHdD) + jp;
    op[0] = a0;
    op[1] = a1;
  }
  if (tid < r) {
    Mpart[obase + (size_t)tid * nch + c] = mh[tid];
    Lpart[obase + (size_t)tid * nch + c] = lh[tid];
  }
}

// (token b, query head h): O[b, h] = sum_c 2^(M_c - M) Opart_c / sum_c 2^(M_c - M) L_c.
__global__ void __launch_bounds__(128)
    attn_decode_combine(const float* __restrict__ Opart, const float* __restrict__ Mpart,
                        const float* __restrict__ Lpart, const uint8_t* __restrict__ mask,
                        int n_kv, int r, int nch, uint16_t* __restrict__ O) {
  const int nq = n_kv * r;
  const int b = blockIdx.x / nq, h = blockIdx.x % nq, g = h / r;
  if (!mask[(size_t)b * n_kv + g]) return;  // never read: the O projection skips it
  const size_t base = (size_t)b * nq * nch + (size_t)h * nch;
  float m = -INFINITY;
  for (int c = 0; c < nch; ++c) m = fmaxf(m, Mpart[base + c]);
  float l = 0.f, acc = 0.f;
  const int j = threadIdx.x;
  for (int c = 0; c < nch; ++c) {
    const float w = exp2f(Mpart[base + c] - m);
    l += w * Lpart[base + c];
    acc += w * Opart[(base + c) * kHdD + j];
  }
  O[((size_t)b * nq + h) * kHdD + j] = f2bf(acc / l);
}

// ------------------------------------------------------------------ launchers

void launch_ffn_decode(const uint16_t* X, const uint16_t* Wg, const uint16_t* Wu,
                       const uint16_t* Wdp, const ReorderView& rv, int B, int d, int F, int n,
                       const uint16_t* residual, uint16_t* H, uint16_t* Y, hipStream_t s) {
  const int G = F / n, chunks = G / 16;
  {
    WIDE_TRACE("ffn_up_decode", s);
    nmask_decode<kNmFfn><<<n * chunks, 256, 0, s>>>(X, Wg, Wu, nullptr, rv.count, rv.perm, B, d, G,
                                                    chunks, 0, 0, 0, 0.f, H, nullptr, nullptr, n);
  }
  launch_kmask_decode("ffn_down_decode", H, Wdp, rv, B, d, F, n, residual, Y, s);
}

void launch_kmask_decode(const char* tname, const uint16_t* A, const uint16_t* Wp,
                         const ReorderView& rv, int B, int d, int F, int n,
                         const uint16_t* residual, uint16_t* Y, hipStream_t s) {
  WIDE_TRACE(tname, s);
  kmask_decode<<<d / 16, 256, 0, s>>>(A, Wp, rv.packed, rv.tile_count, rv.tile_groups, B, d, F,
                                      F / n, (n + 63) / 64, residual, Y);
}

int attn_decode_chunks(int kv_len) { return (kv_len + 1 + kKeyChunk - 1) / kKeyChunk; }

void launch_attn_decode(const uint16_t* X, const uint8_t* mask, const uint16_t* Wq,
                        const uint16_t* Wk, const uint16_t* Wv, const ReorderView& rv, int B, int d,
                        int n_kv, int r, float rope_theta, uint16_t* Kc, uint16_t* Vc, int kv_len,
                        int kv_cap, uint16_t* Qd, float* Opart, float* Mpart, float* Lpart,
                        uint16_t* O, hipStream_t s) {
  const int chunks = (r + 2) * 8;  // 16-row chunks of the group's q, k, v heads
  const float log2_theta = rope_theta > 0.f ? log2f(rope_theta) : 0.f;
  {
    WIDE_TRACE("attn_qkv_decode", s);
    nmask_decode<kNmQkv><<<n_kv * chunks, 256, 0, s>>>(X, Wq, Wk, Wv, rv.count, rv.perm, B, d, kHdD,
                                                       chunks, r, kv_len, kv_cap, log2_theta, Qd,
                                                       Kc, Vc, n_kv);
  }
  const int nch = attn_decode_chunks(kv_len);
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)kHdD);
  {
    WIDE_TRACE("attn_core_decode", s);
    attn_decode_partial<<<B * n_kv * nch, 256, 0, s>>>(Qd, Kc, Vc, mask, B, n_kv, r, kv_len, kv_cap,
                                                       nch, scale_log2, Opart, Mpart, Lpart);
  }
  {
    WIDE_TRACE("attn_combine_decode", s);
    attn_decode_combine<<<B * n_kv * r, kHdD, 0, s>>>(Opart, Mpart, Lpart, mask, n_kv, r, nch, O);
  }
}

}  // namespace wide
