// Internal launch interfaces between the C ABI (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wide {

// Brackets one kernel launch with HIP events when tracing is enabled
// (wide_trace_enable); a no-op otherwise.
class TraceScope {
 public:
  TraceScope(const char* name, hipStream_t s);
  ~TraceScope();

 private:
  hipStream_t s_;
  bool active_;
};
#define WIDE_TRACE(name, stream) ::wide::TraceScope wide_trace_scope_(name, stream)

// Device buffers produced by the mask reordering, as the kernels consume them.
struct ReorderView {
  uint64_t* packed = nullptr;     // [T, nw]
  int32_t* count = nullptr;       // [n]
  int32_t* perm = nullptr;        // [n, T]
  int32_t* rank = nullptr;        // [n, T] (may be null when no kernel needs it)
  int32_t* tile_count = nullptr;  // [ceil(T / tile_m)]
  int32_t* tile_groups = nullptr; // [ceil(T / tile_m), n]
  int32_t* order = nullptr;       // [T] token order of the tiles (null: 0..T-1)
  int32_t* tile_perm = nullptr;   // [ceil(T / tile_m)] tile of each K-masked slot (null: identity)
  int tile_m = 0;
};

// The reorder of one mask, as one role set of the reorder launch.  mask null:
// the packed words are the input (the router wrote them); otherwise they are
// written.  tile_count / tile_groups null: no tile unions.  order non-null: also
// the token order sorted by the whole pattern (n <= kSortMaxGroups), whose tiles'
// unions then fill tile_count / tile_groups, and tile_perm (may be null); with
// more groups, sorted by the pattern of the first kSortMaxGroups, and no unions
// (the K-masked GEMM computes its tiles' unions from the rows' mask words).
struct MaskJob {
  const uint8_t* mask = nullptr;
  uint64_t* packed = nullptr;
  int n = 0, nw = 0, tile_m = 0;
  int32_t* count = nullptr;
  int32_t* perm = nullptr;
  int32_t* rank = nullptr;
  int32_t* tile_count = nullptr;
  int32_t* tile_groups = nullptr;
  int32_t* order = nullptr;
  int32_t* tile_perm = nullptr;
};
// RMSNorm rows folded into the reorder launch (x null: none).
struct NormJob {
  const uint16_t* x = nullptr;
  const uint16_t* gamma = nullptr;
  int d = 0;
  float eps = 0.f;
  uint16_t* y = nullptr;
};
// One launch for up to two masks' reorders (a, b may be null) and the norm of the
// T rows (may be null); every role reads only the call's inputs.
void launch_reorder_jobs(int T, const MaskJob* a, const MaskJob* b, const NormJob* norm,
                         hipStream_t s);
void launch_reorder(const uint8_t* mask, int T, int n, int tile_m, uint64_t* packed,
                    int32_t* group_count, int32_t* group_perm, int32_t* group_rank,
                    int32_t* tile_count, int32_t* tile_groups, hipStream_t s);
// The same from packed mask words (the router's output): no packing launch.
void launch_reorder_packed(const uint64_t* packed, int T, int n, int tile_m,
                           int32_t* group_count, int32_t* group_perm, int32_t* group_rank,
                           int32_t* tile_count, int32_t* tile_groups, hipStream_t s);
// Few groups: the attention reorder also sorts the tokens by their whole pattern
// (the key of at most 8 bits; T <= WIDE_MAX_TOKENS keys fit in LDS).
constexpr int kSortMaxGroups = 8;

void launch_pack_kmajor(const uint16_t* W, int n, int G, int d, uint16_t* Wp, hipStream_t s);

int ffn_down_tile_m();
void launch_ffn_prefill(const uint16_t* X, const uint16_t* Wg, const uint16_t* Wu,
                        const uint16_t* Wdp, const ReorderView& rv, int T, int d, int F, int n,
                        const uint16_t* residual, uint16_t* H, uint16_t* Y, hipStream_t s);

// The masked SwiGLU FFN in fp32 (vector FMA): H [T, F] fp32 scratch, W_down [F, d]
// unpacked; any group size and d.
void launch_ffn_f32(const float* X, const uint8_t* mask, const float* Wg, const float* Wu,
                    const float* Wd, int T, int d, int F, int n, float* H, float* Y,
                    hipStream_t s);

// Which projection a K-masked kernel computes.  The kernels are the same; each
// use gets its own instantiation so profilers report them apart.
enum KmUse { kUseFfnDown = 0, kUseAttnO = 1 };

void launch_kmask_gemm(KmUse use, const uint16_t* A, const uint16_t* Wp,
                       const ReorderView& rv, int T, int d, int F, int n, const uint16_t* residual,
                       uint16_t* Y, hipStream_t s);

// Row pitch (keys) of the transposed V of the prefill attention: whole 16-key
// groups, the unit of its in-group key permutation.
inline int vt_pitch(int T) { return (T + 15) / 16 * 16; }

void launch_attn_prefill(const uint16_t* X, const uint16_t* Wq, const uint16_t* Wk,
                         const uint16_t* Wv, const ReorderView& rv, int T, int d, int n_kv, int r,
                         float rope_theta, uint16_t* Qc, uint16_t* Kc, uint16_t* Vt, uint16_t* O,
                         hipStream_t s);

constexpr int kMaxDecodeBatch = 64;
// Decode launchers read the [B, n] mask directly (no reorder launch).
// The K-masked decode projection splits K over work-groups and adds the fp32
// partial sums in a second launch: it takes a workspace of
// kmask_decode_part_floats() floats (0 when it does not split).
size_t kmask_decode_part_floats(int B, int d, int n, int G);
void launch_ffn_decode(const uint16_t* X, const uint8_t* mask, const uint16_t* Wg,
                       const uint16_t* Wu, const uint16_t* Wdp, int B, int d, int F, int n,
                       const uint16_t* residual, uint16_t* H, float* kpart, uint16_t* Y,
                       hipStream_t s);
void launch_kmask_decode(KmUse use, const uint16_t* A, const uint16_t* Wp,
                         const uint8_t* mask, int B, int d, int F, int n,
                         const uint16_t* residual, float* part, uint16_t* Y, hipStream_t s);
// Key chunks of a decode attention over kv_len cache entries plus the new token.
int attn_decode_chunks(int kv_len);
// A paged K/V cache: pools of n_pages pages of 2^page_shift rows (K and V alike)
// and the page table [B, n_kv, kv_cap >> page_shift] of each (sequence, group).
struct PagedKV {
  const int32_t* table;
  int page_shift, n_pages;
};

void launch_attn_decode(const uint16_t* X, const uint8_t* mask, const uint16_t* Wq,
                        const uint16_t* Wk, const uint16_t* Wv, int B, int d,
                        int n_kv, int r, float rope_theta, uint16_t* Kc, uint16_t* Vc, int kv_len,
                        int kv_cap, const int32_t* kvl, int pos, uint16_t* Qd, float* Opart,
                        float* Mpart, float* Lpart, uint16_t* O, hipStream_t s,
                        const PagedKV* paged = nullptr);

// Router logits X R^T and the top-k mask (ties to the lower group index), with
// the mask's packed bit words; logits and packed may be null.  n <= 256.  R in
// fragment order (launch_pack_router: [ceil(n/16)][d/32][64][8]).
void launch_pack_router(const uint16_t* R, int n, int d, uint16_t* Rp, hipStream_t s);
void launch_router_topk(const uint16_t* X, const uint16_t* Rp, int T, int d, int n, int k,
                        float* logits, uint8_t* mask, uint64_t* packed, hipStream_t s);
// Two routers over the same X (router a's column tiles, then router b's): one
// launch when together they have at most 16 tiles, else two; no logits.
void launch_router_topk2(const uint16_t* X, int T, int d, const uint16_t* Ra, int na, int ka,
                         uint8_t* mask_a, uint64_t* packed_a, const uint16_t* Rb, int nb, int kb,
                         uint8_t* mask_b, uint64_t* packed_b, hipStream_t s);

void launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, int T, int d, float eps, uint16_t* y,
                    hipStream_t s);

}  // namespace wide
