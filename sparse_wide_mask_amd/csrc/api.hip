// C ABI of libwide: argument validation, workspace carving and launch order.
// Every check runs on the host before anything is enqueued.
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "../../include/wide.h"
#include "internal.h"

namespace {

using namespace wide;

bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool null_or_aligned16(const void* p) { return !p || aligned16(p); }

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Bump allocator over the caller's workspace.  With base == nullptr it only
// measures, which is how the *_workspace() queries are answered.
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += round_up(count * sizeof(T));
    return p;
  }
};

int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? WIDE_OK : WIDE_EHIP;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

int ceil_div(int a, int b) { return (a + b - 1) / b; }

ReorderView carve_reorder(Carver& c, int T, int n, int tile_m, bool with_rank) {
  ReorderView v;
  const int nw = ceil_div(n, 64);
  v.packed = c.take<uint64_t>((size_t)T * nw);
  v.count = c.take<int32_t>(n);
  v.perm = c.take<int32_t>((size_t)n * T);
  v.rank = with_rank ? c.take<int32_t>((size_t)n * T) : nullptr;
  v.tile_m = tile_m;
  v.tile_count = c.take<int32_t>(ceil_div(T, tile_m));
  v.tile_groups = c.take<int32_t>((size_t)ceil_div(T, tile_m) * n);
  return v;
}

void run_reorder(const uint8_t* mask, int T, int n, const ReorderView& v, hipStream_t s) {
  launch_reorder(mask, T, n, v.tile_m, v.packed, v.count, v.perm, v.rank, v.tile_count,
                 v.tile_groups, s);
}

// ---------------------------------------------------------------- FFN

// Kernels address operands with 32-bit byte offsets below the skip sentinel.
constexpr int64_t kMaxBytes = 0x7fffff00LL;
bool fits(int64_t a, int64_t b) { return a * b * 2 <= kMaxBytes; }

// fp32 FFN: H [T, d_ff] fp32 in the workspace; 64-bit element offsets in the kernels
int ffn_f32_check(int T, int d, int F, int n) {
  if (T < 0 || d <= 0 || F <= 0 || n <= 0 || F % n) return WIDE_EINVAL;
  if (n > WIDE_MAX_GROUPS || T > WIDE_MAX_TOKENS) return WIDE_EUNSUPPORTED;
  return WIDE_OK;
}

int ffn_check(int T, int d, int F, int n, int mode) {
  if (T < 0 || d <= 0 || F <= 0 || n <= 0) return WIDE_EINVAL;
  if (mode != WIDE_PREFILL && mode != WIDE_DECODE) return WIDE_EINVAL;
  if (F % n) return WIDE_EINVAL;
  if (n > WIDE_MAX_GROUPS || T > WIDE_MAX_TOKENS) return WIDE_EUNSUPPORTED;
  if (!fits(T, d) || !fits(F, d) || !fits(T, F)) return WIDE_EUNSUPPORTED;
  const int G = F / n;
  if ((G % 64 && G != 32) || d % 64) return WIDE_EUNSUPPORTED;  // groups of 64k or 32
  return WIDE_OK;
}

struct FfnWs {
  ReorderView rv;
  uint16_t* H = nullptr;
  float* kpart = nullptr;  // streaming decode: K-split partial sums
};

// Decode kernels take batches up to kMaxDecodeBatch; a larger "decode" batch runs
// the prefill kernels (the FFN keeps no state, so the result is the same).
bool ffn_streaming(int T, int mode) { return mode == WIDE_DECODE && T <= kMaxDecodeBatch; }

FfnWs carve_ffn(Carver& c, int T, int d, int F, int n, int mode) {
  FfnWs w;
  // streaming decode reorders inside its kernels
  if (!ffn_streaming(T, mode)) {
    w.rv = carve_reorder(c, T, n, ffn_down_tile_m(), false);
    w.rv.order = c.take<int32_t>(T);  // the down projection's token order, when sorted
  }
  w.H = c.take<uint16_t>((size_t)T * F);
  if (ffn_streaming(T, mode)) {
    w.kpart = c.take<float>(kmask_decode_part_floats(T, d, n, F / n));
  }
  return w;
}

// The FFN mask's reorder job.  sort: the tokens are also sorted by the pattern of
// their first groups (WIDE_FLAG_FFN_TOKEN_SORT) for the down projection, which then
// computes its tiles' unions itself.
MaskJob ffn_job(const uint8_t* mask, int T, int n, const FfnWs& w, bool packed_ready, bool sort) {
  const ReorderView& v = w.rv;
  MaskJob j;
  j.mask = packed_ready ? nullptr : mask;
  j.packed = v.packed;
  j.n = n, j.nw = (n + 63) / 64, j.tile_m = v.tile_m;
  j.count = v.count, j.perm = v.perm, j.rank = v.rank;
  j.tile_count = sort ? nullptr : v.tile_count;
  j.tile_groups = sort ? nullptr : v.tile_groups;
  j.order = sort ? v.order : nullptr;
  return j;
}

// reorder = false: the mask reorder of this call was already enqueued (by the
// layer's norm + reorder launch, on the same stream)
int ffn_run(const uint16_t* X, const uint8_t* mask, const uint16_t* Wg, const uint16_t* Wu,
            const uint16_t* Wdp, int T, int d, int F, int n, int mode, const uint16_t* residual,
            uint16_t* Y, const FfnWs& w, hipStream_t s, bool reorder = true, bool sort = false) {
  if (ffn_streaming(T, mode)) {
    launch_ffn_decode(X, mask, Wg, Wu, Wdp, T, d, F, n, residual, w.H, w.kpart, Y, s);
  } else {
    if (reorder) {
      const MaskJob j = ffn_job(mask, T, n, w, false, sort);
      launch_reorder_jobs(T, &j, nullptr, nullptr, s);
    }
    ReorderView rv = w.rv;
    if (sort) {
      rv.tile_count = rv.tile_groups = nullptr;
    } else {
      rv.order = nullptr;
    }
    launch_ffn_prefill(X, Wg, Wu, Wdp, rv, T, d, F, n, residual, w.H, Y, s);
  }
  return WIDE_OK;
}

// ---------------------------------------------------------------- attention

constexpr int kHeadDim = 128;

int attn_check(int T, int d, const wide_attn_cfg* cfg, int mode) {
  if (!cfg || T < 0 || d <= 0) return WIDE_EINVAL;
  if (mode != WIDE_PREFILL && mode != WIDE_DECODE) return WIDE_EINVAL;
  const int nq = cfg->n_q_heads, nkv = cfg->n_kv_heads;
  if (nq < 1 || nkv < 1 || nq % nkv || cfg->head_dim < 1) return WIDE_EINVAL;
  if (!(cfg->rope_theta >= 0.f)) return WIDE_EINVAL;  // also rejects NaN
  if (cfg->head_dim != kHeadDim || d % 64) return WIDE_EUNSUPPORTED;
  if (nkv > WIDE_MAX_GROUPS || T > WIDE_MAX_TOKENS) return WIDE_EUNSUPPORTED;
  const int64_t F = (int64_t)nq * kHeadDim;
  if (!fits(T, d) || !fits(F, d) || !fits(T, F)) return WIDE_EUNSUPPORTED;
  if (mode == WIDE_DECODE && (T > kMaxDecodeBatch || nq / nkv > 8)) return WIDE_EUNSUPPORTED;
  return WIDE_OK;
}

// Decode arguments: caches present, 0 <= kv_len < kv_cap, cache sizes addressable.
int attn_decode_check(int T, const wide_attn_cfg* cfg, const uint16_t* K_cache,
                      const uint16_t* V_cache, int kv_len, int kv_cap) {
  if (!aligned16(K_cache) || !aligned16(V_cache) || K_cache == V_cache) return WIDE_EINVAL;
  if (kv_cap < 1 || kv_len < 0 || kv_len >= kv_cap) return WIDE_EINVAL;
  if (!fits((int64_t)T * cfg->n_kv_heads * kv_cap, kHeadDim)) return WIDE_EUNSUPPORTED;
  return WIDE_OK;
}

struct AttnWs {
  ReorderView rv;
  uint16_t *Qc = nullptr, *Kc = nullptr, *Vt = nullptr, *O = nullptr;
  float *Opart = nullptr, *Mpart = nullptr, *Lpart = nullptr;
  float* kpart = nullptr;  // decode O projection: K-split partial sums
};

AttnWs carve_attn(Carver& c, int T, int d, const wide_attn_cfg* cfg, int mode, int kv_cap) {
  AttnWs w;
  const int nq = cfg->n_q_heads, nkv = cfg->n_kv_heads;
  if (mode == WIDE_DECODE) {
    const int nch = attn_decode_chunks(kv_cap > 0 ? kv_cap - 1 : 0);
    w.Qc = c.take<uint16_t>((size_t)T * nq * kHeadDim);
    w.O = c.take<uint16_t>((size_t)T * nq * kHeadDim);
    w.Opart = c.take<float>((size_t)T * nq * nch * kHeadDim);
    w.Mpart = c.take<float>((size_t)T * nq * nch);
    w.Lpart = c.take<float>((size_t)T * nq * nch);
    w.kpart = c.take<float>(kmask_decode_part_floats(T, d, nkv, nq * kHeadDim / nkv));
    return w;
  }
  w.rv = carve_reorder(c, T, nkv, ffn_down_tile_m(), false);
  if (nkv <= kSortMaxGroups) {
    w.rv.order = c.take<int32_t>(T);
    w.rv.tile_perm = c.take<int32_t>(ceil_div(T, w.rv.tile_m));
  }
  w.Qc = c.take<uint16_t>((size_t)nq * T * kHeadDim);
  w.Kc = c.take<uint16_t>((size_t)nkv * T * kHeadDim);
  w.Vt = c.take<uint16_t>((size_t)nkv * kHeadDim * vt_pitch(T));
  w.O = c.take<uint16_t>((size_t)T * nq * kHeadDim);
  return w;
}

// Prefill: group partitions for the QKV projection and the core; for the O
// projection with few groups, tiles of tokens sorted by their head-group
// pattern, so that row blocks and whole tiles share dropped groups.
// The reorder jobs of the attention and FFN masks.  packed_ready: the packed words
// already hold the mask (the router wrote them) and are the input.  With few
// groups the attention job also sorts the tokens by pattern (the O projection's
// tiles and unions).
MaskJob attn_job(const uint8_t* mask, int T, int nkv, const AttnWs& w, bool packed_ready) {
  const ReorderView& v = w.rv;
  const bool sort = nkv <= kSortMaxGroups;
  MaskJob j;
  j.mask = packed_ready ? nullptr : mask;
  j.packed = v.packed;
  j.n = nkv, j.nw = (nkv + 63) / 64, j.tile_m = v.tile_m;
  j.count = v.count, j.perm = v.perm, j.rank = v.rank;
  j.tile_count = v.tile_count, j.tile_groups = v.tile_groups;
  j.order = sort ? v.order : nullptr;
  j.tile_perm = sort ? v.tile_perm : nullptr;
  return j;
}

void attn_reorder(const uint8_t* mask, int T, int nkv, const AttnWs& w, hipStream_t s,
                  bool packed_ready = false) {
  const MaskJob j = attn_job(mask, T, nkv, w, packed_ready);
  launch_reorder_jobs(T, &j, nullptr, nullptr, s);
}

// reorder = false: attn_reorder of this call was already enqueued.
int attn_run(const uint16_t* X, const uint8_t* mask, const uint16_t* Wq, const uint16_t* Wk,
             const uint16_t* Wv, const uint16_t* Wop, int T, int d, const wide_attn_cfg* cfg,
             int mode, uint16_t* K_cache, uint16_t* V_cache, int kv_len, int kv_cap,
             const uint16_t* residual, uint16_t* Y, const AttnWs& w, hipStream_t s,
             const int32_t* pair_len = nullptr, int pos = -1, bool reorder = true,
             const PagedKV* paged = nullptr) {
  const int nq = cfg->n_q_heads, nkv = cfg->n_kv_heads, r = nq / nkv;
  if (mode == WIDE_DECODE) {
    launch_attn_decode(X, mask, Wq, Wk, Wv, T, d, nkv, r, cfg->rope_theta, K_cache, V_cache, kv_len,
                       kv_cap, pair_len, pos < 0 ? kv_len : pos, w.Qc, w.Opart, w.Mpart, w.Lpart,
                       w.O, s, paged);
    launch_kmask_decode(kUseAttnO, w.O, Wop, mask, T, d, nq * kHeadDim, nkv, residual, w.kpart,
                        Y, s);
    return WIDE_OK;
  }
  if (reorder) attn_reorder(mask, T, nkv, w, s);
  launch_attn_prefill(X, Wq, Wk, Wv, w.rv, T, d, nkv, r, cfg->rope_theta, w.Qc, w.Kc, w.Vt, w.O, s);
  launch_kmask_gemm(kUseAttnO, w.O, Wop, w.rv, T, d, nq * kHeadDim, nkv, residual, Y, s);
  return WIDE_OK;
}

// -------------------------------------------------------------------- layer

int layer_check(int T, const wide_layer_cfg* cfg, int mode) {
  if (!cfg) return WIDE_EINVAL;
  if (!(cfg->rms_eps >= 0.f)) return WIDE_EINVAL;
  int st = attn_check(T, cfg->d_model, &cfg->attn, mode);
  if (st != WIDE_OK) return st;
  return ffn_check(T, cfg->d_model, cfg->d_ff, cfg->n_ffn_groups, mode);
}

struct LayerWs {
  uint16_t *u = nullptr, *h = nullptr;
  AttnWs attn;
  FfnWs ffn;
};

LayerWs carve_layer(Carver& c, int T, const wide_layer_cfg* cfg, int mode, int kv_cap) {
  LayerWs w;
  const int d = cfg->d_model;
  w.u = c.take<uint16_t>((size_t)T * d);
  w.h = c.take<uint16_t>((size_t)T * d);
  w.attn = carve_attn(c, T, d, &cfg->attn, mode, kv_cap);
  w.ffn = carve_ffn(c, T, d, cfg->d_ff, cfg->n_ffn_groups, mode);
  return w;
}

// Decode cache of a layer call: one length for the batch (kv_len), or lengths per
// (sequence, group) in device memory (pair_len) with the new tokens' RoPE
// position, optionally in a paged pool.
struct LayerCache {
  uint16_t *K = nullptr, *V = nullptr;
  int kv_len = 0, kv_cap = 0;
  const int32_t* pair_len = nullptr;
  int pos = -1;
  const PagedKV* paged = nullptr;
};

// Launch sequence of a layer call (arguments validated), on the caller's stream
// alone.  Prefill: one launch does the first RMSNorm and both mask reorders (the
// reorders read only the call's inputs, so they run beside the norm rows), then
// the attention kernels, the second RMSNorm and the FFN kernels.  packed_ready:
// the reorders' packed words already hold both masks (the router wrote them).
int layer_run(const uint16_t* X, const uint8_t* attn_mask, const uint8_t* ffn_mask,
              const wide_layer_weights* W, const wide_layer_cfg* cfg, int T, int mode,
              const LayerCache& kv, uint16_t* Y, const LayerWs& w, hipStream_t s,
              bool packed_ready, bool sort_ffn = false) {
  const int d = cfg->d_model, nkv = cfg->attn.n_kv_heads, n = cfg->n_ffn_groups;
  if (mode == WIDE_PREFILL) {
    const MaskJob aj = attn_job(attn_mask, T, nkv, w.attn, packed_ready);
    const MaskJob fj = ffn_job(ffn_mask, T, n, w.ffn, packed_ready, sort_ffn);
    NormJob nj;
    nj.x = X, nj.gamma = W->rms1, nj.d = d, nj.eps = cfg->rms_eps, nj.y = w.u;
    launch_reorder_jobs(T, &aj, &fj, &nj, s);
  } else {
    launch_rmsnorm(X, W->rms1, T, d, cfg->rms_eps, w.u, s);
  }
  attn_run(w.u, attn_mask, W->Wq, W->Wk, W->Wv, W->Wo_packed, T, d, &cfg->attn, mode, kv.K, kv.V,
           kv.kv_len, kv.kv_cap, X, w.h, w.attn, s, kv.pair_len, kv.pos, false, kv.paged);
  launch_rmsnorm(w.h, W->rms2, T, d, cfg->rms_eps, w.u, s);
  ffn_run(w.u, ffn_mask, W->W_gate, W->W_up, W->W_down_packed, T, d, cfg->d_ff, n, mode, w.h, Y,
          w.ffn, s, false, sort_ffn);
  return launch_status();
}

bool layer_weights_ok(const wide_layer_weights* W) {
  return W && aligned16(W->rms1) && aligned16(W->rms2) && aligned16(W->Wq) &&
         aligned16(W->Wk) && aligned16(W->Wv) && aligned16(W->Wo_packed) &&
         aligned16(W->W_gate) && aligned16(W->W_up) && aligned16(W->W_down_packed);
}

// ------------------------------------------------ allocation-free FFN entry point

// The scratch memory of wide_ffn_masked_noalloc: a fixed array in device memory,
// one copy per GPU (held from the library's load on that device until the process
// ends).  In host code `scratch` only names the symbol; its device address on the
// current GPU comes from hipGetSymbolAddress, once per device, and only that
// address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[WIDE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct ScratchAddr {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchAddr g_scratch[kMaxDevices];

// Device address of the current GPU's scratch array, or nullptr if HIP cannot
// give it (the call then fails with WIDE_EHIP).
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  ScratchAddr& a = g_scratch[dev];
  std::call_once(a.once, [&a] {
    a.err = hipGetSymbolAddress(&a.ptr, HIP_SYMBOL(scratch));
    if (a.err != hipSuccess) a.ptr = nullptr;
  });
  return a.ptr;
}

}  // namespace

extern "C" {

const char* wide_status_string(int status) {
  switch (status) {
    case WIDE_OK: return "ok";
    case WIDE_EINVAL: return "invalid argument";
    case WIDE_EUNSUPPORTED: return "unsupported shape or mode";
    case WIDE_EWORKSPACE: return "workspace too small";
    case WIDE_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int wide_version(void) { return 1; }

int wide_mask_reorder(const uint8_t* mask, int T, int n_groups, int tile_m, uint64_t* packed,
                      int32_t* group_count, int32_t* group_perm, int32_t* group_rank,
                      int32_t* tile_count, int32_t* tile_groups, void* stream) {
  if (T < 0 || n_groups < 1 || tile_m < 1 || tile_m > 1024) return WIDE_EINVAL;
  if (n_groups > WIDE_MAX_GROUPS || T > WIDE_MAX_TOKENS) return WIDE_EUNSUPPORTED;
  if (T == 0) return WIDE_OK;
  if (!aligned16(mask) || !aligned16(packed) || !aligned16(group_count) ||
      !aligned16(group_perm) || !aligned16(group_rank) || !null_or_aligned16(tile_count) ||
      !null_or_aligned16(tile_groups) || (tile_count == nullptr) != (tile_groups == nullptr))
    return WIDE_EINVAL;
  (void)hipGetLastError();
  launch_reorder(mask, T, n_groups, tile_m, packed, group_count, group_perm, group_rank,
                 tile_count, tile_groups, as_stream(stream));
  return launch_status();
}

int wide_mask_reorder_packed(const uint64_t* packed, int T, int n_groups, int tile_m,
                             int32_t* group_count, int32_t* group_perm, int32_t* group_rank,
                             int32_t* tile_count, int32_t* tile_groups, void* stream) {
  if (T < 0 || n_groups < 1 || tile_m < 1 || tile_m > 1024) return WIDE_EINVAL;
  if (n_groups > WIDE_MAX_GROUPS || T > WIDE_MAX_TOKENS) return WIDE_EUNSUPPORTED;
  if (T == 0) return WIDE_OK;
  if (!aligned16(packed) || !aligned16(group_count) || !aligned16(group_perm) ||
      !aligned16(group_rank) || !aligned16(tile_count) || !aligned16(tile_groups))
    return WIDE_EINVAL;
  (void)hipGetLastError();
  launch_reorder_packed(packed, T, n_groups, tile_m, group_count, group_perm, group_rank,
                        tile_count, tile_groups, as_stream(stream));
  return launch_status();
}

int wide_pack_router(const uint16_t* R, int n_groups, int d_model, uint16_t* R_packed,
                     void* stream) {
  if (n_groups < 1 || d_model <= 0) return WIDE_EINVAL;
  if (n_groups > WIDE_MAX_GROUPS || d_model % 64 || !fits(n_groups, d_model))
    return WIDE_EUNSUPPORTED;
  if (!aligned16(R) || !aligned16(R_packed) || R == R_packed) return WIDE_EINVAL;
  (void)hipGetLastError();
  launch_pack_router(R, n_groups, d_model, R_packed, as_stream(stream));
  return launch_status();
}

int wide_router_topk(const uint16_t* X, const uint16_t* R, int T, int d_model, int n_groups,
                     int k, float* logits, uint8_t* mask, uint64_t* packed, void* stream) {
  if (T < 0 || d_model <= 0 || n_groups < 1 || k < 0 || k > n_groups) return WIDE_EINVAL;
  if (n_groups > WIDE_MAX_GROUPS || T > WIDE_MAX_TOKENS || d_model % 64) return WIDE_EUNSUPPORTED;
  if (!fits(T, d_model) || !fits(n_groups, d_model)) return WIDE_EUNSUPPORTED;
  if (T == 0) return WIDE_OK;
  if (!aligned16(X) || !aligned16(R) || !aligned16(mask)) return WIDE_EINVAL;
  if ((logits && !aligned16(logits)) || (packed && !aligned16(packed))) return WIDE_EINVAL;
  if ((const void*)mask == (const void*)X || (const void*)mask == (const void*)R ||
      (const void*)logits == (const void*)X || (const void*)logits == (const void*)R ||
      (const void*)packed == (const void*)X || (const void*)packed == (const void*)R)
    return WIDE_EINVAL;
  (void)hipGetLastError();
  launch_router_topk(X, R, T, d_model, n_groups, k, logits, mask, packed, as_stream(stream));
  return launch_status();
}

int wide_pack_kmajor(const uint16_t* W, int n_groups, int G, int d_model, uint16_t* W_packed,
                     void* stream) {
  if (n_groups < 1 || G < 1 || d_model < 1) return WIDE_EINVAL;
  if (!aligned16(W) || !aligned16(W_packed) || W == W_packed) return WIDE_EINVAL;
  if ((G % 64 && G != 32) || d_model % 64 || n_groups > 65535) return WIDE_EUNSUPPORTED;
  (void)hipGetLastError();
  launch_pack_kmajor(W, n_groups, G, d_model, W_packed, as_stream(stream));
  return launch_status();
}

size_t wide_ffn_masked_workspace(int T, int d_model, int d_ff, int n_groups, int mode) {
  if (ffn_check(T, d_model, d_ff, n_groups, mode) != WIDE_OK) return 0;
  Carver c(nullptr);
  carve_ffn(c, T, d_model, d_ff, n_groups, mode);
  return c.used;
}

int wide_ffn_masked(const uint16_t* X, const uint8_t* mask, const uint16_t* W_gate,
                    const uint16_t* W_up, const uint16_t* W_down_packed, int T, int d_model,
                    int d_ff, int n_groups, int mode, uint16_t* Y, void* workspace,
                    size_t workspace_bytes, uint32_t flags, void* stream) {
  int st = ffn_check(T, d_model, d_ff, n_groups, mode);
  if (st != WIDE_OK) return st;
  if (flags & ~WIDE_FLAG_FFN_TOKEN_SORT) return WIDE_EINVAL;
  if (T == 0) return WIDE_OK;
  if (!aligned16(X) || !aligned16(mask) || !aligned16(W_gate) || !aligned16(W_up) ||
      !aligned16(W_down_packed) || !aligned16(Y) || (void*)Y == (void*)X)
    return WIDE_EINVAL;
  Carver probe(nullptr);
  carve_ffn(probe, T, d_model, d_ff, n_groups, mode);
  if (!aligned16(workspace)) return probe.used ? WIDE_EINVAL : WIDE_OK;
  if (workspace_bytes < probe.used) return WIDE_EWORKSPACE;
  Carver c(workspace);
  FfnWs w = carve_ffn(c, T, d_model, d_ff, n_groups, mode);
  (void)hipGetLastError();
  ffn_run(X, mask, W_gate, W_up, W_down_packed, T, d_model, d_ff, n_groups, mode, nullptr, Y, w,
          as_stream(stream), true, (flags & WIDE_FLAG_FFN_TOKEN_SORT) != 0);
  return launch_status();
}

size_t wide_ffn_masked_f32_workspace(int T, int d_model, int d_ff, int n_groups) {
  if (ffn_f32_check(T, d_model, d_ff, n_groups) != WIDE_OK) return 0;
  return round_up((size_t)T * d_ff * sizeof(float));
}

int wide_ffn_masked_f32(const float* X, const uint8_t* mask, const float* W_gate,
                        const float* W_up, const float* W_down, int T, int d_model, int d_ff,
                        int n_groups, float* Y, void* workspace, size_t workspace_bytes,
                        uint32_t flags, void* stream) {
  const int st = ffn_f32_check(T, d_model, d_ff, n_groups);
  if (st != WIDE_OK) return st;
  if (flags != 0) return WIDE_EINVAL;
  if (T == 0) return WIDE_OK;
  if (!aligned16(X) || !aligned16(mask) || !aligned16(W_gate) || !aligned16(W_up) ||
      !aligned16(W_down) || !aligned16(Y) || (void*)Y == (void*)X || !aligned16(workspace))
    return WIDE_EINVAL;
  if (workspace_bytes < wide_ffn_masked_f32_workspace(T, d_model, d_ff, n_groups))
    return WIDE_EWORKSPACE;
  (void)hipGetLastError();
  launch_ffn_f32(X, mask, W_gate, W_up, W_down, T, d_model, d_ff, n_groups,
                 static_cast<float*>(workspace), Y, as_stream(stream));
  return launch_status();
}

int wide_ffn_masked_noalloc(const uint16_t* X, const uint8_t* mask, const uint16_t* W_gate,
                            const uint16_t* W_up, const uint16_t* W_down_packed, int T,
                            int d_model, int d_ff, int n_groups, int mode, uint16_t* Y,
                            uint32_t flags, void* stream) {
  int st = ffn_check(T, d_model, d_ff, n_groups, mode);
  if (st != WIDE_OK) return st;
  if (flags != 0) return WIDE_EINVAL;
  if (T == 0) return WIDE_OK;
  if (!aligned16(X) || !aligned16(mask) || !aligned16(W_gate) || !aligned16(W_up) ||
      !aligned16(W_down_packed) || !aligned16(Y) || (void*)Y == (void*)X)
    return WIDE_EINVAL;
  Carver probe(nullptr);
  carve_ffn(probe, T, d_model, d_ff, n_groups, mode);
  if (probe.used > (size_t)WIDE_NOALLOC_SCRATCH_BYTES) return WIDE_EWORKSPACE;
  void* ws = scratch_address();
  if (!ws) return WIDE_EHIP;
  // nothing in the scratch needs to start at zero: every element a kernel reads
  // there was written earlier in the same call
  Carver c(ws);
  FfnWs w = carve_ffn(c, T, d_model, d_ff, n_groups, mode);
  (void)hipGetLastError();
  ffn_run(X, mask, W_gate, W_up, W_down_packed, T, d_model, d_ff, n_groups, mode, nullptr, Y, w,
          as_stream(stream));
  return launch_status();
}

size_t wide_attn_proj_masked_workspace(int T, int d_model, const wide_attn_cfg* cfg, int mode,
                                       int kv_cap) {
  if (attn_check(T, d_model, cfg, mode) != WIDE_OK) return 0;
  if (mode == WIDE_DECODE && kv_cap < 1) return 0;
  Carver c(nullptr);
  carve_attn(c, T, d_model, cfg, mode, kv_cap);
  return c.used;
}

int wide_attn_proj_masked(const uint16_t* X, const uint8_t* mask, const uint16_t* Wq,
                          const uint16_t* Wk, const uint16_t* Wv, const uint16_t* Wo_packed,
                          int T, int d_model, const wide_attn_cfg* cfg, int mode,
                          uint16_t* K_cache, uint16_t* V_cache, int kv_len, int kv_cap,
                          uint16_t* Y, void* workspace, size_t workspace_bytes, uint32_t flags,
                          void* stream) {
  int st = attn_check(T, d_model, cfg, mode);
  if (st != WIDE_OK) return st;
  if (flags != 0) return WIDE_EINVAL;
  if (mode == WIDE_DECODE) {
    st = attn_decode_check(T, cfg, K_cache, V_cache, kv_len, kv_cap);
    if (st != WIDE_OK) return st;
  }
  if (T == 0) return WIDE_OK;
  if (!aligned16(X) || !aligned16(mask) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv) ||
      !aligned16(Wo_packed) || !aligned16(Y) || (void*)Y == (void*)X)
    return WIDE_EINVAL;
  Carver probe(nullptr);
  carve_attn(probe, T, d_model, cfg, mode, kv_cap);
  if (!aligned16(workspace)) return WIDE_EINVAL;
  if (workspace_bytes < probe.used) return WIDE_EWORKSPACE;
  Carver c(workspace);
  AttnWs w = carve_attn(c, T, d_model, cfg, mode, kv_cap);
  (void)hipGetLastError();
  attn_run(X, mask, Wq, Wk, Wv, Wo_packed, T, d_model, cfg, mode, K_cache, V_cache, kv_len, kv_cap,
           nullptr, Y, w, as_stream(stream));
  return launch_status();
}

int wide_attn_decode_masked_cache(const uint16_t* X, const uint8_t* mask, const uint16_t* Wq,
                                  const uint16_t* Wk, const uint16_t* Wv,
                                  const uint16_t* Wo_packed, int B, int d_model,
                                  const wide_attn_cfg* cfg, uint16_t* K_cache, uint16_t* V_cache,
                                  int kv_cap, const int32_t* kv_len, int pos, uint16_t* Y,
                                  void* workspace, size_t workspace_bytes, uint32_t flags,
                                  void* stream) {
  int st = attn_check(B, d_model, cfg, WIDE_DECODE);
  if (st != WIDE_OK) return st;
  if (flags != 0 || pos < 0) return WIDE_EINVAL;
  // the shape checks of a uniform-length call with the last slot in use
  st = attn_decode_check(B, cfg, K_cache, V_cache, kv_cap - 1, kv_cap);
  if (st != WIDE_OK) return st;
  if (B == 0) return WIDE_OK;
  if (!aligned16(X) || !aligned16(mask) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv) ||
      !aligned16(Wo_packed) || !aligned16(Y) || !aligned16(kv_len) || (void*)Y == (void*)X)
    return WIDE_EINVAL;
  if ((const void*)kv_len == (const void*)K_cache || (const void*)kv_len == (const void*)V_cache)
    return WIDE_EINVAL;
  Carver probe(nullptr);
  carve_attn(probe, B, d_model, cfg, WIDE_DECODE, kv_cap);
  if (!aligned16(workspace)) return WIDE_EINVAL;
  if (workspace_bytes < probe.used) return WIDE_EWORKSPACE;
  Carver c(workspace);
  AttnWs w = carve_attn(c, B, d_model, cfg, WIDE_DECODE, kv_cap);
  (void)hipGetLastError();
  attn_run(X, mask, Wq, Wk, Wv, Wo_packed, B, d_model, cfg, WIDE_DECODE, K_cache, V_cache, 0,
           kv_cap, nullptr, Y, w, as_stream(stream), kv_len, pos);
  return launch_status();
}

int wide_attn_decode_masked_paged(const uint16_t* X, const uint8_t* mask, const uint16_t* Wq,
                                  const uint16_t* Wk, const uint16_t* Wv,
                                  const uint16_t* Wo_packed, int B, int d_model,
                                  const wide_attn_cfg* cfg, uint16_t* K_pool, uint16_t* V_pool,
                                  int n_pages, int page_size, const int32_t* page_table,
                                  int max_pages, const int32_t* kv_len, int pos, uint16_t* Y,
                                  void* workspace, size_t workspace_bytes, uint32_t flags,
                                  void* stream) {
  int st = attn_check(B, d_model, cfg, WIDE_DECODE);
  if (st != WIDE_OK) return st;
  if (flags != 0 || pos < 0) return WIDE_EINVAL;
  if (page_size < 16 || (page_size & (page_size - 1)) || n_pages < 1 || max_pages < 1)
    return WIDE_EINVAL;
  if (!aligned16(K_pool) || !aligned16(V_pool) || K_pool == V_pool) return WIDE_EINVAL;
  // pool rows and one pair's slots each addressable by a 32-bit byte offset
  if (!fits((int64_t)n_pages * page_size, kHeadDim) ||
      !fits((int64_t)max_pages * page_size, kHeadDim))
    return WIDE_EUNSUPPORTED;
  const int kv_cap = max_pages * page_size;
  if (B == 0) return WIDE_OK;
  if (!aligned16(X) || !aligned16(mask) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv) ||
      !aligned16(Wo_packed) || !aligned16(Y) || !aligned16(kv_len) || !aligned16(page_table) ||
      (void*)Y == (void*)X)
    return WIDE_EINVAL;
  for (const void* p : {(const void*)kv_len, (const void*)page_table})
    if (p == (const void*)K_pool || p == (const void*)V_pool) return WIDE_EINVAL;
  Carver probe(nullptr);
  carve_attn(probe, B, d_model, cfg, WIDE_DECODE, kv_cap);
  if (!aligned16(workspace)) return WIDE_EINVAL;
  if (workspace_bytes < probe.used) return WIDE_EWORKSPACE;
  Carver c(workspace);
  AttnWs w = carve_attn(c, B, d_model, cfg, WIDE_DECODE, kv_cap);
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  const PagedKV pg{page_table, shift, n_pages};
  (void)hipGetLastError();
  attn_run(X, mask, Wq, Wk, Wv, Wo_packed, B, d_model, cfg, WIDE_DECODE, K_pool, V_pool, 0, kv_cap,
           nullptr, Y, w, as_stream(stream), kv_len, pos, true, &pg);
  return launch_status();
}

size_t wide_layer_masked_workspace(int T, const wide_layer_cfg* cfg, int mode, int kv_cap) {
  if (layer_check(T, cfg, mode) != WIDE_OK) return 0;
  if (mode == WIDE_DECODE && kv_cap < 1) return 0;
  Carver c(nullptr);
  carve_layer(c, T, cfg, mode, kv_cap);
  return c.used;
}

int wide_layer_masked(const uint16_t* X, const uint8_t* attn_mask, const uint8_t* ffn_mask,
                      const wide_layer_weights* W, const wide_layer_cfg* cfg, int T, int mode,
                      uint16_t* K_cache, uint16_t* V_cache, int kv_len, int kv_cap, uint16_t* Y,
                      void* workspace, size_t workspace_bytes, uint32_t flags, void* stream) {
  int st = layer_check(T, cfg, mode);
  if (st != WIDE_OK) return st;
  if ((flags & ~WIDE_FLAG_FFN_TOKEN_SORT) || !W) return WIDE_EINVAL;
  if (mode == WIDE_DECODE) {
    st = attn_decode_check(T, &cfg->attn, K_cache, V_cache, kv_len, kv_cap);
    if (st != WIDE_OK) return st;
  }
  if (T == 0) return WIDE_OK;
  if (!aligned16(X) || !aligned16(attn_mask) || !aligned16(ffn_mask) || !aligned16(Y) ||
      (void*)Y == (void*)X || !layer_weights_ok(W))
    return WIDE_EINVAL;
  Carver probe(nullptr);
  carve_layer(probe, T, cfg, mode, kv_cap);
  if (!aligned16(workspace)) return WIDE_EINVAL;
  if (workspace_bytes < probe.used) return WIDE_EWORKSPACE;
  Carver c(workspace);
  LayerWs w = carve_layer(c, T, cfg, mode, kv_cap);
  LayerCache kv;
  kv.K = K_cache, kv.V = V_cache, kv.kv_len = kv_len, kv.kv_cap = kv_cap;
  (void)hipGetLastError();
  return layer_run(X, attn_mask, ffn_mask, W, cfg, T, mode, kv, Y, w, as_stream(stream), false,
                   (flags & WIDE_FLAG_FFN_TOKEN_SORT) != 0);
}

int wide_layer_masked_routed(const uint16_t* X, const wide_layer_router* router,
                             const wide_layer_weights* W, const wide_layer_cfg* cfg, int T,
                             int mode, uint16_t* K_cache, uint16_t* V_cache, int kv_len,
                             int kv_cap, uint8_t* attn_mask, uint8_t* ffn_mask, uint16_t* Y,
                             void* workspace, size_t workspace_bytes, uint32_t flags,
                             void* stream) {
  int st = layer_check(T, cfg, mode);
  if (st != WIDE_OK) return st;
  if ((flags & ~WIDE_FLAG_FFN_TOKEN_SORT) || !W || !router) return WIDE_EINVAL;
  const int nkv = cfg->attn.n_kv_heads, n = cfg->n_ffn_groups;
  if (router->k_attn < 0 || router->k_attn > nkv || router->k_ffn < 0 || router->k_ffn > n)
    return WIDE_EINVAL;
  if (mode == WIDE_DECODE) {
    st = attn_decode_check(T, &cfg->attn, K_cache, V_cache, kv_len, kv_cap);
    if (st != WIDE_OK) return st;
  }
  if (T == 0) return WIDE_OK;
  if (!aligned16(X) || !aligned16(attn_mask) || !aligned16(ffn_mask) || !aligned16(Y) ||
      (void*)Y == (void*)X || !layer_weights_ok(W) || !aligned16(router->R_attn_packed) ||
      !aligned16(router->R_ffn_packed) || (void*)attn_mask == (void*)ffn_mask ||
      (const void*)attn_mask == (const void*)X || (const void*)ffn_mask == (const void*)X)
    return WIDE_EINVAL;
  Carver probe(nullptr);
  carve_layer(probe, T, cfg, mode, kv_cap);
  if (!aligned16(workspace)) return WIDE_EINVAL;
  if (workspace_bytes < probe.used) return WIDE_EWORKSPACE;
  Carver c(workspace);
  LayerWs w = carve_layer(c, T, cfg, mode, kv_cap);
  LayerCache kv;
  kv.K = K_cache, kv.V = V_cache, kv.kv_len = kv_len, kv.kv_cap = kv_cap;
  hipStream_t s = as_stream(stream);
  const bool prefill = mode == WIDE_PREFILL;
  (void)hipGetLastError();
  // the routers read the layer input; in prefill their packed words go straight
  // to the reorders' buffers
  launch_router_topk2(X, T, cfg->d_model, router->R_ffn_packed, n, router->k_ffn, ffn_mask,
                      prefill ? w.ffn.rv.packed : nullptr, router->R_attn_packed, nkv,
                      router->k_attn, attn_mask, prefill ? w.attn.rv.packed : nullptr, s);
  return layer_run(X, attn_mask, ffn_mask, W, cfg, T, mode, kv, Y, w, s, prefill,
                   (flags & WIDE_FLAG_FFN_TOKEN_SORT) != 0);
}

int wide_layer_decode_masked_cache(const uint16_t* X, const uint8_t* attn_mask,
                                   const uint8_t* ffn_mask, const wide_layer_weights* W,
                                   const wide_layer_cfg* cfg, int B, uint16_t* K_cache,
                                   uint16_t* V_cache, int kv_cap, const int32_t* kv_len, int pos,
                                   uint16_t* Y, void* workspace, size_t workspace_bytes,
                                   uint32_t flags, void* stream) {
  int st = layer_check(B, cfg, WIDE_DECODE);
  if (st != WIDE_OK) return st;
  if (flags != 0 || !W || pos < 0) return WIDE_EINVAL;
  st = attn_decode_check(B, &cfg->attn, K_cache, V_cache, kv_cap - 1, kv_cap);
  if (st != WIDE_OK) return st;
  if (B == 0) return WIDE_OK;
  if (!aligned16(X) || !aligned16(attn_mask) || !aligned16(ffn_mask) || !aligned16(Y) ||
      !aligned16(kv_len) || (void*)Y == (void*)X || !layer_weights_ok(W))
    return WIDE_EINVAL;
  if ((const void*)kv_len == (const void*)K_cache || (const void*)kv_len == (const void*)V_cache)
    return WIDE_EINVAL;
  Carver probe(nullptr);
  carve_layer(probe, B, cfg, WIDE_DECODE, kv_cap);
  if (!aligned16(workspace)) return WIDE_EINVAL;
  if (workspace_bytes < probe.used) return WIDE_EWORKSPACE;
  Carver c(workspace);
  LayerWs w = carve_layer(c, B, cfg, WIDE_DECODE, kv_cap);
  LayerCache kv;
  kv.K = K_cache, kv.V = V_cache, kv.kv_cap = kv_cap, kv.pair_len = kv_len, kv.pos = pos;
  (void)hipGetLastError();
  return layer_run(X, attn_mask, ffn_mask, W, cfg, B, WIDE_DECODE, kv, Y, w, as_stream(stream),
                   false);
}

int wide_layer_decode_masked_paged(const uint16_t* X, const uint8_t* attn_mask,
                                   const uint8_t* ffn_mask, const wide_layer_weights* W,
                                   const wide_layer_cfg* cfg, int B, uint16_t* K_pool,
                                   uint16_t* V_pool, int n_pages, int page_size,
                                   const int32_t* page_table, int max_pages,
                                   const int32_t* kv_len, int pos, uint16_t* Y, void* workspace,
                                   size_t workspace_bytes, uint32_t flags, void* stream) {
  int st = layer_check(B, cfg, WIDE_DECODE);
  if (st != WIDE_OK) return st;
  if (flags != 0 || !W || pos < 0) return WIDE_EINVAL;
  if (page_size < 16 || (page_size & (page_size - 1)) || n_pages < 1 || max_pages < 1)
    return WIDE_EINVAL;
  if (!aligned16(K_pool) || !aligned16(V_pool) || K_pool == V_pool) return WIDE_EINVAL;
  if (!fits((int64_t)n_pages * page_size, kHeadDim) ||
      !fits((int64_t)max_pages * page_size, kHeadDim))
    return WIDE_EUNSUPPORTED;
  const int kv_cap = max_pages * page_size;
  if (B == 0) return WIDE_OK;
  if (!aligned16(X) || !aligned16(attn_mask) || !aligned16(ffn_mask) || !aligned16(Y) ||
      !aligned16(kv_len) || !aligned16(page_table) || (void*)Y == (void*)X ||
      !layer_weights_ok(W))
    return WIDE_EINVAL;
  for (const void* p : {(const void*)kv_len, (const void*)page_table})
    if (p == (const void*)K_pool || p == (const void*)V_pool) return WIDE_EINVAL;
  Carver probe(nullptr);
  carve_layer(probe, B, cfg, WIDE_DECODE, kv_cap);
  if (!aligned16(workspace)) return WIDE_EINVAL;
  if (workspace_bytes < probe.used) return WIDE_EWORKSPACE;
  Carver c(workspace);
  LayerWs w = carve_layer(c, B, cfg, WIDE_DECODE, kv_cap);
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  const PagedKV pg{page_table, shift, n_pages};
  LayerCache kv;
  kv.K = K_pool, kv.V = V_pool, kv.kv_cap = kv_cap, kv.pair_len = kv_len, kv.pos = pos;
  kv.paged = &pg;
  (void)hipGetLastError();
  return layer_run(X, attn_mask, ffn_mask, W, cfg, B, WIDE_DECODE, kv, Y, w, as_stream(stream),
                   false);
}

}  // extern "C"
