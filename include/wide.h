/*
 * wide.h - C ABI of libwide: WIDE masked dynamic-width execution on MI355X (gfx950).
 *
 * What is computed (the pages about "WIDE: Boosting Adaptive LLM Inference via
 * Token-level Dynamic Width Pruning"):
 *   - every token keeps or skips each attention-head group and each FFN-channel
 *     group through a binary mask (gist.science technical summary, section 2.A);
 *   - the masks are reordered per group along the token dimension so the active
 *     tokens form a contiguous prefix (section 2.B);
 *   - kernels skip tiles, loads and matrix fragments that no kept token needs
 *     (section 2.C; the abstract's "hardware-agnostic block-level skipping" and
 *     "hardware-dependent intra-block skipping").
 * The result equals the dense layer with the dropped groups zeroed.
 *
 * Conventions shared by every entry point
 *   - All pointers except `cfg`/`W` structs are DEVICE pointers, owned by the
 *     caller, 16-byte aligned.  Calls allocate no device memory; scratch comes
 *     from the caller's workspace (wide_ffn_masked_noalloc: from a fixed array in
 *     the library).  Process-wide state, each item created on first use and kept
 *     until the process ends: per device, the scratch address
 *     (wide_ffn_masked_noalloc); the kernel trace while enabled.  Every call runs
 *     on `stream` alone.
 *   - bf16 tensors are passed as uint16_t bit patterns, row-major, contiguous.
 *   - Masks are uint8 [T, n_groups] row-major; any nonzero byte means "keep".
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue work:
 *     no host synchronisation, no device-to-host copy.  Faults during execution
 *     surface at the caller's next synchronisation.
 *   - Arguments are validated on the host before anything is enqueued; a call that
 *     returns an error has launched nothing.  T == 0 is a no-op returning WIDE_OK.
 *   - Inputs are never written.  Outputs must not alias inputs.  Every element of
 *     every output is written on success; dropped groups give an exact 0.
 *   - `flags` must be 0, except where a call names the bits it takes.
 *   - Concurrent calls are safe on different streams with distinct workspaces.
 */
#ifndef WIDE_H
#define WIDE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  WIDE_OK = 0,
  WIDE_EINVAL = 1,        /* NULL / misaligned pointer, inconsistent sizes       */
  WIDE_EUNSUPPORTED = 2,  /* valid but outside what the kernels implement         */
  WIDE_EWORKSPACE = 3,    /* workspace smaller than the matching *_workspace()   */
  WIDE_EHIP = 4           /* a HIP launch reported an error                       */
};
enum { WIDE_PREFILL = 0, WIDE_DECODE = 1 };

/* Limits: 1 <= n_groups <= 256, T <= 65536 (prefill); attention decode batch
 * <= 64 with at most 8 query heads per KV head.  A "decode" FFN call with more
 * than 64 tokens runs the prefill kernels. */
/* flags bit of wide_ffn_masked, wide_layer_masked and wide_layer_masked_routed
 * (prefill): besides the per-group partition, sort the tokens by the pattern of
 * their first 8 FFN groups (reflected Gray-code order) and run the K-masked FFN
 * down projection over that order, each 256-token tile over the union of its own
 * tokens' groups (the mask-pattern token permutation of gist.science technical
 * summary §2.B, and franklineh.com "Considerations for Implementation": tokens
 * with similar masks share the tiles whose dropped groups are skipped).  It pays
 * when masks cluster (tiles of one prototype share dropped blocks); with random
 * masks every tile keeps every group either way.  Results are bit-identical with
 * and without it: a token's sum runs over its own kept groups in ascending order
 * in any tile. */
#define WIDE_FLAG_FFN_TOKEN_SORT 0x2u

#define WIDE_MAX_GROUPS 256
#define WIDE_MAX_TOKENS 65536
#define WIDE_MAX_DECODE_BATCH 64

const char* wide_status_string(int status);
int wide_version(void);

/*
 * wide_mask_reorder - mask reordering (gist.science technical summary §2.B).
 *
 * For each group g, the tokens are sorted stably on "dropped" (kept first):
 *   group_count[g]     number of tokens that keep g
 *   group_perm[g, i]   token at position i (i < count: kept, ascending; then the
 *                      dropped ones, ascending) - a permutation of 0..T-1
 *   group_rank[g, t]   position of token t in group_perm[g]  (inverse permutation)
 * and for every tile of tile_m consecutive tokens (the last one may be short):
 *   tile_count[i]      number of groups kept by at least one token of tile i
 *   tile_groups[i, j]  those groups, ascending, then -1 up to n_groups
 * packed[t, w] bit j = mask[t, 64w + j] != 0 (little-endian words).
 *
 * mask        [T, n_groups] uint8              (input)
 * packed      [T, ceil(n_groups/64)] uint64    (output)
 * group_count [n_groups] int32;  group_perm, group_rank [n_groups, T] int32
 * tile_count  [ceil(T/tile_m)] int32;  tile_groups [ceil(T/tile_m), n_groups] int32
 *             (both NULL: no tile unions; the grouping and the packing then take one
 *             launch instead of two; one of them NULL: WIDE_EINVAL)
 * 1 <= tile_m <= 1024.  Results are bit-exact and deterministic.
 */
int wide_mask_reorder(const uint8_t* mask, int T, int n_groups, int tile_m,
                      uint64_t* packed, int32_t* group_count, int32_t* group_perm,
                      int32_t* group_rank, int32_t* tile_count, int32_t* tile_groups,
                      void* stream);

/*
 * wide_mask_reorder_packed - wide_mask_reorder from packed mask words (as
 * wide_router_topk writes them) instead of mask bytes: the same group_count,
 * group_perm, group_rank, tile_count and tile_groups, without the packing step
 * (gist.science technical summary §2.A router decisions feeding the §2.B
 * reordering directly).
 * packed [T, ceil(n_groups/64)] uint64 (input); bits past n_groups must be 0.
 * Other arguments, limits and errors as wide_mask_reorder.
 */
int wide_mask_reorder_packed(const uint64_t* packed, int T, int n_groups, int tile_m,
                             int32_t* group_count, int32_t* group_perm, int32_t* group_rank,
                             int32_t* tile_count, int32_t* tile_groups, void* stream);

/*
 * wide_router_topk - router and top-k selection, the step before the masked path
 * (gist.science technical summary §2.A: a router gives every token one binary
 * execute/skip decision per group; the abstract: each token selects its own
 * attention-head and FFN-channel groups).  A linear router without bias:
 *   logits[t, g] = sum_j X[t, j] R[g, j]      (bf16 inputs, fp32 accumulation)
 *   mask[t, g]   = 1 for the k largest logits of token t, else 0; ties go to the
 *                  lower group index, and -0.0 equals +0.0
 *   packed[t, w] bit j = mask[t, 64w + j]    (little-endian words, as
 *                  wide_mask_reorder packs them)
 * The selection is exact on the fp32 logits the call computes (returned when
 * `logits` is not NULL): every row keeps exactly k groups.
 *
 * X       [T, d_model] bf16                   (input)
 * R_packed the router weights R [n_groups, d_model] (group-major) in fragment
 *         order (wide_pack_router), bf16   (input)
 * logits  [T, n_groups] float32 or NULL       (output)
 * mask    [T, n_groups] uint8                 (output)
 * packed  [T, ceil(n_groups/64)] uint64 or NULL (output)
 * 1 <= n_groups <= 256, 0 <= k <= n_groups, d_model % 64 == 0, T <= 65536.
 */
int wide_router_topk(const uint16_t* X, const uint16_t* R_packed, int T, int d_model,
                     int n_groups, int k, float* logits, uint8_t* mask, uint64_t* packed,
                     void* stream);

/*
 * wide_pack_router - weight layout of wide_router_topk (done once per weight set):
 * R [n_groups, d_model] bf16 -> R_packed [ceil(n_groups/16) * 16 * d_model] bf16 in
 * the order the router's matrix-core fragments read it: block (j, s) for group tile
 * j = 0 .. ceil(n/16)-1 and K step s = 0 .. d_model/32-1 holds 64 rows of 8 values,
 * row l = R[16 j + (l mod 16), 32 s + 8 (l / 16) .. +7] (zeros past n_groups).
 * 1 <= n_groups <= 256, d_model % 64 == 0.
 */
int wide_pack_router(const uint16_t* R, int n_groups, int d_model, uint16_t* R_packed,
                     void* stream);

/*
 * wide_pack_kmajor - lay out a K-masked weight for the library (a pure permutation).
 *
 * W [n_groups * G, d_model] is the mathematical matrix of Y = H @ W (FFN down:
 * W_down [d_ff, d_model]; attention out: Wo [n_q*head_dim, d_model], which is
 * o_proj.weight transposed).  W_packed [n_groups, d_model, G] holds, for every
 * group g, the block W[gG:(g+1)G, :] transposed, so each group's block is one
 * contiguous region with the contraction index innermost.  Run once at weight load.
 * G a multiple of 64, or 32; d_model a multiple of 64.
 */
int wide_pack_kmajor(const uint16_t* W, int n_groups, int G, int d_model, uint16_t* W_packed,
                     void* stream);

/*
 * wide_ffn_masked - masked SwiGLU FFN (gist.science §2.A: contiguous channel groups
 * of the intermediate dimension D'; one binary execute/skip bit per token and group).
 *
 *   Y[t] = sum over groups g kept by t of  silu(X[t] Wg_g^T) * (X[t] Wu_g^T) @ Wd_g
 *
 * X             [T, d_model] bf16
 * mask          [T, n_groups] uint8
 * W_gate, W_up  [d_ff, d_model] bf16 (nn.Linear layout; group g = rows gG..gG+G-1)
 * W_down_packed [n_groups, d_model, G] bf16 (wide_pack_kmajor of W_down [d_ff, d_model])
 * Y             [T, d_model] bf16 (a token that keeps no group gets exact zeros)
 * mode          WIDE_PREFILL (any T) or WIDE_DECODE (T = batch; weight streaming over
 *               the groups the batch keeps when T <= 64)
 * Needs G = d_ff / n_groups a multiple of 64, or 32 (groups of 32 run at a lower
 * rate: every kept row is multiplied by 64 weight columns at a time), and d_model
 * a multiple of 64.
 */
size_t wide_ffn_masked_workspace(int T, int d_model, int d_ff, int n_groups, int mode);
int wide_ffn_masked(const uint16_t* X, const uint8_t* mask, const uint16_t* W_gate,
                    const uint16_t* W_up, const uint16_t* W_down_packed, int T, int d_model,
                    int d_ff, int n_groups, int mode, uint16_t* Y, void* workspace,
                    size_t workspace_bytes, uint32_t flags, void* stream);

/*
 * wide_ffn_masked_f32 - the masked SwiGLU FFN of wide_ffn_masked (gist.science §2.A)
 * computed in fp32 throughout: fp32 inputs, weights, intermediate H and output, fp32
 * products and sums on the vector units (no bf16 rounding anywhere).  For problems
 * that are checked at fp32 precision, such as a tiny FFN layer given in fp32; it
 * runs far below the bf16 path's rate.
 *
 * X              [T, d_model] fp32
 * mask           [T, n_groups] uint8
 * W_gate, W_up   [d_ff, d_model] fp32 (group g = rows gG..gG+G-1)
 * W_down         [d_ff, d_model] fp32, as is (the matrix of Y = H @ W_down; no packing)
 * Y              [T, d_model] fp32 (a token that keeps no group gets exact zeros)
 * Any group size G = d_ff / n_groups and any d_model.  Workspace:
 * wide_ffn_masked_f32_workspace() bytes (H).  Each output is one fixed-order sum, so a
 * repeated call gives the same bits.  Errors and conventions as wide_ffn_masked
 * (pointers 16-byte aligned, T <= WIDE_MAX_TOKENS, n_groups <= WIDE_MAX_GROUPS).
 */
size_t wide_ffn_masked_f32_workspace(int T, int d_model, int d_ff, int n_groups);
int wide_ffn_masked_f32(const float* X, const uint8_t* mask, const float* W_gate,
                        const float* W_up, const float* W_down, int T, int d_model, int d_ff,
                        int n_groups, float* Y, void* workspace, size_t workspace_bytes,
                        uint32_t flags, void* stream);

/*
 * wide_ffn_masked_noalloc - wide_ffn_masked for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes no workspace and allocates nothing (no hipMalloc, hipFree or
 * allocating library call); the caller still passes the inputs and Y.
 *
 * Scratch: a fixed device array of WIDE_NOALLOC_SCRATCH_BYTES inside the library,
 * one per GPU, held from the library's load on that GPU until the process ends.
 * Its device address is looked up once per device, on the first call there.
 * Limit: a call whose wide_ffn_masked_workspace(T, d_model, d_ff, n_groups, mode)
 * exceeds WIDE_NOALLOC_SCRATCH_BYTES returns WIDE_EWORKSPACE and launches nothing
 * (e.g. decode batches up to 64 fit at d_model 4096, d_ff 14336 in 112 groups).
 * Concurrency: every call on one GPU uses that GPU's one array.  Calls ordered on one
 * stream are safe; calls that may run at the same time on one GPU (different
 * streams, or several host threads) race on the scratch and give wrong results.
 * The scratch keeps the last call's contents; nothing in it needs to start at zero.
 * Arguments, results and errors otherwise as wide_ffn_masked; WIDE_EHIP also when
 * HIP cannot give the scratch address.
 */
#define WIDE_NOALLOC_SCRATCH_BYTES (16u << 20)
int wide_ffn_masked_noalloc(const uint16_t* X, const uint8_t* mask, const uint16_t* W_gate,
                            const uint16_t* W_up, const uint16_t* W_down_packed, int T,
                            int d_model, int d_ff, int n_groups, int mode, uint16_t* Y,
                            uint32_t flags, void* stream);

/*
 * wide_attn_proj_masked - masked attention sublayer over GQA-aligned head groups
 * (gist.science §2.A).  Group g = KV head g and query heads g*r .. g*r+r-1,
 * r = n_q_heads / n_kv_heads.  A token that drops g has no q/k/v in g and gets a
 * zero output for g's heads; a token that keeps g attends (causally) to the tokens
 * that also keep g.  Scale 1/sqrt(head_dim).  RoPE (rotate-half, angle
 * pos * theta^(-2i/head_dim)) when rope_theta > 0.
 *
 * X        [T, d_model] bf16
 * mask     [T, n_kv_heads] uint8
 * Wq       [n_q*hd, d_model], Wk, Wv [n_kv*hd, d_model] bf16 (nn.Linear layout)
 * Wo_packed[n_kv, d_model, r*hd] bf16 (wide_pack_kmajor of Wo [n_q*hd, d_model])
 * Y        [T, d_model] bf16 = O @ Wo
 * Prefill: positions 0..T-1; K_cache/V_cache may be NULL and are not touched.
 * Decode : T = batch; one new token per sequence at position kv_len (0 <= kv_len <
 *          kv_cap); K_cache, V_cache [T, n_kv, kv_cap, hd] bf16 hold kv_len valid
 *          entries per (sequence, group).  For every kept (sequence, group) the new
 *          roped k and v are written to slot kv_len; other slots are not written.
 * Needs head_dim == 128.
 */
typedef struct {
  int n_q_heads;
  int n_kv_heads;
  int head_dim;
  float rope_theta; /* 0 = no RoPE */
} wide_attn_cfg;

/* Workspace bytes for a call with these sizes (0 for invalid arguments).  kv_cap is
 * the cache capacity of decode calls (the split-KV partials scale with it); it is
 * ignored in prefill. */
size_t wide_attn_proj_masked_workspace(int T, int d_model, const wide_attn_cfg* cfg, int mode,
                                       int kv_cap);
int wide_attn_proj_masked(const uint16_t* X, const uint8_t* mask, const uint16_t* Wq,
                          const uint16_t* Wk, const uint16_t* Wv, const uint16_t* Wo_packed,
                          int T, int d_model, const wide_attn_cfg* cfg, int mode,
                          uint16_t* K_cache, uint16_t* V_cache, int kv_len, int kv_cap,
                          uint16_t* Y, void* workspace, size_t workspace_bytes, uint32_t flags,
                          void* stream);

/*
 * wide_attn_decode_masked_cache - one decode step of the masked attention sublayer
 * over caches in which tokens that skipped a group left no entry (gist.science
 * §2.A groups, with wide_attn_proj_masked's reading that a token sees only the
 * earlier tokens that also kept its group, carried across decode steps).
 *
 * kv_len  [B, n_kv_heads] int32 (device, input): the number of valid entries of
 *         each (sequence, group) cache, slots 0 .. kv_len-1.  A kept (b, g) writes
 *         the new roped k and v at slot kv_len[b, g] and attends to slots
 *         0 .. kv_len[b, g] (the new token included); a dropped pair writes nothing
 *         and outputs zero.  A length outside [0, kv_cap) behaves like a dropped pair
 *         (nothing written, zero output).  The library does not change kv_len: after
 *         the call the caller advances it by the mask (kv_len += mask != 0).
 * pos     RoPE position of the new tokens (>= 0; one position for the batch).
 * Other arguments as wide_attn_proj_masked in decode mode (B <= 64, head_dim 128);
 * workspace: wide_attn_proj_masked_workspace(B, d_model, cfg, WIDE_DECODE, kv_cap).
 */
int wide_attn_decode_masked_cache(const uint16_t* X, const uint8_t* mask, const uint16_t* Wq,
                                  const uint16_t* Wk, const uint16_t* Wv,
                                  const uint16_t* Wo_packed, int B, int d_model,
                                  const wide_attn_cfg* cfg, uint16_t* K_cache, uint16_t* V_cache,
                                  int kv_cap, const int32_t* kv_len, int pos, uint16_t* Y,
                                  void* workspace, size_t workspace_bytes, uint32_t flags,
                                  void* stream);

/*
 * wide_attn_decode_masked_paged - wide_attn_decode_masked_cache over a paged cache:
 * the (sequence, group) caches live in pages of a shared pool, found through a page
 * table (the paged layout of the masked-cache decode, gist.science §2.A groups;
 * the pages give no page format, this one is the library's own).
 *
 * K_pool, V_pool [n_pages, page_size, 128] bf16 (device, in/out): page p holds
 *         page_size consecutive slots of one (sequence, group) cache.
 * page_size   power of two, >= 16.
 * page_table  [B, n_kv_heads, max_pages] int32 (device, input): slot s of pair
 *         (b, g) is row s % page_size of page page_table[b, g, s / page_size];
 *         a pair holds up to max_pages * page_size slots.  An entry outside
 *         [0, n_pages) is an unmapped page: its slots read as zero keys and values
 *         and take no write.  A pair whose new slot kv_len[b, g] is on an unmapped
 *         page behaves like a dropped pair (nothing written, zero output).
 *         Pages may be shared between pairs for reading; the new slots of the kept
 *         pairs must be distinct pool rows (two writes to one row race).
 * kv_len  [B, n_kv_heads] int32 (device, input): as in
 *         wide_attn_decode_masked_cache, with kv_cap = max_pages * page_size.
 * Other arguments as wide_attn_decode_masked_cache; workspace:
 * wide_attn_proj_masked_workspace(B, d_model, cfg, WIDE_DECODE, max_pages * page_size).
 * All pointers 16-byte aligned.  Returns WIDE_EINVAL for a bad page size, pool or
 * table, WIDE_EUNSUPPORTED when n_pages * page_size or max_pages * page_size rows
 * of 256 bytes pass 2 GiB.
 */
int wide_attn_decode_masked_paged(const uint16_t* X, const uint8_t* mask, const uint16_t* Wq,
                                  const uint16_t* Wk, const uint16_t* Wv,
                                  const uint16_t* Wo_packed, int B, int d_model,
                                  const wide_attn_cfg* cfg, uint16_t* K_pool, uint16_t* V_pool,
                                  int n_pages, int page_size, const int32_t* page_table,
                                  int max_pages, const int32_t* kv_len, int pos, uint16_t* Y,
                                  void* workspace, size_t workspace_bytes, uint32_t flags,
                                  void* stream);

/*
 * wide_layer_masked - one pre-norm decoder layer with both masked sublayers:
 *   u = RMSNorm(x; rms1), h = x + Attn(u; attn_mask), w = RMSNorm(h; rms2),
 *   y = h + FFN(w; ffn_mask),  RMSNorm(x) = x / sqrt(mean(x^2) + eps) * gamma.
 * Weights as in the two calls above; rms1, rms2 [d_model] bf16.  Same prefill /
 * decode and cache rules as wide_attn_proj_masked.  With all-zero masks y == x.
 * Prefill runs the first RMSNorm and both mask reorders in one launch (the
 * reorders read only the masks, so they run beside the norm rows), then the
 * attention kernels, the second RMSNorm and the FFN kernels, all on `stream`.
 */
typedef struct {
  const uint16_t* rms1;
  const uint16_t* Wq;
  const uint16_t* Wk;
  const uint16_t* Wv;
  const uint16_t* Wo_packed;
  const uint16_t* rms2;
  const uint16_t* W_gate;
  const uint16_t* W_up;
  const uint16_t* W_down_packed;
} wide_layer_weights;

typedef struct {
  int d_model;
  int d_ff;
  int n_ffn_groups;
  wide_attn_cfg attn;
  float rms_eps;
} wide_layer_cfg;

size_t wide_layer_masked_workspace(int T, const wide_layer_cfg* cfg, int mode, int kv_cap);
int wide_layer_masked(const uint16_t* X, const uint8_t* attn_mask, const uint8_t* ffn_mask,
                      const wide_layer_weights* W, const wide_layer_cfg* cfg, int T, int mode,
                      uint16_t* K_cache, uint16_t* V_cache, int kv_len, int kv_cap, uint16_t* Y,
                      void* workspace, size_t workspace_bytes, uint32_t flags, void* stream);

/*
 * wide_layer_masked_routed - wide_layer_masked with the masks chosen on the GPU by
 * two linear routers on the layer input (gist.science technical summary §2.A: a
 * router gives every token one binary execute/skip decision per group; its
 * decisions go straight to the §2.B reordering):
 *   attn_mask = top-k_attn of X R_attn^T,  ffn_mask = top-k_ffn of X R_ffn^T
 * with wide_router_topk's rule (ties to the lower group index).  In prefill the
 * routers' packed words feed the mask reorders directly (no packing step).
 *
 * router->R_attn_packed  wide_pack_router of R_attn [n_kv_heads, d_model] (input)
 * router->R_ffn_packed   wide_pack_router of R_ffn [n_ffn_groups, d_model] (input)
 * router->k_attn, k_ffn  groups each token keeps (0 .. n_kv_heads, 0 .. n_ffn_groups)
 * attn_mask [T, n_kv_heads], ffn_mask [T, n_ffn_groups] uint8 (outputs, 1 = keep)
 * Other arguments as wide_layer_masked; workspace: wide_layer_masked_workspace.
 */
typedef struct {
  const uint16_t* R_attn_packed;
  const uint16_t* R_ffn_packed;
  int k_attn;
  int k_ffn;
} wide_layer_router;

int wide_layer_masked_routed(const uint16_t* X, const wide_layer_router* router,
                             const wide_layer_weights* W, const wide_layer_cfg* cfg, int T,
                             int mode, uint16_t* K_cache, uint16_t* V_cache, int kv_len,
                             int kv_cap, uint8_t* attn_mask, uint8_t* ffn_mask, uint16_t* Y,
                             void* workspace, size_t workspace_bytes, uint32_t flags,
                             void* stream);

/*
 * wide_layer_decode_masked_cache - one decode step of the whole layer over attention
 * caches in which tokens that skipped a group left no entry (gist.science §2.A
 * groups; the reading of wide_attn_decode_masked_cache carried across decode
 * steps): u = RMSNorm(x), h = x + Attn(u) with per-(sequence, group) cache
 * lengths kv_len [B, n_kv_heads] (device, input, not modified: the caller
 * advances it by attn_mask after the call) and RoPE position pos for the new
 * tokens, w = RMSNorm(h), y = h + FFN(w; ffn_mask).
 * Cache rules as wide_attn_decode_masked_cache (kept pairs append at slot
 * kv_len[b, g]; a length outside [0, kv_cap) acts as a dropped pair).
 * B <= 64; workspace: wide_layer_masked_workspace(B, cfg, WIDE_DECODE, kv_cap).
 */
int wide_layer_decode_masked_cache(const uint16_t* X, const uint8_t* attn_mask,
                                   const uint8_t* ffn_mask, const wide_layer_weights* W,
                                   const wide_layer_cfg* cfg, int B, uint16_t* K_cache,
                                   uint16_t* V_cache, int kv_cap, const int32_t* kv_len, int pos,
                                   uint16_t* Y, void* workspace, size_t workspace_bytes,
                                   uint32_t flags, void* stream);

/*
 * wide_layer_decode_masked_paged - wide_layer_decode_masked_cache over a paged
 * cache: pools, page table and lengths exactly as wide_attn_decode_masked_paged.
 * Workspace: wide_layer_masked_workspace(B, cfg, WIDE_DECODE, max_pages * page_size).
 */
int wide_layer_decode_masked_paged(const uint16_t* X, const uint8_t* attn_mask,
                                   const uint8_t* ffn_mask, const wide_layer_weights* W,
                                   const wide_layer_cfg* cfg, int B, uint16_t* K_pool,
                                   uint16_t* V_pool, int n_pages, int page_size,
                                   const int32_t* page_table, int max_pages,
                                   const int32_t* kv_len, int pos, uint16_t* Y, void* workspace,
                                   size_t workspace_bytes, uint32_t flags, void* stream);

/*
 * Kernel timing, for benchmarking (not part of the method).  While enabled, each
 * kernel launch the library makes is bracketed by two HIP events on its stream.
 *   wide_trace_enable(on)   start (on != 0) or stop recording; returns 0
 *   wide_trace_collect()    waits for the recorded events, folds them into
 *                           per-kernel totals; returns the number of distinct
 *                           kernels, or -1 if a HIP event query failed
 *   wide_trace_get(i, ...)  name (NUL-terminated, truncated to name_len), launch
 *                           count and summed milliseconds of kernel i; 0 on
 *                           success, 1 for a bad index or NULL argument
 *   wide_trace_reset()      drops all records and totals
 * The trace is process-wide state guarded by a mutex.
 */
int wide_trace_enable(int on);
int wide_trace_collect(void);
int wide_trace_get(int i, char* name, int name_len, int* launches, double* total_ms);
void wide_trace_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* WIDE_H */
