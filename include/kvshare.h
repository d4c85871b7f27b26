/*
 * kvshare.h -- C ABI of a cross-layer shared-KV attention library for AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed.  GQA attention in which transformer layer l attends over
 * the cached keys/values of the layer(s) a sharing map names for it:
 *   - adjacent sharing (Cross-Layer Attention, "Reducing Transformer
 *     Key-Value Cache Size with Cross-Layer Attention", Methodology and
 *     Abstract: some layers compute K/V, the following ones reuse it);
 *   - any "bottom" partitioning of the unified framework of "A Systematic
 *     Study of Cross-Layer KV Sharing for Efficient LLM Inference" (TL;DR):
 *     every source at or below its reader;
 *   - two-source mixing (DepthGraft, "DepthGraft: Structural Regularization
 *     through Hierarchical Cross-Layer KV Reconstruction", Abstract: deep-layer
 *     K/V rebuilt from stride-aligned shallow/middle source pairs), read as
 *     K~ = w1 K_s1 + w2 K_s2 (same weights for V);
 *   - a factorized cache (DepthWeave-KV, "DepthWeave-KV: Smarter KV Cache
 *     Compression by Sharing Across Layers and Adapting Per Token", Core
 *     Mechanism and Framework Shift): K_l[t] = c[t] B_pair
 *     + s_l[t] * sum_{j<r_t} d_l[t,j] U_l[j], V alike, c/B shared by a layer
 *     pair, int8 codes d with an fp16 per-token scale s, rank r_t per token.
 * Attention is softmax(q K~^T / sqrt(head_dim)) V~, query head h reading K/V
 * head floor(h / (n_q_heads / n_kv_heads)).
 *
 * Conventions for every call.
 *   - The library never allocates device memory and never creates streams.
 *     All device buffers (cache pools, page table, queries, outputs,
 *     workspace) are owned by the caller; sizes come from kvs_cache_layout()
 *     and kvs_decode_workspace_size().
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Compute calls are asynchronous on that stream; device faults surface at
 *     the caller's next synchronisation.
 *   - Arguments are validated on the host before any HIP call; on error the
 *     call returns a non-zero kvs_status, launches nothing, and
 *     kvs_last_error() (thread-local) describes the problem.
 *   - Device pointers to tensors must be 16-byte aligned (KVS_ERR_ALIGN).
 *   - Tensors are dense and row-major in the shapes given.
 *   - "bf16" data is passed as raw 16-bit bfloat16 patterns.
 */
#ifndef KVSHARE_H
#define KVSHARE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define KVS_API __attribute__((visibility("default")))
#else
#define KVS_API
#endif

typedef enum {
  KVS_OK = 0,
  KVS_ERR_ARG = 1,          /* null pointer, size or enum out of range         */
  KVS_ERR_MAP = 2,          /* malformed sharing map row                        */
  KVS_ERR_NOT_SOURCE = 3,   /* map names a non-owner as source; append to a
                               layer that owns no cache entries                 */
  KVS_ERR_RANGE = 4,        /* count beyond cache capacity or workspace size    */
  KVS_ERR_UNSUPPORTED = 5,  /* valid request the library does not implement
                               (an unsupported head_dim / group size / dtype /
                               rank combination)                                */
  KVS_ERR_ALIGN = 6,        /* a device pointer is not 16-byte aligned          */
  KVS_ERR_HIP = 7           /* a HIP launch failed                              */
} kvs_status;

typedef enum { KVS_F32 = 0, KVS_BF16 = 1 } kvs_dtype;
typedef enum { KVS_DENSE = 0, KVS_FACTORIZED = 1 } kvs_kind;

/* Model and capacity description. */
typedef struct {
  int32_t n_layers;        /* L >= 1                                           */
  int32_t n_q_heads;       /* Hq, multiple of n_kv_heads                        */
  int32_t n_kv_heads;      /* Hkv                                               */
  int32_t head_dim;        /* hd: 64 or 128                                     */
  int32_t dtype;           /* kvs_dtype of the dense cache and the queries;
                              the factorized cache is bf16                      */
  int32_t kind;            /* kvs_kind                                          */
  int32_t basis_rank;      /* factorized: R, basis rows per pair (32)          */
  int32_t resid_rank_max;  /* factorized: Rmax, residual codes per token (16)  */
  int32_t max_batch;       /* sequences the cache holds                        */
  int32_t max_ctx;         /* tokens per sequence the cache holds               */
} kvs_config;

/* Immutable host-side plan built from a sharing map.  Thread-safe to share. */
typedef struct kvs_plan kvs_plan;

/* What one layer reads.  Owner slots are numbered 0.. in ascending order of
 * the layers that own cache entries. */
typedef struct {
  int32_t owns_kv;         /* 1: the layer writes its own cache entries        */
  int32_t n_src;           /* 1 or 2                                            */
  int32_t src_layer[2];    /* source layers (-1 when unused)                    */
  int32_t src_slot[2];     /* their owner slots (-1 when unused)                */
  float   weight[2];       /* mixing weights as stored (fp32)                   */
  int32_t masks_current;   /* 1: a source sits above the layer (top/middle
                              configuration), so the layer's query sees only
                              earlier positions (diagonal masking)           */
} kvs_layer_info;

typedef struct {
  int32_t n_layers;
  int32_t n_slots;           /* owner slots = layers holding cache entries     */
  int32_t last_owner_layer;  /* deepest owner; deeper layers write no cache     */
  int32_t n_mixed_layers;    /* layers reading two sources                      */
} kvs_plan_info;

/* Byte sizes of the caller-allocated device buffers.  Pool layouts (64-token
 * pages; page p of sequence b lives in physical page page_table[b][p]):
 *   dense K pool  [n_slots][n_phys_pages][Hkv][8][hd/(8E)][8][8][E],
 *                 E = 16 B / elem: chunk c (E elements) of token t of a page
 *                 at (((t/8)*(hd/(8E)) + c/8)*64 + 8*(t%8) + c%8)*E
 *   dense V pool  [n_slots][n_phys_pages][Hkv][32][hd][2]     token pairs
 *                 (element (t, d) of a page at (t/2)*hd*2 + d*2 + t%2)
 *   page table    [max_batch][pages_per_seq] int32 in [0, n_phys_pages)
 *   factorized (R = 32, Rmax = 16), per (page, KV head):
 *     cK   [n_slots][n_phys_pages][Hkv][4][64][8] bf16: coefficients
 *          8c..8c+7 of token t at (c*64 + t)*8
 *     cV   [n_slots][n_phys_pages][Hkv][4][64][2][4] bf16: coefficient i of
 *          token t at ((m/2)*64 + 4*(t/4) + i%4)*8 + (m%2)*4 + t%4, m = i/4
 *     dK / dV  [n_layers][n_phys_pages][Hkv][128][8] int8: rank-packed code
 *          granules; token t owns ceil(r_t/8) granules starting at granule
 *          o_t = sum over the page's earlier tokens of ceil(r/8); codes
 *          j >= r_t inside them are zero
 *     sK / sV  [n_layers][n_phys_pages][Hkv][64] fp16
 *     rank (the meta pool) [n_phys_pages][64] uint16 = r_t | o_t << 8 (shared
 *          by all layers and heads)
 *     BK / BV  [n_slots][Hkv][R][hd] bf16;  UK / UV  [n_layers][Hkv][Rmax][hd]
 *          bf16 (written by the caller, e.g. with kvs_pair_basis and
 *          kvs_residual_basis)                                             */
typedef struct {
  int32_t page_tokens;         /* 64                                           */
  int32_t pages_per_seq;       /* ceil(max_ctx / 64)                           */
  int32_t n_phys_pages;        /* max_batch * pages_per_seq                    */
  int32_t n_slots;
  size_t  k_pool_bytes;        /* dense: each of the K and V pools             */
  size_t  v_pool_bytes;
  size_t  page_table_bytes;
  size_t  coef_pool_bytes;     /* factorized: each of cK, cV                   */
  size_t  resid_pool_bytes;    /* factorized: each of dK, dV                   */
  size_t  scale_pool_bytes;    /* factorized: each of sK, sV                   */
  size_t  rank_pool_bytes;     /* factorized: the meta pool (rank, offset)     */
  size_t  basis_bytes;         /* factorized: each of BK, BV                   */
  size_t  resid_basis_bytes;   /* factorized: each of UK, UV                   */
} kvs_cache_sizes;

/* Device pointers of one cache instance (all caller-owned). */
typedef struct {
  void* k_pool;
  void* v_pool;
  const int32_t* page_table;
  void* ck_pool;
  void* cv_pool;
  void* dk_pool;
  void* dv_pool;
  void* sk_pool;
  void* sv_pool;
  void* rank_pool;
  const void* basis_k;
  const void* basis_v;
  const void* ubasis_k;
  const void* ubasis_v;
} kvs_cache;

/* ---------------------------------------------------------------- planning */

/* Build a plan from a sharing map.
 *   src  [n_layers][2] host int32: source layers of each layer; the second
 *        entry is -1 for a single source.  A layer owns its cache entries iff
 *        its row is (l, -1) with weight 1.
 *   w    [n_layers][2] host float or NULL (NULL: all weights 1).
 * Rules (first violation wins, layers scanned in order): indices in range and
 * weights finite, else KVS_ERR_MAP; a row naming its own layer must be the
 * plain owner row, else KVS_ERR_MAP; a source that owns no entries ->
 * KVS_ERR_NOT_SOURCE (reusing layers compute no K/V, CLA Methodology, so
 * chains are invalid).  A source may sit above its reader (the top/middle
 * configurations of "A Systematic Study of Cross-Layer KV Sharing for
 * Efficient LLM Inference", TL;DR): that source writes the current token's
 * entry only after the reader has run, so the reader's decode query sees
 * positions 0..seq_len-2 and its causal prefill query at position P sees
 * keys 0..P-1 (diagonal masking; a query with no key yields zeros).  KVS_FACTORIZED plans take single
 * sources only: src[l][0] is the layer that writes the pair's coefficients.  A factorized
 * cache must satisfy max_batch * ceil(max_ctx/64) * n_kv_heads <= 2^19 (its
 * pools are addressed with 32-bit offsets per slot and layer), else
 * KVS_ERR_UNSUPPORTED.
 * On success *out receives a plan to release with kvs_plan_free(). */
KVS_API kvs_status kvs_share_plan(const kvs_config* cfg, const int32_t* src,
                                  const float* w, kvs_plan** out);
KVS_API void kvs_plan_free(kvs_plan* plan);
KVS_API kvs_status kvs_plan_layer(const kvs_plan* plan, int32_t layer,
                                  kvs_layer_info* out);
KVS_API kvs_status kvs_plan_summary(const kvs_plan* plan, kvs_plan_info* out);
KVS_API kvs_status kvs_cache_layout(const kvs_plan* plan, kvs_cache_sizes* out);

/* Split-K partitions per (sequence, KV head) the decode uses when n_splits=0
 * is passed to kvs_attn_decode: chosen from batch, KV heads, the longest
 * sequence and the plan's decode kernel so the launch fills the GPU (one
 * workgroup per CU for the factorized and MFMA kernels; for the dot-product
 * kernel three per four CUs (192) on calls streaming more than 384 MB and on
 * smaller calls whose (sequence, KV head) pairs reach 192 to 224 workgroups
 * with a whole number of partitions, otherwise four per CU (at most 32
 * partitions) on smaller calls, one per CU for groups of 8 heads); at least
 * 4 pages per partition, at most 64 partitions; partition boundaries fall
 * on 64-key page boundaries. */
KVS_API kvs_status kvs_decode_splits(const kvs_plan* plan, int32_t batch,
                                     int32_t max_seq_len, int32_t* n_splits);
/* Workspace bytes kvs_attn_decode needs for (batch, n_splits), n_splits in
 * [1, 64]: per-partition partial results, maxima and sums (fp32).  Calls
 * sharing a workspace must not overlap in time. */
KVS_API kvs_status kvs_decode_workspace_size(const kvs_plan* plan, int32_t batch,
                                             int32_t n_splits, size_t* bytes);

/* ----------------------------------------------------------------- writing */

/* Write n new tokens' K/V of an owner layer into its slot.  Only layers that
 * compute their own K/V store them; the layers that reuse them store nothing
 * ("Reducing Transformer Key-Value Cache Size with Cross-Layer Attention",
 * Methodology: some layers compute fresh K/V, the layers after them reuse
 * those; Abstract: the cache holds the owners' entries only).
 *   k, v       device [batch][n][Hkv][hd], cache dtype
 *   start_pos  device int32 [batch]: token i of sequence b goes to position
 *              start_pos[b] + i.  Positions outside [0, max_ctx), or whose
 *              page-table entry is outside [0, n_phys_pages), are skipped.
 * Errors: layer not an owner -> KVS_ERR_NOT_SOURCE; n > max_ctx or
 * batch > max_batch -> KVS_ERR_RANGE; factorized plan -> KVS_ERR_ARG. */
KVS_API kvs_status kvs_append(const kvs_plan* plan, const kvs_cache* cache, int32_t layer,
                              const void* k, const void* v, int32_t n,
                              const int32_t* start_pos, int32_t batch, void* stream);

/* Factorized write of n tokens for `layer`: the entries of the factorized
 * cache of "DepthWeave-KV: Smarter KV Cache Compression by Sharing Across
 * Layers and Adapting Per Token" (Core Mechanism: coefficients on a basis
 * shared by a layer pair, and a per-layer low-rank residual kept as int8
 * codes; Framework Shift: the residual's rank is chosen per token).
 *   ck, cv     device bf16 [batch][n][Hkv][R]: the pair coefficients; given
 *              only by the layer that owns the pair's slot (else NULL)
 *   dk, dv     device int8 [batch][n][Hkv][Rmax]; codes at j >= r_t are
 *              ignored (stored as zero)
 *   sk, sv     device fp16 [batch][n][Hkv]
 *   rank       device uint8 [batch][n] (values above Rmax count as Rmax);
 *              required on every call: a token's codes are placed after those
 *              of the page's earlier tokens, so tokens of a page are appended
 *              in position order and a token's rank, shared by all layers,
 *              never changes once written
 *   start_pos  as for kvs_append.
 * Errors as for kvs_append; ck given for a layer that does not own its pair's
 * slot -> KVS_ERR_NOT_SOURCE. */
KVS_API kvs_status kvs_append_factorized(const kvs_plan* plan, const kvs_cache* cache,
                                         int32_t layer, const void* ck, const void* cv,
                                         const int8_t* dk, const int8_t* dv,
                                         const void* sk, const void* sv,
                                         const uint8_t* rank, int32_t n,
                                         const int32_t* start_pos, int32_t batch,
                                         void* stream);

/* --------------------------------------------- factorized write side (encoder)
 * The factorized cache of "DepthWeave-KV: Smarter KV Cache Compression by
 * Sharing Across Layers and Adapting Per Token" (Core Mechanism): a channel
 * basis computed from a pair of neighbouring layers' own K/V, without
 * training, and a small low-rank quantized residual per layer.  The page
 * gives no numerical recipe; these calls implement the readings
 *   c_t = bf16(B x^o_t), x^o the rows of the layer that writes the pair's
 *         coefficients (the slot owner);
 *   y_t = U_l (x_t - c_t B);  s_t = fp16(max_{j<r_t} |y_tj| / 127);
 *   d_tj = clamp(round_half_even(y_tj / s_t), -127, 127) for j < r_t, else 0
 *         (s_t = 0 and no codes when r_t = 0 or the maximum is 0);
 *   B = the R leading right singular vectors of the pair's token rows
 *       stacked (uncentred), U_l = the Rmax leading right singular vectors of
 *       layer l's residual rows x_t - c_t B, per KV head, largest first, each
 *       row's largest-magnitude entry positive, rounded to bf16.
 * Products in the encoder run in fp32 (bf16 MFMA with the residual split into
 * a bf16 high part and remainder); the basis builder accumulates fp32 Gram
 * matrices and diagonalizes them with fp32 Jacobi rotations.                */

/* Workspace bytes kvs_encode_factorized needs for (batch, n). */
KVS_API kvs_status kvs_encode_workspace_size(const kvs_plan* plan, int32_t batch, int32_t n,
                                             size_t* bytes);

/* Encode n new tokens of `layer` from its K/V rows and append them
 * (coefficients when the layer owns its pair's slot, codes, scales, rank).
 *   k, v             device bf16 [batch][n][Hkv][hd]: the layer's rows
 *   k_owner, v_owner rows of the layer owning the pair's slot for the same
 *                    tokens (NULL when `layer` is that layer); the
 *                    coefficients are recomputed from them exactly as the
 *                    owner's call stored them
 *   rank             device uint8 [batch][n], as kvs_append_factorized
 *   start_pos        as kvs_append
 *   workspace        device, >= kvs_encode_workspace_size(batch, n) bytes
 * The bases are read from the cache (BK/BV of the pair's slot, UK/UV of the
 * layer).  Errors: non-factorized plan, or a non-owner layer without owner
 * rows -> KVS_ERR_ARG; head_dim not 64/128 or ranks not 32/16 ->
 * KVS_ERR_UNSUPPORTED; otherwise as kvs_append_factorized. */
KVS_API kvs_status kvs_encode_factorized(const kvs_plan* plan, const kvs_cache* cache,
                                         int32_t layer, const void* k, const void* v,
                                         const void* k_owner, const void* v_owner,
                                         const uint8_t* rank, int32_t n,
                                         const int32_t* start_pos, int32_t batch,
                                         void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes kvs_pair_basis / kvs_residual_basis need for (batch, n):
 * one basis item (K and V of one pair or layer). */
KVS_API kvs_status kvs_basis_workspace_size(const kvs_plan* plan, int32_t batch, int32_t n,
                                            size_t* bytes);

/* Pair basis (K and V) from the rows of the pair's two layers.
 *   k_a, v_a, k_b, v_b  device bf16 [batch][n][Hkv][hd]; k_b / v_b NULL for
 *                       a single layer
 *   n_tokens            device int32 [batch]: rows t < n_tokens[b] count
 *   basis_k, basis_v    device bf16 [Hkv][R][hd] out (e.g. the slot's BK/BV)
 * Fewer counted rows than R leave the trailing rows an arbitrary orthonormal
 * completion. */
KVS_API kvs_status kvs_pair_basis(const kvs_plan* plan, const void* k_a, const void* v_a,
                                  const void* k_b, const void* v_b, const int32_t* n_tokens,
                                  int32_t n, int32_t batch, void* basis_k, void* basis_v,
                                  void* workspace, size_t ws_bytes, void* stream);

/* kvs_pair_basis for n_items pairs at once: every argument named for one pair
 * becomes a host array of n_items device pointers (k_b / v_b: NULL, or an
 * array whose entries may be NULL).  All pairs share n, batch and n_tokens.
 * The matrices of as many items as the workspace holds
 * (ws_bytes / kvs_basis_workspace_size, at most 32) are diagonalized in one
 * launch, so a larger workspace lets more of the GPU work at once; results
 * equal those of one call per item. */
KVS_API kvs_status kvs_pair_bases(const kvs_plan* plan, int32_t n_items, const void* const* k_a,
                                  const void* const* v_a, const void* const* k_b,
                                  const void* const* v_b, const int32_t* n_tokens, int32_t n,
                                  int32_t batch, void* const* basis_k, void* const* basis_v,
                                  void* workspace, size_t ws_bytes, void* stream);

/* Residual directions (UK and UV) of a layer from its rows, the slot owner's
 * rows (NULL when the layer is the owner) and the pair basis (bf16
 * [Hkv][R][hd], as stored).  ubasis_k / ubasis_v: device bf16
 * [Hkv][Rmax][hd] out. */
KVS_API kvs_status kvs_residual_basis(const kvs_plan* plan, const void* k, const void* v,
                                      const void* k_owner, const void* v_owner,
                                      const void* basis_k, const void* basis_v,
                                      const int32_t* n_tokens, int32_t n, int32_t batch,
                                      void* ubasis_k, void* ubasis_v, void* workspace,
                                      size_t ws_bytes, void* stream);

/* kvs_residual_basis for n_items layers at once, in the manner of
 * kvs_pair_bases (k_owner / v_owner: NULL, or arrays whose entries may be
 * NULL for owner layers). */
KVS_API kvs_status kvs_residual_bases(const kvs_plan* plan, int32_t n_items, const void* const* k,
                                      const void* const* v, const void* const* k_owner,
                                      const void* const* v_owner, const void* const* basis_k,
                                      const void* const* basis_v, const int32_t* n_tokens,
                                      int32_t n, int32_t batch, void* const* ubasis_k,
                                      void* const* ubasis_v, void* workspace, size_t ws_bytes,
                                      void* stream);

/* ---------------------------------------------------------------- attention */

/* One decode query per (sequence, q head) of `layer` over keys
 * 0..seq_len[b]-1 of the layer's source(s) (the current token's entry
 * included: its owner appends it first).  The layer attends over the cached
 * K/V of its source layer ("Reducing Transformer Key-Value Cache Size with
 * Cross-Layer Attention", Methodology), of the stride-aligned source pair
 * mixed with the layer's weights ("DepthGraft: Structural Regularization
 * through Hierarchical Cross-Layer KV Reconstruction", Abstract), or of the
 * factorized entries read in place ("DepthWeave-KV: Smarter KV Cache
 * Compression by Sharing Across Layers and Adapting Per Token", Core
 * Mechanism: basis lookup, residual dequantization and attention in one
 * pass).  Keys of a page whose page-table entry lies outside
 * [0, n_phys_pages) get no weight (the entry is never dereferenced).
 *   q           device [batch][Hq][hd], cache dtype (bf16 for factorized)
 *   seq_len     device int32 [batch]; values are clamped to [0, max_ctx]; a
 *               sequence with no keys yields zeros
 *   max_seq_len host: the largest seq_len (used only to pick n_splits)
 *   n_splits    split-K partitions per (sequence, KV head); 0 = library choice
 *   out         device [batch][Hq][hd] of out_dtype (KVS_F32 or KVS_BF16)
 *   workspace   device, >= kvs_decode_workspace_size(batch, n_splits) bytes
 * Result is deterministic for fixed n_splits. */
KVS_API kvs_status kvs_attn_decode(const kvs_plan* plan, const kvs_cache* cache,
                                   int32_t layer, const void* q, const int32_t* seq_len,
                                   int32_t batch, int32_t max_seq_len, int32_t n_splits,
                                   void* out, int32_t out_dtype, void* workspace,
                                   size_t ws_bytes, void* stream);

/* kvs_attn_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels and results as kvs_attn_decode with the same
 * n_splits, with the split-K partials held in a 16 MiB device array that the
 * library keeps (one per GPU, alive until the process ends) instead of a
 * caller workspace.  The call allocates nothing itself; the first call on a
 * device looks the array's address up (hipGetSymbolAddress) with that device
 * current.
 *   n_splits  0: the library's choice, lowered until the partials fit; a
 *             given count whose partials (kvs_decode_workspace_size) exceed
 *             16 MiB -> KVS_ERR_RANGE, nothing launched
 * Every partition writes its whole partial row before the merge reads it, so
 * nothing in the array needs clearing between calls.  All calls on one GPU
 * share the array: calls that overlap in time on one GPU (other streams,
 * other threads) race and must be serialised by the caller.  Other arguments
 * and errors as kvs_attn_decode. */
KVS_API kvs_status kvs_attn_decode_noalloc(const kvs_plan* plan, const kvs_cache* cache,
                                           int32_t layer, const void* q, const int32_t* seq_len,
                                           int32_t batch, int32_t max_seq_len, int32_t n_splits,
                                           void* out, int32_t out_dtype, void* stream);

/* A chunk of n queries per sequence that sit at the last n positions of each
 * sequence (their K/V already appended): query i of sequence b is at
 * P = seq_len[b] - n + i and sees keys 0..P when causal != 0 (inclusive
 * diagonal), else keys 0..seq_len[b]-1.  The source layers' caches serve the
 * prompt's keys as they serve the decode ("Reducing Transformer Key-Value
 * Cache Size with Cross-Layer Attention", Methodology); only the owner
 * layers of a DepthGraft map need the whole prompt ("DepthGraft: Structural
 * Regularization through Hierarchical Cross-Layer KV Reconstruction",
 * Abstract: prefill completes early).  Keys of a page whose page-table entry
 * lies outside [0, n_phys_pages) get no weight, as in the decode.  Query and
 * key tiles go through bf16 MFMA with fp32 accumulation; a two-source
 * layer's mixed K~/V~ tiles (mixed in fp32) are rounded to fp16 and its
 * products run on fp16 operands (queries converted from bf16 exactly,
 * probabilities in fp16), which needs |q|, |K~|, |V~| below 65504.
 *   q        device bf16 [batch][n][Hq][hd]
 *   seq_len  device int32 [batch], each >= n; a row whose position P is
 *            below 0 (seq_len[b] < n) sees no key and yields zeros
 *   out      device [batch][n][Hq][hd] of out_dtype
 * Dense bf16 plans, and factorized plans (head_dim 64/128, ranks 32/16),
 * which attend in the coefficient space: q~ = B^K q and u~ = U^K q once per
 * query, scores c_t . q~ + s_t (d_t . u~), value accumulators in the 48
 * coefficients mapped back through B^V and U^V once per query row; the score
 * products take fp16 operands (q~, u~ and the scaled codes s_t d_t rounded
 * to fp16, the coefficients c_t converted exactly: their magnitudes must stay
 * below 65504), the value products bf16 (probabilities, c^V_t, and
 * s^V_t d^V_t rounded to bf16).  Other plans ->
 * KVS_ERR_UNSUPPORTED. */
KVS_API kvs_status kvs_attn_prefill_chunk(const kvs_plan* plan, const kvs_cache* cache,
                                          int32_t layer, const void* q, int32_t n,
                                          const int32_t* seq_len, int32_t batch,
                                          int32_t causal, void* out, int32_t out_dtype,
                                          void* stream);

/* --------------------------------------------------------- token router
 * The token router of "DepthWeave-KV: Smarter KV Cache Compression by Sharing
 * Across Layers and Adapting Per Token" (Core Mechanism, Key Concepts) reads
 * attention statistics, entropy and peak scores, and gives focused tokens a
 * higher residual rank, generic ones a lower one, online at every generation
 * step.  The page gives neither formulas nor thresholds; the readings here:
 * the statistics of a decode query are its attention entropy (nats) and its
 * peak probability; the rank of a sequence's current token follows from the
 * mean over statistic sets and query heads of entropy / ln(n) and from the
 * largest peak (kvs_router).  A routed rank is applied by encoding the
 * current token again at that rank (kvs_encode_factorized at its position):
 * it is the last token of its page, so no later token's codes move.       */

/* kvs_attn_decode on a factorized plan that also writes, per sequence and
 * query head, the attention statistics:
 *   stats  device float [batch][Hq][2]: entropy -sum p ln p (nats) and peak
 *          probability max p of the row's softmax over the keys it saw,
 *          computed from the same bf16-rounded probabilities as the output;
 *          (0, 0) for a query that sees no key.
 * The workspace is that of kvs_attn_decode.  Dense plans ->
 * KVS_ERR_UNSUPPORTED. */
KVS_API kvs_status kvs_attn_decode_stats(const kvs_plan* plan, const kvs_cache* cache,
                                         int32_t layer, const void* q, const int32_t* seq_len,
                                         int32_t batch, int32_t max_seq_len, int32_t n_splits,
                                         void* out, int32_t out_dtype, float* stats,
                                         void* workspace, size_t ws_bytes, void* stream);

typedef struct {
  float entropy_focused;   /* mean normalized entropy below this: rank_focused  */
  float entropy_diffuse;   /* at or above this: rank_diffuse; between: rank_mid  */
  float peak_focused;      /* a peak probability at or above this: rank_focused  */
  int32_t rank_focused;    /* ranks, clamped to [0, Rmax]                        */
  int32_t rank_mid;
  int32_t rank_diffuse;
} kvs_router;

/* Residual rank of each sequence's current token.
 *   stats    device float [n_sets][batch][Hq][2] from kvs_attn_decode_stats
 *            (one set per layer consulted)
 *   n_keys   device int32 [batch]: keys those queries saw (seq_len, less one
 *            for a layer with masks_current); h = 0 when n_keys <= 1
 *   rank_out device uint8 [batch]
 * h = mean over sets and heads of entropy / ln(n_keys) in fp32, p = the
 * largest peak; rank = rank_focused if h < entropy_focused or
 * p >= peak_focused, else rank_mid if h < entropy_diffuse, else
 * rank_diffuse.  Errors: non-factorized plan -> KVS_ERR_ARG. */
KVS_API kvs_status kvs_route_ranks(const kvs_plan* plan, const float* stats, int32_t n_sets,
                                   const int32_t* n_keys, int32_t batch,
                                   const kvs_router* router, uint8_t* rank_out, void* stream);

/* Kernel timing, for benchmarks and profilers (no passage of the pages: it
 * measures the calls above).  Arms the calling thread's next
 * kvs_attn_decode, kvs_attn_decode_stats or kvs_attn_prefill_chunk call so
 * that its main kernel (the split-K partition kernel, or the prefill kernel)
 * is launched with hipExtLaunchKernel and records start_event when it starts
 * executing and stop_event when it ends; hipEventElapsedTime of the pair is
 * that kernel's duration.  A merge launch that follows is outside the pair.
 *   start_event, stop_event  hipEvent_t handles the caller created (either
 *                            may be NULL; both NULL disarms); the caller
 *                            keeps ownership
 * The next such call consumes the arming whether it succeeds or not.
 * Always KVS_OK. */
KVS_API kvs_status kvs_time_next_launch(void* start_event, void* stop_event);

/* Description of the last error on this thread ("" if none). */
KVS_API const char* kvs_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* KVSHARE_H */
