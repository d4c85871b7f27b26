// C ABI glue: host-side argument validation (before any HIP call) and the
// dispatch to the gfx950 launchers.  Pure C++; the launchers live in the .hip
// files.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <string>

#include "internal.h"

using namespace kvs;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

kvs_status check_layer(const kvs_plan* plan, int32_t layer) {
  if (!plan) return fail(KVS_ERR_ARG, "null plan");
  if (layer < 0 || layer >= plan->p.cfg.n_layers) return fail(KVS_ERR_ARG, "layer out of range");
  return KVS_OK;
}

kvs_status check_batch(const kvs_plan* plan, int32_t batch) {
  if (batch < 1 || batch > plan->p.cfg.max_batch) return fail(KVS_ERR_RANGE, "batch out of range");
  return KVS_OK;
}

// events armed by kvs_time_next_launch for this thread's next attention call
thread_local KernelEvents g_next_events;

kvs_status hip_status(int err, const char* what) {
  if (err == 0) return KVS_OK;
  return fail(KVS_ERR_HIP, std::string(what) + ": " + hip_error_name(err));
}

float scale_log2(int32_t hd) { return (float)(1.4426950408889634 / std::sqrt((double)hd)); }

}  // namespace

extern "C" kvs_status kvs_append(const kvs_plan* plan, const kvs_cache* cache, int32_t layer,
                                 const void* k, const void* v, int32_t n,
                                 const int32_t* start_pos, int32_t batch, void* stream) {
  clear_error();
  kvs_status st = check_layer(plan, layer);
  if (st != KVS_OK) return st;
  const Plan& p = plan->p;
  if (p.cfg.kind != KVS_DENSE) return fail(KVS_ERR_ARG, "kvs_append needs a dense plan");
  if (!cache || !k || !v || !start_pos || !cache->k_pool || !cache->v_pool || !cache->page_table)
    return fail(KVS_ERR_ARG, "null argument");
  if ((st = check_batch(plan, batch)) != KVS_OK) return st;
  if (n < 0 || n > p.cfg.max_ctx) return fail(KVS_ERR_RANGE, "n out of range");
  if (!p.layers[layer].owns_kv)
    return fail(KVS_ERR_NOT_SOURCE, "layer " + std::to_string(layer) + " owns no cache entries");
  if (!aligned16(k) || !aligned16(v) || !aligned16(cache->k_pool) || !aligned16(cache->v_pool))
    return fail(KVS_ERR_ALIGN, "k, v and the pools must be 16-byte aligned");
  if (!aligned4(start_pos) || !aligned4(cache->page_table)) return fail(KVS_ERR_ALIGN, "misaligned int32 array");
  if (n == 0) return KVS_OK;
  AppendLaunch a;
  a.k_pool = cache->k_pool;
  a.v_pool = cache->v_pool;
  a.page_table = cache->page_table;
  a.pages_per_seq = p.pages_per_seq;
  a.n_phys_pages = p.n_phys_pages;
  a.n_kv_heads = p.cfg.n_kv_heads;
  a.head_dim = p.cfg.head_dim;
  a.dtype = p.cfg.dtype;
  a.slot_offset = (int64_t)p.layers[layer].src_slot[0] * p.n_phys_pages * p.cfg.n_kv_heads * kPage *
                  p.cfg.head_dim;
  a.k = k;
  a.v = v;
  a.n = n;
  a.start_pos = start_pos;
  a.batch = batch;
  a.max_ctx = p.cfg.max_ctx;
  return hip_status(launch_append(a, stream), "append launch");
}

namespace {

kvs_status decode_impl(const kvs_plan* plan, const kvs_cache* cache, int32_t layer, const void* q,
                       const int32_t* seq_len, int32_t batch, int32_t max_seq_len, int32_t n_splits,
                       void* out, int32_t out_dtype, float* stats, void* workspace, size_t ws_bytes,
                       void* stream) {
  const KernelEvents ev = take_kernel_events();
  kvs_status st = check_layer(plan, layer);
  if (st != KVS_OK) return st;
  const Plan& p = plan->p;
  if (!cache || !q || !seq_len || !out || !workspace) return fail(KVS_ERR_ARG, "null argument");
  if ((st = check_batch(plan, batch)) != KVS_OK) return st;
  if (out_dtype != KVS_F32 && out_dtype != KVS_BF16) return fail(KVS_ERR_ARG, "bad out_dtype");
  if (n_splits == 0) {
    if ((st = kvs_decode_splits(plan, batch, max_seq_len, &n_splits)) != KVS_OK) return st;
  }
  size_t need = 0;
  if ((st = kvs_decode_workspace_size(plan, batch, n_splits, &need)) != KVS_OK) return st;
  if (ws_bytes < need) return fail(KVS_ERR_RANGE, "workspace too small: need " + std::to_string(need));
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace) || !aligned4(seq_len))
    return fail(KVS_ERR_ALIGN, "q, out and workspace must be 16-byte aligned");
  const kvs_layer_info& li = p.layers[layer];
  const int32_t group = p.cfg.n_q_heads / p.cfg.n_kv_heads;
  if (p.cfg.kind == KVS_FACTORIZED) {
    if (!cache->ck_pool || !cache->cv_pool || !cache->dk_pool || !cache->dv_pool || !cache->sk_pool ||
        !cache->sv_pool || !cache->rank_pool || !cache->page_table || !cache->basis_k ||
        !cache->basis_v || !cache->ubasis_k || !cache->ubasis_v)
      return fail(KVS_ERR_ARG, "null factorized cache buffer");
    if (!aligned16(cache->ck_pool) || !aligned16(cache->cv_pool) || !aligned16(cache->dk_pool) ||
        !aligned16(cache->dv_pool) || !aligned16(cache->basis_k) || !aligned16(cache->basis_v) ||
        !aligned16(cache->ubasis_k) || !aligned16(cache->ubasis_v) || !aligned16(cache->sk_pool) ||
        !aligned16(cache->sv_pool) || !aligned16(cache->rank_pool) || !aligned4(cache->page_table))
      return fail(KVS_ERR_ALIGN, "factorized buffers must be 16-byte aligned");
    FactDecodeLaunch f;
    f.ev = ev;
    f.ck_pool = cache->ck_pool;
    f.cv_pool = cache->cv_pool;
    f.dk_pool = cache->dk_pool;
    f.dv_pool = cache->dv_pool;
    f.sk_pool = cache->sk_pool;
    f.sv_pool = cache->sv_pool;
    f.rank_pool = cache->rank_pool;
    f.basis_k = cache->basis_k;
    f.basis_v = cache->basis_v;
    f.ubasis_k = cache->ubasis_k;
    f.ubasis_v = cache->ubasis_v;
    f.page_table = cache->page_table;
    f.pages_per_seq = p.pages_per_seq;
    f.n_phys_pages = p.n_phys_pages;
    f.n_kv_heads = p.cfg.n_kv_heads;
    f.n_q_heads = p.cfg.n_q_heads;
    f.head_dim = p.cfg.head_dim;
    f.basis_rank = p.cfg.basis_rank;
    f.resid_rank_max = p.cfg.resid_rank_max;
    f.coef_slot = li.src_slot[0];
    f.layer = layer;
    f.q = q;
    f.seq_len = seq_len;
    f.max_ctx = p.cfg.max_ctx;
    f.key_excl = li.masks_current;
    f.batch = batch;
    f.n_splits = n_splits;
    f.scale_log2 = scale_log2(p.cfg.head_dim);
    f.ws = static_cast<float*>(workspace);
    f.out = out;
    f.out_dtype = out_dtype;
    f.stats = stats;
    return hip_status(launch_fact_decode(f, stream), "factorized decode launch");
  }
  if (stats) return fail(KVS_ERR_UNSUPPORTED, "router statistics are produced for factorized plans");
  if (!cache->k_pool || !cache->v_pool || !cache->page_table) return fail(KVS_ERR_ARG, "null cache pool");
  if (!aligned16(cache->k_pool) || !aligned16(cache->v_pool) || !aligned4(cache->page_table))
    return fail(KVS_ERR_ALIGN, "pools must be 16-byte aligned");
  DecodeLaunch a;
  a.ev = ev;
  a.k_pool = cache->k_pool;
  a.v_pool = cache->v_pool;
  a.page_table = cache->page_table;
  a.pages_per_seq = p.pages_per_seq;
  a.n_phys_pages = p.n_phys_pages;
  a.n_kv_heads = p.cfg.n_kv_heads;
  a.n_q_heads = p.cfg.n_q_heads;
  a.head_dim = p.cfg.head_dim;
  a.group = group;
  a.dtype = p.cfg.dtype;
  a.slot_stride = (int64_t)p.n_phys_pages * p.cfg.n_kv_heads * kPage * p.cfg.head_dim;
  a.n_src = li.n_src;
  a.slot[0] = li.src_slot[0];
  a.slot[1] = li.src_slot[1];
  a.weight[0] = li.weight[0];
  a.weight[1] = li.weight[1];
  a.q = q;
  a.seq_len = seq_len;
  a.max_ctx = p.cfg.max_ctx;
  a.key_excl = li.masks_current;
  a.batch = batch;
  a.n_splits = n_splits;
  a.scale_log2 = scale_log2(p.cfg.head_dim);
  a.ws = static_cast<float*>(workspace);
  a.out = out;
  a.out_dtype = out_dtype;
  return hip_status(launch_decode(a, stream), "decode launch");
}

}  // namespace

extern "C" kvs_status kvs_attn_decode(const kvs_plan* plan, const kvs_cache* cache, int32_t layer,
                                      const void* q, const int32_t* seq_len, int32_t batch,
                                      int32_t max_seq_len, int32_t n_splits, void* out,
                                      int32_t out_dtype, void* workspace, size_t ws_bytes,
                                      void* stream) {
  clear_error();
  return decode_impl(plan, cache, layer, q, seq_len, batch, max_seq_len, n_splits, out, out_dtype,
                     nullptr, workspace, ws_bytes, stream);
}

extern "C" kvs_status kvs_attn_decode_noalloc(const kvs_plan* plan, const kvs_cache* cache,
                                              int32_t layer, const void* q, const int32_t* seq_len,
                                              int32_t batch, int32_t max_seq_len, int32_t n_splits,
                                              void* out, int32_t out_dtype, void* stream) {
  clear_error();
  kvs_status st = check_layer(plan, layer);
  if (st != KVS_OK) return st;
  if ((st = check_batch(plan, batch)) != KVS_OK) return st;
  const size_t cap = scratch_bytes();
  size_t need = 0;
  if (n_splits == 0) {
    // the library's choice, lowered until the partials fit the scratch
    if ((st = kvs_decode_splits(plan, batch, max_seq_len, &n_splits)) != KVS_OK) return st;
    if ((st = kvs_decode_workspace_size(plan, batch, 1, &need)) != KVS_OK) return st;
    const size_t fit = need ? cap / need : size_t(n_splits);
    if (fit >= 1 && size_t(n_splits) > fit) n_splits = int32_t(fit);
  }
  if ((st = kvs_decode_workspace_size(plan, batch, n_splits, &need)) != KVS_OK) return st;
  if (need > cap)
    return fail(KVS_ERR_RANGE, "kvs_attn_decode_noalloc: batch " + std::to_string(batch) + " x " +
                                   std::to_string(n_splits) + " partitions need " +
                                   std::to_string(need) + " bytes of partials; the library's "
                                   "scratch holds " + std::to_string(cap) +
                                   " (use fewer partitions or kvs_attn_decode with a workspace)");
  void* ptr = nullptr;
  if ((st = hip_status(scratch_address(&ptr), "scratch address")) != KVS_OK) return st;
  return decode_impl(plan, cache, layer, q, seq_len, batch, max_seq_len, n_splits, out, out_dtype,
                     nullptr, ptr, cap, stream);
}

extern "C" kvs_status kvs_attn_decode_stats(const kvs_plan* plan, const kvs_cache* cache,
                                            int32_t layer, const void* q, const int32_t* seq_len,
                                            int32_t batch, int32_t max_seq_len, int32_t n_splits,
                                            void* out, int32_t out_dtype, float* stats,
                                            void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  if (!stats) return fail(KVS_ERR_ARG, "null stats");
  if (!aligned4(stats)) return fail(KVS_ERR_ALIGN, "stats must be 4-byte aligned");
  return decode_impl(plan, cache, layer, q, seq_len, batch, max_seq_len, n_splits, out, out_dtype,
                     stats, workspace, ws_bytes, stream);
}

extern "C" kvs_status kvs_route_ranks(const kvs_plan* plan, const float* stats, int32_t n_sets,
                                      const int32_t* n_keys, int32_t batch,
                                      const kvs_router* router, uint8_t* rank_out, void* stream) {
  clear_error();
  if (!plan || !stats || !n_keys || !router || !rank_out) return fail(KVS_ERR_ARG, "null argument");
  const Plan& p = plan->p;
  if (p.cfg.kind != KVS_FACTORIZED) return fail(KVS_ERR_ARG, "ranks route a factorized plan");
  kvs_status st = check_batch(plan, batch);
  if (st != KVS_OK) return st;
  if (n_sets < 1) return fail(KVS_ERR_RANGE, "n_sets must be >= 1");
  if (!std::isfinite(router->entropy_focused) || !std::isfinite(router->entropy_diffuse) ||
      std::isnan(router->peak_focused))
    return fail(KVS_ERR_ARG, "router thresholds must be numbers");
  if (!aligned4(stats) || !aligned4(n_keys)) return fail(KVS_ERR_ALIGN, "stats and n_keys must be 4-byte aligned");
  RouteLaunch r;
  r.stats = stats;
  r.n_sets = n_sets;
  r.n_keys = n_keys;
  r.batch = batch;
  r.n_q_heads = p.cfg.n_q_heads;
  r.entropy_focused = router->entropy_focused;
  r.entropy_diffuse = router->entropy_diffuse;
  r.peak_focused = router->peak_focused;
  const int32_t rmax = p.cfg.resid_rank_max;
  r.rank_focused = std::min(std::max(router->rank_focused, 0), rmax);
  r.rank_mid = std::min(std::max(router->rank_mid, 0), rmax);
  r.rank_diffuse = std::min(std::max(router->rank_diffuse, 0), rmax);
  r.rank_out = rank_out;
  return hip_status(launch_route(r, stream), "route launch");
}

extern "C" kvs_status kvs_attn_prefill_chunk(const kvs_plan* plan, const kvs_cache* cache,
                                             int32_t layer, const void* q, int32_t n,
                                             const int32_t* seq_len, int32_t batch, int32_t causal,
                                             void* out, int32_t out_dtype, void* stream) {
  clear_error();
  const KernelEvents ev = take_kernel_events();
  kvs_status st = check_layer(plan, layer);
  if (st != KVS_OK) return st;
  const Plan& p = plan->p;
  if (!cache || !q || !seq_len || !out) return fail(KVS_ERR_ARG, "null argument");
  if ((st = check_batch(plan, batch)) != KVS_OK) return st;
  if (n < 1 || n > p.cfg.max_ctx) return fail(KVS_ERR_RANGE, "n out of range");
  if (out_dtype != KVS_F32 && out_dtype != KVS_BF16) return fail(KVS_ERR_ARG, "bad out_dtype");
  const int32_t group = p.cfg.n_q_heads / p.cfg.n_kv_heads;
  const kvs_layer_info& li = p.layers[layer];
  if (p.cfg.kind == KVS_FACTORIZED) {
    if (!fact_prefill_shape_supported(p.cfg.head_dim, group, p.cfg.basis_rank, p.cfg.resid_rank_max))
      return fail(KVS_ERR_UNSUPPORTED, "no factorized prefill kernel for this shape");
    if (!cache->ck_pool || !cache->cv_pool || !cache->dk_pool || !cache->dv_pool || !cache->sk_pool ||
        !cache->sv_pool || !cache->rank_pool || !cache->page_table || !cache->basis_k ||
        !cache->basis_v || !cache->ubasis_k || !cache->ubasis_v)
      return fail(KVS_ERR_ARG, "null factorized cache buffer");
    if (!aligned16(q) || !aligned16(out) || !aligned4(seq_len) || !aligned16(cache->ck_pool) ||
        !aligned16(cache->cv_pool) || !aligned16(cache->dk_pool) || !aligned16(cache->dv_pool) ||
        !aligned16(cache->basis_k) || !aligned16(cache->basis_v) || !aligned16(cache->ubasis_k) ||
        !aligned16(cache->ubasis_v) || !aligned16(cache->sk_pool) || !aligned16(cache->sv_pool) ||
        !aligned16(cache->rank_pool) || !aligned4(cache->page_table))
      return fail(KVS_ERR_ALIGN, "q, out and the factorized buffers must be 16-byte aligned");
    FactPrefillLaunch f;
    f.ev = ev;
    f.ck_pool = cache->ck_pool;
    f.cv_pool = cache->cv_pool;
    f.dk_pool = cache->dk_pool;
    f.dv_pool = cache->dv_pool;
    f.sk_pool = cache->sk_pool;
    f.sv_pool = cache->sv_pool;
    f.rank_pool = cache->rank_pool;
    f.basis_k = cache->basis_k;
    f.basis_v = cache->basis_v;
    f.ubasis_k = cache->ubasis_k;
    f.ubasis_v = cache->ubasis_v;
    f.page_table = cache->page_table;
    f.pages_per_seq = p.pages_per_seq;
    f.n_phys_pages = p.n_phys_pages;
    f.n_kv_heads = p.cfg.n_kv_heads;
    f.n_q_heads = p.cfg.n_q_heads;
    f.head_dim = p.cfg.head_dim;
    f.coef_slot = li.src_slot[0];
    f.layer = layer;
    f.q = q;
    f.n = n;
    f.seq_len = seq_len;
    f.max_ctx = p.cfg.max_ctx;
    f.key_excl = li.masks_current;
    f.batch = batch;
    f.causal = causal != 0;
    f.scale_log2 = scale_log2(p.cfg.head_dim);
    f.out = out;
    f.out_dtype = out_dtype;
    return hip_status(launch_fact_prefill(f, stream), "factorized prefill launch");
  }
  if (p.cfg.dtype != KVS_BF16)
    return fail(KVS_ERR_UNSUPPORTED, "prefill runs on bf16 caches (bf16 MFMA)");
  if (!prefill_shape_supported(p.cfg.head_dim, group, li.n_src))
    return fail(KVS_ERR_UNSUPPORTED, "no prefill kernel for this head_dim/group size/source count");
  if (!cache->k_pool || !cache->v_pool || !cache->page_table) return fail(KVS_ERR_ARG, "null cache pool");
  if (!aligned16(q) || !aligned16(out) || !aligned16(cache->k_pool) || !aligned16(cache->v_pool) ||
      !aligned4(seq_len) || !aligned4(cache->page_table))
    return fail(KVS_ERR_ALIGN, "q, out and the pools must be 16-byte aligned");
  PrefillLaunch a;
  a.ev = ev;
  a.k_pool = cache->k_pool;
  a.v_pool = cache->v_pool;
  a.page_table = cache->page_table;
  a.pages_per_seq = p.pages_per_seq;
  a.n_phys_pages = p.n_phys_pages;
  a.n_kv_heads = p.cfg.n_kv_heads;
  a.n_q_heads = p.cfg.n_q_heads;
  a.head_dim = p.cfg.head_dim;
  a.slot_stride = (int64_t)p.n_phys_pages * p.cfg.n_kv_heads * kPage * p.cfg.head_dim;
  a.n_src = li.n_src;
  a.slot[0] = li.src_slot[0];
  a.slot[1] = li.src_slot[1];
  a.weight[0] = li.weight[0];
  a.weight[1] = li.weight[1];
  a.q = q;
  a.n = n;
  a.seq_len = seq_len;
  a.max_ctx = p.cfg.max_ctx;
  a.key_excl = li.masks_current;
  a.batch = batch;
  a.causal = causal != 0;
  a.scale_log2 = scale_log2(p.cfg.head_dim);
  a.out = out;
  a.out_dtype = out_dtype;
  return hip_status(launch_prefill(a, stream), "prefill launch");
}

extern "C" kvs_status kvs_append_factorized(const kvs_plan* plan, const kvs_cache* cache,
                                            int32_t layer, const void* ck, const void* cv,
                                            const int8_t* dk, const int8_t* dv, const void* sk,
                                            const void* sv, const uint8_t* rank, int32_t n,
                                            const int32_t* start_pos, int32_t batch, void* stream) {
  clear_error();
  kvs_status st = check_layer(plan, layer);
  if (st != KVS_OK) return st;
  const Plan& p = plan->p;
  if (p.cfg.kind != KVS_FACTORIZED) return fail(KVS_ERR_ARG, "kvs_append_factorized needs a factorized plan");
  if (!cache || !dk || !dv || !sk || !sv || !rank || !start_pos) return fail(KVS_ERR_ARG, "null argument");
  if (!cache->ck_pool || !cache->cv_pool || !cache->dk_pool || !cache->dv_pool || !cache->sk_pool ||
      !cache->sv_pool || !cache->rank_pool || !cache->page_table)
    return fail(KVS_ERR_ARG, "null cache pool");
  if ((st = check_batch(plan, batch)) != KVS_OK) return st;
  if (n < 0 || n > p.cfg.max_ctx) return fail(KVS_ERR_RANGE, "n out of range");
  const kvs_layer_info& li = p.layers[layer];
  if ((ck == nullptr) != (cv == nullptr)) return fail(KVS_ERR_ARG, "give both ck and cv, or neither");
  if (ck && !li.owns_kv)
    return fail(KVS_ERR_NOT_SOURCE, "layer " + std::to_string(layer) + " does not own its pair's coefficients");
  if ((ck && (!aligned16(ck) || !aligned16(cv))) || !aligned16(dk) || !aligned16(dv) ||
      !aligned16(cache->ck_pool) || !aligned16(cache->cv_pool) || !aligned16(cache->dk_pool) ||
      !aligned16(cache->dv_pool))
    return fail(KVS_ERR_ALIGN, "coefficients, codes and pools must be 16-byte aligned");
  if (!aligned4(start_pos) || !aligned4(cache->page_table) || ((uintptr_t)sk & 1) || ((uintptr_t)sv & 1) ||
      ((uintptr_t)cache->rank_pool & 1))
    return fail(KVS_ERR_ALIGN, "misaligned scale or int32 array");
  if (n == 0) return KVS_OK;
  FactAppendLaunch a;
  a.ck_pool = cache->ck_pool;
  a.cv_pool = cache->cv_pool;
  a.dk_pool = cache->dk_pool;
  a.dv_pool = cache->dv_pool;
  a.sk_pool = cache->sk_pool;
  a.sv_pool = cache->sv_pool;
  a.rank_pool = cache->rank_pool;
  a.page_table = cache->page_table;
  a.pages_per_seq = p.pages_per_seq;
  a.n_phys_pages = p.n_phys_pages;
  a.n_kv_heads = p.cfg.n_kv_heads;
  a.basis_rank = p.cfg.basis_rank;
  a.resid_rank_max = p.cfg.resid_rank_max;
  a.coef_slot = ck ? li.src_slot[0] : -1;
  a.layer = layer;
  a.ck = ck;
  a.cv = cv;
  a.dk = dk;
  a.dv = dv;
  a.sk = sk;
  a.sv = sv;
  a.rank = rank;
  a.n = n;
  a.start_pos = start_pos;
  a.batch = batch;
  a.max_ctx = p.cfg.max_ctx;
  return hip_status(launch_fact_append(a, stream), "factorized append launch");
}

// ------------------------------------------------------------- write side

namespace {

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Encoder workspace: per side (K, V) the coefficients [B][n][Hkv][R] bf16,
// codes [B][n][Hkv][Rmax] int8 and scales [B][n][Hkv] fp16.
struct EncodeWs {
  size_t c, d, s, total;
};
EncodeWs encode_ws(const Plan& p, int32_t batch, int32_t n) {
  const size_t rows = (size_t)batch * n * p.cfg.n_kv_heads;
  EncodeWs w;
  w.c = round256(rows * p.cfg.basis_rank * 2);
  w.d = round256(rows * p.cfg.resid_rank_max);
  w.s = round256(rows * 2);
  w.total = 2 * (w.c + w.d + w.s);
  return w;
}

// Basis workspace of one item (K and V of one pair or layer): Gram matrices
// [2][Hkv][hd][hd] and eigenvalues [2][Hkv][hd] (fp32), and for residual
// directions the residual rows [2][B][n][Hkv][hd] (fp32).  A batched call
// lays out the Gram matrices of all its items, then their eigenvalues, then
// their rows.
struct BasisWs {
  size_t gram, evals, rows, item;
};
BasisWs basis_ws(const Plan& p, int32_t batch, int32_t n) {
  const size_t hd = p.cfg.head_dim, H = p.cfg.n_kv_heads;
  BasisWs w;
  w.gram = round256(2 * H * hd * hd * 4);
  w.evals = round256(2 * H * hd * 4);
  w.rows = round256((size_t)batch * n * H * hd * 4);
  w.item = w.gram + w.evals + 2 * w.rows;
  return w;
}

kvs_status check_write_side(const kvs_plan* plan, int32_t batch, int32_t n) {
  if (!plan) return fail(KVS_ERR_ARG, "null plan");
  const Plan& p = plan->p;
  if (p.cfg.kind != KVS_FACTORIZED) return fail(KVS_ERR_ARG, "needs a factorized plan");
  if (!encode_shape_supported(p.cfg.head_dim, p.cfg.basis_rank, p.cfg.resid_rank_max))
    return fail(KVS_ERR_UNSUPPORTED, "no write-side kernels for this head_dim / rank");
  kvs_status st = check_batch(plan, batch);
  if (st != KVS_OK) return st;
  if (n < 1 || n > p.cfg.max_ctx) return fail(KVS_ERR_RANGE, "n out of range");
  return KVS_OK;
}

}  // namespace

extern "C" kvs_status kvs_encode_workspace_size(const kvs_plan* plan, int32_t batch, int32_t n,
                                                size_t* bytes) {
  clear_error();
  kvs_status st = check_write_side(plan, batch, n);
  if (st != KVS_OK) return st;
  if (!bytes) return fail(KVS_ERR_ARG, "null argument");
  *bytes = encode_ws(plan->p, batch, n).total;
  return KVS_OK;
}

extern "C" kvs_status kvs_encode_factorized(const kvs_plan* plan, const kvs_cache* cache,
                                            int32_t layer, const void* k, const void* v,
                                            const void* k_owner, const void* v_owner,
                                            const uint8_t* rank, int32_t n,
                                            const int32_t* start_pos, int32_t batch,
                                            void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  kvs_status st = check_layer(plan, layer);
  if (st != KVS_OK) return st;
  if ((st = check_write_side(plan, batch, n)) != KVS_OK) return st;
  const Plan& p = plan->p;
  const kvs_layer_info& li = p.layers[layer];
  if (!cache || !k || !v || !rank || !start_pos || !workspace) return fail(KVS_ERR_ARG, "null argument");
  if ((k_owner == nullptr) != (v_owner == nullptr)) return fail(KVS_ERR_ARG, "give both k_owner and v_owner, or neither");
  if (!li.owns_kv && !k_owner)
    return fail(KVS_ERR_ARG, "layer " + std::to_string(layer) +
                                 " does not write its pair's coefficients: pass the writing layer's rows");
  if (!cache->basis_k || !cache->basis_v || !cache->ubasis_k || !cache->ubasis_v || !cache->ck_pool ||
      !cache->cv_pool || !cache->dk_pool || !cache->dv_pool || !cache->sk_pool || !cache->sv_pool ||
      !cache->rank_pool || !cache->page_table)
    return fail(KVS_ERR_ARG, "null factorized cache buffer");
  if (!aligned16(k) || !aligned16(v) || (k_owner && (!aligned16(k_owner) || !aligned16(v_owner))) ||
      !aligned16(workspace) || !aligned16(cache->basis_k) || !aligned16(cache->basis_v) ||
      !aligned16(cache->ubasis_k) || !aligned16(cache->ubasis_v) || !aligned16(cache->ck_pool) ||
      !aligned16(cache->cv_pool) || !aligned16(cache->dk_pool) || !aligned16(cache->dv_pool) ||
      !aligned4(start_pos) || !aligned4(cache->page_table) || ((uintptr_t)cache->sk_pool & 1) ||
      ((uintptr_t)cache->sv_pool & 1) || ((uintptr_t)cache->rank_pool & 1))
    return fail(KVS_ERR_ALIGN, "rows, workspace, bases and pools must be 16-byte aligned");
  const EncodeWs w = encode_ws(p, batch, n);
  if (ws_bytes < w.total) return fail(KVS_ERR_RANGE, "workspace too small: need " + std::to_string(w.total));
  const size_t hd = p.cfg.head_dim, H = p.cfg.n_kv_heads;
  const int32_t slot = li.src_slot[0];
  char* ws = static_cast<char*>(workspace);
  EncodeLaunch e;
  const void* x[2] = {k, v};
  const void* xo[2] = {k_owner ? k_owner : k, v_owner ? v_owner : v};
  const void* bases[2] = {cache->basis_k, cache->basis_v};
  const void* ubases[2] = {cache->ubasis_k, cache->ubasis_v};
  for (int side = 0; side < 2; ++side) {
    char* base = ws + side * (w.c + w.d + w.s);
    e.x[side] = x[side];
    e.xo[side] = xo[side];
    e.basis[side] = static_cast<const uint16_t*>(bases[side]) + (size_t)slot * H * p.cfg.basis_rank * hd;
    e.ubasis[side] = static_cast<const uint16_t*>(ubases[side]) + (size_t)layer * H * p.cfg.resid_rank_max * hd;
    e.c_out[side] = li.owns_kv ? base : nullptr;
    e.d_out[side] = base + w.c;
    e.s_out[side] = base + w.c + w.d;
    e.e_out[side] = nullptr;
  }
  e.rank = rank;
  e.n_tokens = nullptr;
  e.n = n;
  e.batch = batch;
  e.n_kv_heads = p.cfg.n_kv_heads;
  e.head_dim = p.cfg.head_dim;
  e.residual_mode = 0;
  if ((st = hip_status(launch_encode(e, stream), "encode launch")) != KVS_OK) return st;
  return kvs_append_factorized(plan, cache, layer, e.c_out[0], e.c_out[1],
                               static_cast<const int8_t*>(e.d_out[0]),
                               static_cast<const int8_t*>(e.d_out[1]), e.s_out[0], e.s_out[1], rank,
                               n, start_pos, batch, stream);
}

extern "C" kvs_status kvs_basis_workspace_size(const kvs_plan* plan, int32_t batch, int32_t n,
                                               size_t* bytes) {
  clear_error();
  kvs_status st = check_write_side(plan, batch, n);
  if (st != KVS_OK) return st;
  if (!bytes) return fail(KVS_ERR_ARG, "null argument");
  *bytes = basis_ws(plan->p, batch, n).item;
  return KVS_OK;
}

namespace {

// items processed per launch group: as many as the workspace holds, at most
// kMaxBasisSets / 2
kvs_status basis_group(const kvs_plan* plan, int32_t n_items, const int32_t* n_tokens, int32_t n,
                       int32_t batch, void* workspace, size_t ws_bytes, int32_t* group) {
  kvs_status st = check_write_side(plan, batch, n);
  if (st != KVS_OK) return st;
  if (n_items < 1) return fail(KVS_ERR_ARG, "n_items must be >= 1");
  if (!n_tokens || !workspace) return fail(KVS_ERR_ARG, "null argument");
  if (!aligned4(n_tokens) || !aligned16(workspace)) return fail(KVS_ERR_ALIGN, "n_tokens / workspace misaligned");
  const BasisWs w = basis_ws(plan->p, batch, n);
  if (ws_bytes < w.item) return fail(KVS_ERR_RANGE, "workspace too small: need at least " + std::to_string(w.item));
  *group = (int32_t)std::min<size_t>(ws_bytes / w.item, kMaxBasisSets / 2);
  return KVS_OK;
}

BasisLaunch basis_launch(const Plan& p, const int32_t* n_tokens, int32_t n, int32_t batch, int32_t k_out,
                         int32_t items, void* workspace) {
  const BasisWs w = basis_ws(p, batch, n);
  char* ws = static_cast<char*>(workspace);
  BasisLaunch b;
  b.n_sets = 2 * items;
  b.n_tokens = n_tokens;
  b.n = n;
  b.batch = batch;
  b.n_kv_heads = p.cfg.n_kv_heads;
  b.head_dim = p.cfg.head_dim;
  b.k_out = k_out;
  b.gram = reinterpret_cast<float*>(ws);
  b.evals = reinterpret_cast<float*>(ws + items * w.gram);
  return b;
}

}  // namespace

extern "C" kvs_status kvs_pair_bases(const kvs_plan* plan, int32_t n_items, const void* const* k_a,
                                     const void* const* v_a, const void* const* k_b,
                                     const void* const* v_b, const int32_t* n_tokens, int32_t n,
                                     int32_t batch, void* const* basis_k, void* const* basis_v,
                                     void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  int32_t group = 0;
  kvs_status st = basis_group(plan, n_items, n_tokens, n, batch, workspace, ws_bytes, &group);
  if (st != KVS_OK) return st;
  if (!k_a || !v_a || !basis_k || !basis_v) return fail(KVS_ERR_ARG, "null array");
  for (int32_t i = 0; i < n_items; ++i) {
    const void* kb = k_b ? k_b[i] : nullptr;
    const void* vb = v_b ? v_b[i] : nullptr;
    if (!k_a[i] || !v_a[i] || !basis_k[i] || !basis_v[i]) return fail(KVS_ERR_ARG, "null argument");
    if ((kb == nullptr) != (vb == nullptr)) return fail(KVS_ERR_ARG, "give both k_b and v_b, or neither");
    if (!aligned16(k_a[i]) || !aligned16(v_a[i]) || (kb && (!aligned16(kb) || !aligned16(vb))) ||
        !aligned16(basis_k[i]) || !aligned16(basis_v[i]))
      return fail(KVS_ERR_ALIGN, "rows and outputs must be 16-byte aligned");
  }
  for (int32_t i0 = 0; i0 < n_items; i0 += group) {
    const int32_t cnt = std::min(group, n_items - i0);
    BasisLaunch b = basis_launch(plan->p, n_tokens, n, batch, plan->p.cfg.basis_rank, cnt, workspace);
    for (int32_t j = 0; j < cnt; ++j) {
      const int32_t i = i0 + j;
      b.x[2 * j][0] = k_a[i];
      b.x[2 * j][1] = k_b ? k_b[i] : nullptr;
      b.x[2 * j + 1][0] = v_a[i];
      b.x[2 * j + 1][1] = v_b ? v_b[i] : nullptr;
      b.out[2 * j] = basis_k[i];
      b.out[2 * j + 1] = basis_v[i];
    }
    b.rows_f32 = 0;
    if ((st = hip_status(launch_basis(b, stream), "pair basis launch")) != KVS_OK) return st;
  }
  return KVS_OK;
}

extern "C" kvs_status kvs_pair_basis(const kvs_plan* plan, const void* k_a, const void* v_a,
                                     const void* k_b, const void* v_b, const int32_t* n_tokens,
                                     int32_t n, int32_t batch, void* basis_k, void* basis_v,
                                     void* workspace, size_t ws_bytes, void* stream) {
  return kvs_pair_bases(plan, 1, &k_a, &v_a, &k_b, &v_b, n_tokens, n, batch, &basis_k, &basis_v,
                        workspace, ws_bytes, stream);
}

extern "C" kvs_status kvs_residual_bases(const kvs_plan* plan, int32_t n_items, const void* const* k,
                                         const void* const* v, const void* const* k_owner,
                                         const void* const* v_owner, const void* const* basis_k,
                                         const void* const* basis_v, const int32_t* n_tokens,
                                         int32_t n, int32_t batch, void* const* ubasis_k,
                                         void* const* ubasis_v, void* workspace, size_t ws_bytes,
                                         void* stream) {
  clear_error();
  int32_t group = 0;
  kvs_status st = basis_group(plan, n_items, n_tokens, n, batch, workspace, ws_bytes, &group);
  if (st != KVS_OK) return st;
  if (!k || !v || !basis_k || !basis_v || !ubasis_k || !ubasis_v) return fail(KVS_ERR_ARG, "null array");
  for (int32_t i = 0; i < n_items; ++i) {
    const void* ko = k_owner ? k_owner[i] : nullptr;
    const void* vo = v_owner ? v_owner[i] : nullptr;
    if (!k[i] || !v[i] || !basis_k[i] || !basis_v[i] || !ubasis_k[i] || !ubasis_v[i])
      return fail(KVS_ERR_ARG, "null argument");
    if ((ko == nullptr) != (vo == nullptr)) return fail(KVS_ERR_ARG, "give both k_owner and v_owner, or neither");
    if (!aligned16(k[i]) || !aligned16(v[i]) || !aligned16(basis_k[i]) || !aligned16(basis_v[i]) ||
        !aligned16(ubasis_k[i]) || !aligned16(ubasis_v[i]) || (ko && (!aligned16(ko) || !aligned16(vo))))
      return fail(KVS_ERR_ALIGN, "rows, bases and outputs must be 16-byte aligned");
  }
  const Plan& p = plan->p;
  const BasisWs w = basis_ws(p, batch, n);
  char* ws = static_cast<char*>(workspace);
  for (int32_t i0 = 0; i0 < n_items; i0 += group) {
    const int32_t cnt = std::min(group, n_items - i0);
    BasisLaunch b = basis_launch(p, n_tokens, n, batch, p.cfg.resid_rank_max, cnt, workspace);
    char* rows_base = ws + cnt * (w.gram + w.evals);
    for (int32_t j = 0; j < cnt; ++j) {
      const int32_t i = i0 + j;
      float* rows[2] = {reinterpret_cast<float*>(rows_base + (2 * j) * w.rows),
                        reinterpret_cast<float*>(rows_base + (2 * j + 1) * w.rows)};
      EncodeLaunch e;
      const void* x[2] = {k[i], v[i]};
      const void* xo[2] = {k_owner && k_owner[i] ? k_owner[i] : k[i], v_owner && v_owner[i] ? v_owner[i] : v[i]};
      const void* bases[2] = {basis_k[i], basis_v[i]};
      for (int side = 0; side < 2; ++side) {
        e.x[side] = x[side];
        e.xo[side] = xo[side];
        e.basis[side] = bases[side];
        e.ubasis[side] = nullptr;
        e.c_out[side] = nullptr;
        e.d_out[side] = nullptr;
        e.s_out[side] = nullptr;
        e.e_out[side] = rows[side];
      }
      e.rank = nullptr;
      e.n_tokens = n_tokens;
      e.n = n;
      e.batch = batch;
      e.n_kv_heads = p.cfg.n_kv_heads;
      e.head_dim = p.cfg.head_dim;
      e.residual_mode = 1;
      if ((st = hip_status(launch_encode(e, stream), "residual rows launch")) != KVS_OK) return st;
      b.x[2 * j][0] = rows[0];
      b.x[2 * j][1] = nullptr;
      b.x[2 * j + 1][0] = rows[1];
      b.x[2 * j + 1][1] = nullptr;
      b.out[2 * j] = ubasis_k[i];
      b.out[2 * j + 1] = ubasis_v[i];
    }
    b.rows_f32 = 1;
    if ((st = hip_status(launch_basis(b, stream), "residual basis launch")) != KVS_OK) return st;
  }
  return KVS_OK;
}

extern "C" kvs_status kvs_residual_basis(const kvs_plan* plan, const void* k, const void* v,
                                         const void* k_owner, const void* v_owner,
                                         const void* basis_k, const void* basis_v,
                                         const int32_t* n_tokens, int32_t n, int32_t batch,
                                         void* ubasis_k, void* ubasis_v, void* workspace,
                                         size_t ws_bytes, void* stream) {
  return kvs_residual_bases(plan, 1, &k, &v, &k_owner, &v_owner, &basis_k, &basis_v, n_tokens, n,
                            batch, &ubasis_k, &ubasis_v, workspace, ws_bytes, stream);
}

namespace kvs {
KernelEvents take_kernel_events() {
  const KernelEvents ev = g_next_events;
  g_next_events = KernelEvents{};
  return ev;
}
}  // namespace kvs

extern "C" kvs_status kvs_time_next_launch(void* start_event, void* stop_event) {
  clear_error();
  g_next_events.start = start_event;
  g_next_events.stop = stop_event;
  return KVS_OK;
}
