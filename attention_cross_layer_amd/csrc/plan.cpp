// Host-side planner: sharing-map validation, owner-slot numbering, cache
// layout sizes and the split-K partition choice.  Pure C++ (no HIP).
//
// Map semantics: the CLA page ("Reducing Transformer Key-Value Cache Size with
// Cross-Layer Attention", Methodology) has some layers compute K/V and the
// others reuse it, so a reusing layer is never a source; DepthGraft
// ("DepthGraft: Structural Regularization through Hierarchical Cross-Layer KV
// Reconstruction", Abstract) reads a pair of stride-aligned sources; the
// cross-layer sharing study ("A Systematic Study of Cross-Layer KV Sharing for
// Efficient LLM Inference", TL;DR) distinguishes bottom configurations (sources
// below the reader) from top/middle ones (sources above, served with diagonal
// masking: such a layer runs before its source has written the current
// token, so its query skips the current position).
#include <cmath>
#include <cstring>
#include <new>

#include "internal.h"

namespace kvs {

static thread_local std::string g_err;

kvs_status fail(kvs_status st, const std::string& msg) {
  g_err = msg;
  return st;
}
void clear_error() { g_err.clear(); }

}  // namespace kvs

using namespace kvs;

static bool is_owner_row(const int32_t* src, const float* w, int32_t l) {
  return src[2 * l] == l && src[2 * l + 1] < 0 && (w == nullptr || w[2 * l] == 1.0f);
}

static kvs_status check_config(const kvs_config* c) {
  if (c->n_layers < 1 || c->n_layers > 4096) return fail(KVS_ERR_ARG, "n_layers out of range");
  if (c->n_kv_heads < 1 || c->n_q_heads < 1 || c->n_q_heads % c->n_kv_heads != 0)
    return fail(KVS_ERR_ARG, "n_q_heads must be a positive multiple of n_kv_heads");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(KVS_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c->dtype != KVS_F32 && c->dtype != KVS_BF16) return fail(KVS_ERR_ARG, "bad dtype");
  if (c->kind != KVS_DENSE && c->kind != KVS_FACTORIZED) return fail(KVS_ERR_ARG, "bad kind");
  if (c->max_batch < 1 || c->max_ctx < 1) return fail(KVS_ERR_ARG, "max_batch/max_ctx must be >= 1");
  const int64_t pages = (int64_t(c->max_ctx) + kPage - 1) / kPage;
  if (pages * c->max_batch > (int64_t(1) << 30)) return fail(KVS_ERR_RANGE, "cache too large");
  const int32_t group = c->n_q_heads / c->n_kv_heads;
  if (c->kind == KVS_DENSE) {
    if (!decode_shape_supported(c->dtype, c->head_dim, group, 1))
      return fail(KVS_ERR_UNSUPPORTED, "no decode kernel for this dtype/head_dim/group size");
  } else {
    if (c->dtype != KVS_BF16) return fail(KVS_ERR_UNSUPPORTED, "factorized cache is bf16 only");
    // the factorized kernels address one slot's or layer's pages through
    // 32-bit buffer offsets (4 KiB of coefficients per page and KV head),
    // with 2^31 as the out-of-range offset
    if (pages * c->max_batch * c->n_kv_heads > (int64_t(1) << 19))
      return fail(KVS_ERR_UNSUPPORTED, "factorized cache too large: max_batch * pages * n_kv_heads must be <= 2^19");
    if (!fact_shape_supported(c->head_dim, group, c->basis_rank, c->resid_rank_max))
      return fail(KVS_ERR_UNSUPPORTED, "no factorized kernel for this head_dim/group/ranks");
  }
  return KVS_OK;
}

extern "C" kvs_status kvs_share_plan(const kvs_config* cfg, const int32_t* src, const float* w,
                                     kvs_plan** out) {
  clear_error();
  if (!cfg || !src || !out) return fail(KVS_ERR_ARG, "null argument");
  *out = nullptr;
  kvs_status st = check_config(cfg);
  if (st != KVS_OK) return st;
  const int32_t L = cfg->n_layers;
  for (int32_t l = 0; l < L; ++l) {
    const int32_t s0 = src[2 * l], s1 = src[2 * l + 1];
    if (s0 < 0 || s0 >= L) return fail(KVS_ERR_MAP, "layer " + std::to_string(l) + ": source out of range");
    if (!(s1 == -1 || (s1 >= 0 && s1 < L)))
      return fail(KVS_ERR_MAP, "layer " + std::to_string(l) + ": second source out of range");
    const int n = s1 < 0 ? 1 : 2;
    if (w)
      for (int j = 0; j < n; ++j)
        if (!std::isfinite(w[2 * l + j]))
          return fail(KVS_ERR_MAP, "layer " + std::to_string(l) + ": non-finite weight");
    if (cfg->kind == KVS_FACTORIZED && n > 1)
      return fail(KVS_ERR_UNSUPPORTED, "factorized plans take one source per layer");
    if ((s0 == l || s1 == l) && !is_owner_row(src, w, l))
      return fail(KVS_ERR_MAP, "layer " + std::to_string(l) + ": a self-reference must be the plain owner row");
    if (!is_owner_row(src, w, s0) || (n == 2 && !is_owner_row(src, w, s1)))
      return fail(KVS_ERR_NOT_SOURCE, "layer " + std::to_string(l) + ": source owns no cache entries");
  }
  kvs_plan* plan = new (std::nothrow) kvs_plan;
  if (!plan) return fail(KVS_ERR_ARG, "out of host memory");
  Plan& p = plan->p;
  p.cfg = *cfg;
  p.layers.resize(L);
  std::vector<int32_t> slot_of(L, -1);
  for (int32_t l = 0; l < L; ++l)
    if (is_owner_row(src, w, l)) {
      slot_of[l] = p.n_slots++;
      p.last_owner = l;
    }
  for (int32_t l = 0; l < L; ++l) {
    kvs_layer_info& li = p.layers[l];
    li.owns_kv = slot_of[l] >= 0 && src[2 * l] == l;
    li.n_src = src[2 * l + 1] < 0 ? 1 : 2;
    for (int j = 0; j < 2; ++j) {
      const bool used = j < li.n_src;
      li.src_layer[j] = used ? src[2 * l + j] : -1;
      li.src_slot[j] = used ? slot_of[src[2 * l + j]] : -1;
      li.weight[j] = used ? (w ? w[2 * l + j] : 1.0f) : 0.0f;
    }
    if (li.n_src == 2) ++p.n_mixed;
    li.masks_current = (li.src_layer[0] > l || li.src_layer[1] > l) ? 1 : 0;
  }
  if (p.n_mixed > 0 &&
      !decode_shape_supported(cfg->dtype, cfg->head_dim, cfg->n_q_heads / cfg->n_kv_heads, 2)) {
    delete plan;
    return fail(KVS_ERR_UNSUPPORTED, "no two-source decode kernel for this dtype/head_dim/group size");
  }
  p.pages_per_seq = (cfg->max_ctx + kPage - 1) / kPage;
  p.n_phys_pages = p.pages_per_seq * cfg->max_batch;
  *out = plan;
  return KVS_OK;
}

extern "C" void kvs_plan_free(kvs_plan* plan) { delete plan; }

extern "C" kvs_status kvs_plan_layer(const kvs_plan* plan, int32_t layer, kvs_layer_info* out) {
  clear_error();
  if (!plan || !out) return fail(KVS_ERR_ARG, "null argument");
  if (layer < 0 || layer >= plan->p.cfg.n_layers) return fail(KVS_ERR_ARG, "layer out of range");
  *out = plan->p.layers[layer];
  return KVS_OK;
}

extern "C" kvs_status kvs_plan_summary(const kvs_plan* plan, kvs_plan_info* out) {
  clear_error();
  if (!plan || !out) return fail(KVS_ERR_ARG, "null argument");
  out->n_layers = plan->p.cfg.n_layers;
  out->n_slots = plan->p.n_slots;
  out->last_owner_layer = plan->p.last_owner;
  out->n_mixed_layers = plan->p.n_mixed;
  return KVS_OK;
}

extern "C" kvs_status kvs_cache_layout(const kvs_plan* plan, kvs_cache_sizes* out) {
  clear_error();
  if (!plan || !out) return fail(KVS_ERR_ARG, "null argument");
  const Plan& p = plan->p;
  const kvs_config& c = p.cfg;
  std::memset(out, 0, sizeof(*out));
  out->page_tokens = kPage;
  out->pages_per_seq = p.pages_per_seq;
  out->n_phys_pages = p.n_phys_pages;
  out->n_slots = p.n_slots;
  out->page_table_bytes = size_t(c.max_batch) * p.pages_per_seq * sizeof(int32_t);
  const size_t page_rows = size_t(p.n_phys_pages) * c.n_kv_heads * kPage;
  if (c.kind == KVS_DENSE) {
    out->k_pool_bytes = size_t(p.n_slots) * page_rows * c.head_dim * elem_bytes(c.dtype);
    out->v_pool_bytes = out->k_pool_bytes;
  } else {
    out->coef_pool_bytes = size_t(p.n_slots) * page_rows * c.basis_rank * 2;
    out->resid_pool_bytes = size_t(c.n_layers) * page_rows * c.resid_rank_max;
    out->scale_pool_bytes = size_t(c.n_layers) * page_rows * 2;
    out->rank_pool_bytes = size_t(p.n_phys_pages) * kPage * 2;
    out->basis_bytes = size_t(p.n_slots) * c.n_kv_heads * c.basis_rank * c.head_dim * 2;
    out->resid_basis_bytes = size_t(c.n_layers) * c.n_kv_heads * c.resid_rank_max * c.head_dim * 2;
  }
  return KVS_OK;
}

// Split-K choice.  A decode launch has one 4-wave workgroup per (partition,
// KV head, sequence), and at least 4 pages (one per wave) per partition, at
// most max_decode_splits() partitions.  Targets, from split sweeps on one
// MI355X (cache flushed before each call):
//  * the factorized kernel and the bf16 MFMA kernel (hd 64, and hd 128 at
//    G = 16): one workgroup per CU (256); with S = 1 the merge launch
//    disappears as well;
//  * the VALU kernel (hd 128, fp32, two sources): three workgroups per four
//    CUs (192) when a call streams more than 384 MB, and for smaller calls
//    whose (sequence, KV head) count reaches 192 to 224 workgroups with a
//    whole number of partitions; other small calls take four per CU (1024)
//    with S <= 32.  At 64K context fewer streams read HBM faster: 192
//    workgroups against 256, kernel alone, two alternations on one box:
//    154.1-155.8 vs 157.9-159.0 us at batch 4, 83.0-83.5 vs 85.6-86.8 at
//    batch 2, 302.8-303.3 vs 311.5-317.0 at batch 8 (224 and 160 workgroups
//    in between and below: 156.3-157.9, 173.0-174.0 at batch 4).  The same
//    holds for 134-268 MB calls (8 KV heads, kernel alone, 192 against 1024
//    or 32 partitions: batch x ctx 8 x 8K 45.7 vs 50.4 us, 4 x 16K 45.3 vs
//    50.6, 2 x 32K 45.3 vs 53.6, 1 x 64K 45.4 vs 49.9, 8 x 4K 27.2 vs 29.0,
//    1 x 32K 27.2 vs 29.4, 2 x 16K 27.4 vs 28.5); where 192 is out of reach
//    (16 or 32 sequences: 256 workgroups at S = 2 or 1) 512 to 2048
//    workgroups do as well or better (16 x 4K: 50.1 at 256, 50.7 at 1024).
static const int32_t kGroupsPerCu1 = 256;
static const int32_t kGroupsLarge = 192;
static const int32_t kGroupsLargeMax = 224;
static const int32_t kGroupsPerCu4 = 1024;
static const double kSmallCallBytes = 384.0 * (1 << 20);

extern "C" kvs_status kvs_decode_splits(const kvs_plan* plan, int32_t batch, int32_t max_seq_len,
                                        int32_t* n_splits) {
  clear_error();
  if (!plan || !n_splits) return fail(KVS_ERR_ARG, "null argument");
  if (batch < 1 || batch > plan->p.cfg.max_batch) return fail(KVS_ERR_RANGE, "batch out of range");
  const kvs_config& c = plan->p.cfg;
  int32_t seq = max_seq_len < 1 ? 1 : (max_seq_len > c.max_ctx ? c.max_ctx : max_seq_len);
  const int32_t pages = (seq + kPage - 1) / kPage;
  const int32_t groups = batch * c.n_kv_heads;
  const int32_t G = c.n_q_heads / c.n_kv_heads;
  const bool mfma_kernel = c.dtype == KVS_BF16 && ((c.head_dim == 64 && G <= 32) || (c.head_dim == 128 && G == 16));
  int32_t target = kGroupsPerCu1, s_max = max_decode_splits();
  if (c.kind == KVS_DENSE && !mfma_kernel) {
    const double call_bytes = double(groups) * pages * kPage * c.head_dim * 2 * elem_bytes(c.dtype);
    const int32_t grid_large = ((kGroupsLarge + groups - 1) / groups) * groups;
    if (call_bytes > kSmallCallBytes || (G < 8 && grid_large <= kGroupsLargeMax)) {
      target = kGroupsLarge;
    } else if (G < 8) {
      target = kGroupsPerCu4;
      s_max = 32;
    } else {
      // groups of 8 hold one wave per SIMD: more workgroups than CUs only
      // queue (8 heads at hd 128, batch 4 x 16K: 52.0, 55.9, 65.1 us at
      // 256, 512, 1024 workgroups)
      target = kGroupsPerCu1;
    }
  }
  int32_t s = (target + groups - 1) / groups;
  const int32_t cap = pages / 4;
  if (s > cap) s = cap;
  if (s > s_max) s = s_max;
  if (s < 1) s = 1;
  *n_splits = s;
  return KVS_OK;
}

// Workspace: per-partition partial results [B][Hq][S][W] fp32 (W = hd for a
// dense plan, R + Rmax coefficients for a factorized one), then the running
// maxima and sums [B][Hq][S] fp32 each.
extern "C" kvs_status kvs_decode_workspace_size(const kvs_plan* plan, int32_t batch,
                                                int32_t n_splits, size_t* bytes) {
  clear_error();
  if (!plan || !bytes) return fail(KVS_ERR_ARG, "null argument");
  if (batch < 1 || batch > plan->p.cfg.max_batch) return fail(KVS_ERR_RANGE, "batch out of range");
  if (n_splits < 1 || n_splits > max_decode_splits()) return fail(KVS_ERR_RANGE, "n_splits out of range");
  const kvs_config& c = plan->p.cfg;
  // a factorized plan's partial results live in the R + Rmax coefficient space
  const int32_t width = c.kind == KVS_DENSE ? c.head_dim : c.basis_rank + c.resid_rank_max;
  // per partition row: the partial result, its maximum and sum, and for a
  // factorized plan the entropy accumulator of the router statistics
  const int32_t extra = c.kind == KVS_DENSE ? 2 : 3;
  *bytes = size_t(batch) * c.n_q_heads * n_splits * (width + extra) * sizeof(float);
  return KVS_OK;
}

extern "C" const char* kvs_last_error(void) { return kvs::g_err.c_str(); }
