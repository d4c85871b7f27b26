// Library-internal declarations shared by the host planner, the ABI glue and
// the HIP launchers.  Nothing here is exported.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "kvshare.h"

namespace kvs {

constexpr int kPage = 64;   // tokens per page == keys per decode tile
// Lanes that share one key's dot product in the decode; it fixes the K page
// layout [kWays][NCH/kWays][64/kWays][kWays][E] (E elements per 16 bytes,
// NCH = 16-byte chunks per key row): chunk c of token t sits at
// (((t / (64/kWays)) * (NCH/kWays) + c / kWays) * 64 + (t % (64/kWays)) * kWays
//  + c % kWays) * E.
constexpr int kWays = 8;

// Element offset of chunk c (E elements) of token t within a K page.
inline constexpr int k_chunk_offset(int t, int c, int nch, int e) {
  return (((t / (kPage / kWays)) * (nch / kWays) + c / kWays) * kPage + (t % (kPage / kWays)) * kWays +
          c % kWays) * e;
}

struct Plan {
  kvs_config cfg;
  std::vector<kvs_layer_info> layers;
  int32_t n_slots = 0;
  int32_t last_owner = -1;
  int32_t n_mixed = 0;
  int32_t pages_per_seq = 0;
  int32_t n_phys_pages = 0;
};

// thread-local error text
kvs_status fail(kvs_status st, const std::string& msg);
void clear_error();

inline size_t elem_bytes(int32_t dtype) { return dtype == KVS_F32 ? 4 : 2; }

// Whether the decode kernels are instantiated for this shape and source count.
bool decode_shape_supported(int32_t dtype, int32_t head_dim, int32_t group, int32_t n_src);
// Largest split-K partition count one decode launch merges.
int max_decode_splits();

// ------------------------------------------------------------ HIP launchers
// Implemented in the .hip files; each returns a hipError_t value (0 = ok).

// hipEvent_t pair a launcher attaches to its main kernel (hipExtLaunchKernel:
// start and end of that kernel's execution); both null: a plain launch.
struct KernelEvents {
  void* start = nullptr;
  void* stop = nullptr;
};
// The events kvs_time_next_launch armed on this thread, cleared by the call.
KernelEvents take_kernel_events();

struct DecodeLaunch {
  const void* k_pool;          // base of the K pool
  const void* v_pool;
  const int32_t* page_table;
  int32_t pages_per_seq;
  int32_t n_phys_pages;
  int32_t n_kv_heads;
  int32_t n_q_heads;
  int32_t head_dim;
  int32_t group;
  int32_t dtype;
  int64_t slot_stride;         // elements per slot
  int32_t n_src;
  int32_t slot[2];
  float weight[2];
  const void* q;
  const int32_t* seq_len;
  int32_t max_ctx;
  int32_t key_excl;            // 1: the current position is masked (source above the layer)
  int32_t batch;
  int32_t n_splits;
  float scale_log2;            // log2(e) / sqrt(hd)
  float* ws;                   // workspace base
  void* out;
  int32_t out_dtype;
  KernelEvents ev;             // on the split-K partition kernel
};
int launch_decode(const DecodeLaunch& a, void* stream);

struct AppendLaunch {
  void* k_pool;
  void* v_pool;
  const int32_t* page_table;
  int32_t pages_per_seq;
  int32_t n_phys_pages;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t dtype;
  int64_t slot_offset;         // elements to the layer's slot
  const void* k;
  const void* v;
  int32_t n;
  const int32_t* start_pos;
  int32_t batch;
  int32_t max_ctx;
};
int launch_append(const AppendLaunch& a, void* stream);

bool prefill_shape_supported(int32_t head_dim, int32_t group, int32_t n_src);

struct PrefillLaunch {
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_table;
  int32_t pages_per_seq;
  int32_t n_phys_pages;
  int32_t n_kv_heads;
  int32_t n_q_heads;
  int32_t head_dim;
  int64_t slot_stride;
  int32_t n_src;
  int32_t slot[2];
  float weight[2];
  const void* q;
  int32_t n;
  const int32_t* seq_len;
  int32_t max_ctx;
  int32_t key_excl;            // 1: the current position is masked (source above the layer)
  int32_t batch;
  int32_t causal;
  float scale_log2;
  void* out;
  int32_t out_dtype;
  KernelEvents ev;
};
int launch_prefill(const PrefillLaunch& a, void* stream);

struct FactAppendLaunch {
  void* ck_pool; void* cv_pool;
  void* dk_pool; void* dv_pool;
  void* sk_pool; void* sv_pool;
  void* rank_pool;
  const int32_t* page_table;
  int32_t pages_per_seq;
  int32_t n_phys_pages;
  int32_t n_kv_heads;
  int32_t basis_rank;
  int32_t resid_rank_max;
  int32_t coef_slot;           // -1: no coefficient write
  int32_t layer;
  const void* ck; const void* cv;
  const int8_t* dk; const int8_t* dv;
  const void* sk; const void* sv;
  const uint8_t* rank;
  int32_t n;
  const int32_t* start_pos;
  int32_t batch;
  int32_t max_ctx;
};
int launch_fact_append(const FactAppendLaunch& a, void* stream);

struct FactDecodeLaunch {
  const void* ck_pool; const void* cv_pool;
  const void* dk_pool; const void* dv_pool;
  const void* sk_pool; const void* sv_pool;
  const void* rank_pool;
  const void* basis_k; const void* basis_v;
  const void* ubasis_k; const void* ubasis_v;
  const int32_t* page_table;
  int32_t pages_per_seq;
  int32_t n_phys_pages;
  int32_t n_kv_heads;
  int32_t n_q_heads;
  int32_t head_dim;
  int32_t basis_rank;
  int32_t resid_rank_max;
  int32_t coef_slot;
  int32_t layer;
  const void* q;
  const int32_t* seq_len;
  int32_t max_ctx;
  int32_t key_excl;            // 1: the current position is masked (source above the layer)
  int32_t batch;
  int32_t n_splits;
  float scale_log2;
  float* ws;
  void* out;
  int32_t out_dtype;
  float* stats;                // [B][Hq][2] entropy, peak probability; or null
  KernelEvents ev;             // on the split-K partition kernel
};
int launch_fact_decode(const FactDecodeLaunch& a, void* stream);
bool fact_shape_supported(int32_t head_dim, int32_t group, int32_t basis_rank,
                          int32_t resid_rank_max);

struct FactPrefillLaunch {
  const void* ck_pool; const void* cv_pool;
  const void* dk_pool; const void* dv_pool;
  const void* sk_pool; const void* sv_pool;
  const void* rank_pool;
  const void* basis_k; const void* basis_v;
  const void* ubasis_k; const void* ubasis_v;
  const int32_t* page_table;
  int32_t pages_per_seq;
  int32_t n_phys_pages;
  int32_t n_kv_heads;
  int32_t n_q_heads;
  int32_t head_dim;
  int32_t coef_slot;
  int32_t layer;
  const void* q;
  int32_t n;
  const int32_t* seq_len;
  int32_t max_ctx;
  int32_t key_excl;            // 1: the current position is masked (source above the layer)
  int32_t batch;
  int32_t causal;
  float scale_log2;
  void* out;
  int32_t out_dtype;
  KernelEvents ev;
};
int launch_fact_prefill(const FactPrefillLaunch& a, void* stream);
bool fact_prefill_shape_supported(int32_t head_dim, int32_t group, int32_t basis_rank,
                                  int32_t resid_rank_max);

// Encoder: side 0 = K, side 1 = V.
struct EncodeLaunch {
  const void* x[2];            // [B][n][Hkv][hd] bf16 rows of the layer
  const void* xo[2];           // rows of the pair's coefficient-writing layer
  const void* basis[2];        // [Hkv][R][hd] bf16
  const void* ubasis[2];       // [Hkv][Rmax][hd] bf16 (codes mode)
  void* c_out[2];              // [B][n][Hkv][R] bf16 or null
  void* d_out[2];              // [B][n][Hkv][Rmax] int8
  void* s_out[2];              // [B][n][Hkv] fp16
  float* e_out[2];             // residual mode: [B][n][Hkv][hd] fp32
  const uint8_t* rank;         // [B][n]
  const int32_t* n_tokens;     // residual mode: [B]
  int32_t n;
  int32_t batch;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t residual_mode;
};
int launch_encode(const EncodeLaunch& a, void* stream);
bool encode_shape_supported(int32_t head_dim, int32_t basis_rank, int32_t resid_rank_max);

// Basis builder: Gram matrices of the rows, then leading eigenvectors, for
// up to kMaxBasisSets matrix sets per launch (a set = K or V of one basis).
constexpr int kMaxBasisSets = 64;
struct BasisLaunch {
  int32_t n_sets;
  const void* x[kMaxBasisSets][2];   // [set][source] rows, [B][n][Hkv][hd]; source 1 may be null
  int32_t rows_f32;            // rows are fp32 (residual rows) instead of bf16
  const int32_t* n_tokens;     // [B]
  int32_t n;
  int32_t batch;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t k_out;
  float* gram;                 // workspace [set][Hkv][hd][hd]
  float* evals;                // workspace [set][Hkv][hd]
  void* out[kMaxBasisSets];    // [Hkv][k_out][hd] bf16 per set
};
int launch_basis(const BasisLaunch& a, void* stream);

struct RouteLaunch {
  const float* stats;          // [n_sets][B][Hq][2]
  int32_t n_sets;
  const int32_t* n_keys;       // [B]
  int32_t batch;
  int32_t n_q_heads;
  float entropy_focused, entropy_diffuse, peak_focused;
  int32_t rank_focused, rank_mid, rank_diffuse;
  uint8_t* rank_out;           // [B]
};
int launch_route(const RouteLaunch& a, void* stream);

const char* hip_error_name(int err);

// Device scratch of kvs_attn_decode_noalloc: its size, and this device's
// address of it (taken once per device with hipGetSymbolAddress); returns a
// hipError_t value.
size_t scratch_bytes();
int scratch_address(void** out);

}  // namespace kvs

struct kvs_plan {
  kvs::Plan p;
};
