// Causal (or full) prefill-chunk attention over the factorized cache, in the
// 48-wide coefficient space, on MFMA with fp32 accumulation (fp16 operands
// for the scores, bf16 for the values).
//
// Keys and values follow DepthWeave-KV ("DepthWeave-KV: Smarter KV Cache
// Compression by Sharing Across Layers and Adapting Per Token", Core
// Mechanism and Framework Shift); per KV head
//   K_l[t] = c[t] B_pair + s_l[t] * sum_{j < r_t} d_l[t, j] U_l[j]   (V alike).
// No key or value row is rebuilt.  With q~ = B^K q and u~ = U^K q, the score
// of key t is c_t . q~ + s_t (d_t . u~), and the output is
// (sum_t p_t c^V_t) B^V + (sum_t p_t s^V_t d^V_t) U^V: the same values as
// attention over the rebuilt rows (up to rounding order), with each
// (query, key) pair contracting 48 coefficients on each side instead of
// head_dim, and the bases entering once per query row at both ends.
//
// Decomposition (v_mfma_f32_32x32x16_f16 / _bf16: lane l of A/B holds row or column
// l%32 and k = 8(l/32)+e; result register r of lane l is row
// 8(r/4) + 4(l/32) + r%4, column l%32):
//   workgroup = 4 waves on one KV head, each owning 32 query rows of one head
//   (min(G, 4) heads x 4/min(G, 4) blocks of 32 positions), as the dense
//   prefill.
//   prologue  Q~^T = B^K Q^T and U~^T = [U^K; 0] Q^T (2 hd/16 MFMAs), each
//             rounded to fp16.  Their result registers serve as B operands
//             unchanged: register r holds
//             coefficient 8(r/4) + 4(l/32) + r%4, so in every product over the
//             coefficient space the k index visits coefficients in that order.
//             Staged tiles store each 16-wide group with its quads 1 and 2
//             swapped (swz16), which puts a lane's 8 operand values in one
//             16-byte LDS read.
//   per 64-key page, double-buffered in LDS, the global loads of the next two
//   pages in two register stages (their meta entries one page further ahead):
//     staging  C^K [64 keys][32] (converted to fp16: exact for magnitudes
//              up to 65504), S^K = s^K d^K [64][16] (codes taken from their
//              rank-packed granules, scaled in fp32, rounded to fp16),
//              C^V^T [32][64 keys], S^V^T = (s^V d^V)^T [16][64 keys] (bf16,
//              the scaled codes rounded to bf16); keys
//              past the sequence end, or on a corrupt page-table entry, are
//              zero on the value side and have no codes.
//     S^T = C^K Q~^T + S^K U~^T   6 fp16 MFMAs per wave (bf16 operands
//              would need a high part and a remainder of Q~, U~ each, twice
//              the products, for the same accuracy)
//     softmax  online per query row, as the dense prefill
//     A^T += C^V^T P^T, D^T += S^V^T P^T   8 MFMAs (rows 16..31 of the second
//              product's A operand are zero)
//   epilogue  O^T = B^V^T A^T + U^V^T D^T with A and D split into a bf16 high
//             part and the bf16 rounding of the remainder (two products each);
//             B^V and U^V of the head are staged transposed in LDS.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "common.h"
#include "internal.h"

namespace kvs {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

using dev::kOOB;
using dev::ld16;
using dev::ld2;
using dev::ld4;
using dev::rsrc;

constexpr int kR = 32;            // basis rank
constexpr int kRM = 16;           // residual codes per token at most
constexpr int kGranules = 128;    // 8-byte code granules per page blob
constexpr int kRows = 32;         // query rows per wave
constexpr int kVRow = 64 + 8;     // C^V^T / S^V^T row pitch in keys
constexpr int kBRow = 48 + 8;     // transposed basis row pitch in coefficients
constexpr int kCK = 64 * kR;      // staged page parts, bf16 elements
constexpr int kSK = 64 * kRM;
constexpr int kCV = kR * kVRow;
// S^V^T is staged with 32 rows: rows 0..15 the scaled value codes of each
// page, row 16 ones and rows 17..31 zeros, written once per launch, so the
// 32-row value product accumulates the softmax's running sum in its row 16
// and needs no per-tile selects for the rows past the codes
constexpr int kSV = 2 * kRM * kVRow;
constexpr int kOnesRow = kRM;
constexpr int kTile = kCK + kSK + kCV + kSV;

struct FactPrefillParams {
  const uint16_t* ck; const uint16_t* cv;   // cK / cV pages of the pair's slot
  const int8_t* dk; const int8_t* dv;       // code pages of the layer
  const uint16_t* sk; const uint16_t* sv;   // scale pages of the layer
  const uint16_t* meta;
  const uint16_t* bk; const uint16_t* bv;   // [Hkv][R][hd] of the slot
  const uint16_t* uk; const uint16_t* uv;   // [Hkv][RM][hd] of the layer
  const int32_t* page_table;
  int32_t pages_per_seq;
  int32_t n_phys_pages;
  int32_t n_kv_heads;
  int32_t n_q_heads;
  const uint16_t* q;    // [B][n][Hq][hd]
  int32_t n;
  const int32_t* seq_len;
  int32_t max_ctx;
  int32_t causal;
  int32_t key_excl;     // 1: query at P sees keys 0..P-1 (source above the layer)
  float scale_log2;
  void* out;            // [B][n][Hq][hd]
  int32_t out_bf16;
  int32_t n_pos_groups;
  int32_t head_groups;
};

__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma32h(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                0, 0, 0);
}

// two floats -> packed fp16 pair, round to nearest even
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  const f16x2_t v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// eight bf16 values -> eight fp16 values (exact for magnitudes in
// [2^-14, 65504]; smaller ones keep fp16's subnormal precision)
__device__ __forceinline__ uint4 bf16x8_to_f16(const uint4& x) {
  auto cv = [](uint32_t w) { return pack_f16(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)); };
  return make_uint4(cv(x.x), cv(x.y), cv(x.z), cv(x.w));
}

// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

constexpr float kBumpLog2 = 8.f;                // lazy-maximum slack (log2 units)

// Position of entry j inside its 16-wide group with quads 1 and 2 swapped
// (an involution; higher bits of j pass through).
__device__ __forceinline__ int swz16(int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); }

// bf16 high parts and bf16 remainders of 8 accumulator registers
__device__ __forceinline__ void split8(const f32x16_t& x, int r0, uint4& hi, uint4& lo) {
  float h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float v = x[r0 + e];
    h[e] = (float)(__bf16)v;
    l[e] = v - h[e];
  }
  hi = make_uint4(pack_bf16(h[0], h[1]), pack_bf16(h[2], h[3]), pack_bf16(h[4], h[5]), pack_bf16(h[6], h[7]));
  lo = make_uint4(pack_bf16(l[0], l[1]), pack_bf16(l[2], l[3]), pack_bf16(l[4], l[5]), pack_bf16(l[6], l[7]));
}

// four int8 codes (the bytes of w) times s, as four fp16 values
__device__ __forceinline__ uint2 scaled_codes_f16(uint32_t w, float s) {
  return make_uint2(pack_f16(s * (float)(int8_t)(w & 0xffu), s * (float)(int8_t)((w >> 8) & 0xffu)),
                    pack_f16(s * (float)(int8_t)((w >> 16) & 0xffu), s * (float)(int8_t)(w >> 24)));
}

// eight accumulator registers as fp16 (round to nearest even)
__device__ __forceinline__ uint4 to_f16x8(const f32x16_t& x, int r0) {
  return make_uint4(pack_f16(x[r0], x[r0 + 1]), pack_f16(x[r0 + 2], x[r0 + 3]), pack_f16(x[r0 + 4], x[r0 + 5]),
                    pack_f16(x[r0 + 6], x[r0 + 7]));
}

// four int8 codes (the bytes of w) times s, as four bf16 values
__device__ __forceinline__ uint2 scaled_codes(uint32_t w, float s) {
  return make_uint2(pack_bf16(s * (float)(int8_t)(w & 0xffu), s * (float)(int8_t)((w >> 8) & 0xffu)),
                    pack_bf16(s * (float)(int8_t)((w >> 16) & 0xffu), s * (float)(int8_t)(w >> 24)));
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return __half2float(__ushort_as_half((unsigned short)h));
}

template <int HD, int G>
__global__ __launch_bounds__(256, 2) void fact_prefill_kernel(FactPrefillParams a) {
  constexpr int HW = G < 4 ? G : 4;          // heads per workgroup
  constexpr int PB = 4 / HW;                 // 32-row position blocks per workgroup
  constexpr int KS = HD / 16;                // MFMA k-steps over the head dim
  constexpr int MB = HD / 32;                // 32-dim blocks of O^T
  static_assert(HD * kBRow <= 2 * kTile, "transposed bases fit in the page buffers");

  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;                  // k half of the MFMA operands
  const int col = lane & 31;                 // MFMA column owned by this lane

  // ---- which (sequence, KV head, heads, positions)
  const int b = blockIdx.y;
  int x = blockIdx.x;
  const int kvh = x % a.n_kv_heads;
  x /= a.n_kv_heads;
  const int hg = x % a.head_groups;
  const int pgrp = a.n_pos_groups - 1 - x / a.head_groups;   // late positions first
  const int head = kvh * G + hg * HW + (wave % HW);
  const int i0 = (pgrp * PB + wave / HW) * kRows;            // this wave's first row
  const int n = a.n;

  const int T = min(max(a.seq_len[b], 0), a.max_ctx);
  const int wg_last_row = min(n, (pgrp + 1) * PB * kRows) - 1;
  int kend = T;
  if (a.causal) kend = min(T, T - n + wg_last_row + 1 - a.key_excl);
  kend = max(kend, 0);
  const int n_tiles = (kend + 63) / 64;

  const int row = i0 + col;
  const bool row_ok = row < n;
  const int pos = T - n + row;
  const int row_kend = !row_ok ? 0 : (a.causal ? max(min(T, pos + 1 - a.key_excl), 0) : T);
  const int wave_kend = (i0 + kRows <= n) ? (a.causal ? max(min(T, T - n + i0 + 1 - a.key_excl), 0) : T) : 0;
  const int unmasked_tiles = wave_kend / 64;

  // ---- global sources of the staged pages
  const uint32_t P = (uint32_t)a.n_phys_pages, H = (uint32_t)a.n_kv_heads;
  const auto r_ck = rsrc(a.ck, P * H * (kPage * kR * 2));
  const auto r_cv = rsrc(a.cv, P * H * (kPage * kR * 2));
  const auto r_dk = rsrc(a.dk, P * H * (kGranules * 8));
  const auto r_dv = rsrc(a.dv, P * H * (kGranules * 8));
  const auto r_sk = rsrc(a.sk, P * H * (kPage * 2));
  const auto r_sv = rsrc(a.sv, P * H * (kPage * 2));
  const auto r_meta = rsrc(a.meta, P * (kPage * 2));
  // page-table entries through the constant address space: scalar loads,
  // whose waits leave the vector loads of the staged pages in flight
  typedef const __attribute__((address_space(4))) int32_t const_i32;
  const_i32* pt = (const_i32*)(a.page_table + (size_t)b * a.pages_per_seq);

  // staging roles of this thread: 16-byte chunk `tid` of the cK and cV pages;
  // codes 4cq..4cq+3 and the scales of key skey
  const int skey = tid >> 2, cq = tid & 3;
  // physical page of tile t, or -1 past the last tile or on a corrupt entry
  auto phys_of = [&](int t) {
    if (t >= n_tiles) return -1;
    const int ph = pt[t];
    return (unsigned)ph < P ? ph : -1;
  };
  auto load_meta = [&](int t, int ph) -> uint32_t {
    const bool on = ph >= 0 && t * 64 + skey < T;
    return ld2(r_meta, on ? ((uint32_t)ph * kPage + skey) * 2 : kOOB);
  };

  // one page's global loads, held in registers until the page is staged
  struct Stage {
    uint4 ck, cv;
    uint32_t dk, dv, sk, sv;
    int ph;
  };
  auto load_tile = [&](int t, int ph, uint32_t meta, Stage& st) {
    st.ph = ph;
    const uint32_t page_kv = (uint32_t)ph * H + kvh;
    const uint32_t cb = ph >= 0 ? page_kv * (kPage * kR * 2) + tid * 16 : kOOB;
    st.ck = ld16(r_ck, cb);
    st.cv = ld16(r_cv, cb);
    // meta is zero for absent keys: rank 0, no granule
    const int rank = min((int)(meta & 0xffu), kRM);
    const uint32_t g = min(meta >> 8, (uint32_t)(kGranules - 2)) + (cq >> 1);
    const uint32_t co = 8 * (cq >> 1) < rank ? page_kv * (kGranules * 8) + g * 8 + 4 * (cq & 1) : kOOB;
    st.dk = ld4(r_dk, co);
    st.dv = ld4(r_dv, co);
    // scales of absent keys (unwritten memory) stay zero: a NaN pattern
    // times a zero code would not
    const uint32_t so = ph >= 0 && t * 64 + skey < T ? (page_kv * kPage + skey) * 2 : kOOB;
    st.sk = ld2(r_sk, so);
    st.sv = ld2(r_sv, so);
  };
  auto store_tile = [&](int t, int buf, const Stage& st) {
    uint16_t* base = lds + buf * kTile;
    const int key0 = t * 64;
    const bool page_ok = st.ph >= 0;
    // C^K: chunk tid of the cK page = coefficients 8cc..8cc+7 of token tk
    {
      const int cc = tid >> 6, tk = tid & 63;
      const int p0 = swz16(8 * cc), p1 = swz16(8 * cc + 4);
      uint16_t* rowp = base + tk * kR;
      const int sw = (tk >> 2) & 3;
      const uint4 ch = bf16x8_to_f16(st.ck);
      *reinterpret_cast<uint2*>(rowp + (((p0 >> 3) ^ sw) << 3) + (p0 & 7)) = make_uint2(ch.x, ch.y);
      *reinterpret_cast<uint2*>(rowp + (((p1 >> 3) ^ sw) << 3) + (p1 & 7)) = make_uint2(ch.z, ch.w);
    }
    // S^K: codes 4cq..4cq+3 of key skey, times its scale
    {
      const float s = half_bits_to_float(st.sk);
      const int p = swz16(4 * cq);
      uint16_t* rowp = base + kCK + skey * kRM;
      *reinterpret_cast<uint2*>(rowp + (((p >> 3) ^ ((skey >> 3) & 1)) << 3) + (p & 7)) = scaled_codes_f16(st.dk, s);
    }
    // C^V^T: chunk tid of the cV page = coefficients ia and ia + 4 of tokens
    // 4tq..4tq+3; absent keys zero
    {
      const int mh = tid >> 6, tq = (tid >> 2) & 15, i4 = tid & 3;
      const int ia = 8 * mh + i4;
      const int k0 = key0 + 4 * tq;
      uint32_t m0 = 0, m1 = 0;
      if (page_ok && key0 + 64 <= T) {          // uniform: a page wholly in range
        m0 = m1 = 0xffffffffu;
      } else if (page_ok) {
        m0 = (k0 < T ? 0x0000ffffu : 0u) | (k0 + 1 < T ? 0xffff0000u : 0u);
        m1 = (k0 + 2 < T ? 0x0000ffffu : 0u) | (k0 + 3 < T ? 0xffff0000u : 0u);
      }
      uint16_t* cvt = base + kCK + kSK;
      const int p = swz16(4 * tq);
      *reinterpret_cast<uint2*>(cvt + ia * kVRow + p) = make_uint2(st.cv.x & m0, st.cv.y & m1);
      *reinterpret_cast<uint2*>(cvt + (ia + 4) * kVRow + p) = make_uint2(st.cv.z & m0, st.cv.w & m1);
    }
    // S^V^T: codes 4cq..4cq+3 of key skey (zero codes for absent keys)
    {
      const float s = half_bits_to_float(st.sv);
      const uint2 w = scaled_codes(st.dv, s);
      uint16_t* svt = base + kCK + kSK + kCV + swz16(skey);
      svt[(4 * cq + 0) * kVRow] = (uint16_t)(w.x & 0xffffu);
      svt[(4 * cq + 1) * kVRow] = (uint16_t)(w.x >> 16);
      svt[(4 * cq + 2) * kVRow] = (uint16_t)(w.y & 0xffffu);
      svt[(4 * cq + 3) * kVRow] = (uint16_t)(w.y >> 16);
    }
  };

  // ---- the permanent rows of both S^V^T buffers (ones, zeros); ordered
  // before their first read by the loop's first barrier
  for (int e = tid; e < 2 * kRM * kVRow; e += 256) {
    const int buf = e / (kRM * kVRow), r = (e / kVRow) % kRM;
    lds[buf * kTile + kCK + kSK + kCV + (kRM + r) * kVRow + e % kVRow] =
        r == 0 ? (uint16_t)0x3F80u : (uint16_t)0u;
  }

  // ---- the first two pages' requests, then the query contraction with the
  // bases.  Two register stages: a page's loads are issued two tiles before
  // it is staged, its meta entries (which the code addresses need) one tile
  // before that.
  Stage sa, sb;
  int ph_2, ph_3;                       // pages of the loop's tiles t + 2, t + 3
  uint32_t meta_2;                      // meta entries of tile t + 2
  {
    const int ph0 = phys_of(0), ph1 = phys_of(1);
    const uint32_t m0 = load_meta(0, ph0), m1 = load_meta(1, ph1);
    ph_2 = phys_of(2);
    meta_2 = load_meta(2, ph_2);
    ph_3 = phys_of(3);
    load_tile(0, ph0, m0, sa);
    load_tile(1, ph1, m1, sb);
  }

  // Q~ and U~ as fp16 (11 significant bits): rounded to bf16 (8 bits) they
  // moved scores enough to take single outputs past 1e-2 where a few keys
  // dominate a row
  uint4 bq[2], bu;
  {
    const int qrow = row_ok ? row : (n - 1);
    const uint16_t* qp = a.q + (((size_t)b * n + qrow) * a.n_q_heads + head) * HD;
    const uint16_t* bkh = a.bk + (size_t)kvh * kR * HD;
    const uint16_t* ukh = a.uk + (size_t)kvh * kRM * HD;
    f32x16_t qt = f32x16_t{}, qu = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 qv = *reinterpret_cast<const uint4*>(qp + (2 * ks + hh) * 8);
      const uint4 ab = *reinterpret_cast<const uint4*>(bkh + col * HD + (2 * ks + hh) * 8);
      uint4 au = *reinterpret_cast<const uint4*>(ukh + (col & 15) * HD + (2 * ks + hh) * 8);
      if (col >= kRM) au = make_uint4(0, 0, 0, 0);
      qt = mfma32(ab, qv, qt);
      qu = mfma32(au, qv, qu);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) bq[ks] = to_f16x8(qt, 8 * ks);
    bu = to_f16x8(qu, 0);
  }

  f32x16_t acc_c = f32x16_t{}, acc_d = f32x16_t{};
  float m_run = -INFINITY;
  const float bump_gap = kBumpLog2 / a.scale_log2;   // in raw score units

  auto tile_step = [&](int t, int buf, Stage& st) {
    // meta entries of tile t + 3 first: loads complete in order, so waiting
    // for them one tile later does not wait for the page loads issued below
    const uint32_t meta_3 = load_meta(t + 3, ph_3);
    const int ph_4 = phys_of(t + 4);
    // a page-table entry outside [0, n_phys_pages) (uniform): its keys get no
    // weight, as the decode skips such a page
    const bool tile_ok = st.ph >= 0;
    store_tile(t, buf, st);
    load_tile(t + 2, ph_2, meta_2, st);     // absent past the last tile
    ph_2 = ph_3;
    meta_2 = meta_3;
    ph_3 = ph_4;
    __syncthreads();
    const uint16_t* base = lds + buf * kTile;

    // ---- S^T = C^K Q~^T + S^K U~^T: two 32-key blocks
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = 32 * kb + col;
      const int sw = (key >> 2) & 3;
      const uint16_t* rowp = base + key * kR;
      const uint4 c0 = *reinterpret_cast<const uint4*>(rowp + (((0 + hh) ^ sw) << 3));
      const uint4 c1 = *reinterpret_cast<const uint4*>(rowp + (((2 + hh) ^ sw) << 3));
      const uint4 dq = *reinterpret_cast<const uint4*>(base + kCK + key * kRM + ((hh ^ ((key >> 3) & 1)) << 3));
      s[kb] = mfma32h(c0, bq[0], f32x16_t{});
      s[kb] = mfma32h(c1, bq[1], s[kb]);
      s[kb] = mfma32h(dq, bu, s[kb]);
    }

    // ---- online softmax for this lane's query row on raw scores
    if (t >= unmasked_tiles || !tile_ok) {
      const int lim = tile_ok ? row_kend : 0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t * 64 + 32 * kb + 8 * (r / 4) + 4 * hh + (r % 4);
          s[kb][r] = key < lim ? s[kb][r] : -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mt = dev::fmax3_ieee(mt, s[kb][r], s[kb][r + 1]);
    mt = dev::fmax_ieee(mt, __shfl_xor(mt, 32));
    // The reference maximum moves only when a score passes it by more than
    // kBumpLog2 in log2 units: probabilities stay <= 2^kBumpLog2 (exact
    // enough in bf16, sums safe in fp32) and the accumulators are rescaled a
    // few times per row instead of at most tiles.  exp2(scale * (s - m)) is
    // one fma; a row with no key yet keeps p = 0.
    const bool bump = mt > m_run + bump_gap;
    const float mn = bump ? mt : m_run;
    const float neg = mn == -INFINITY ? 0.f : -mn * a.scale_log2;
    const float alpha = bump ? dev::fast_exp2(fmaf(m_run, a.scale_log2, neg)) : 1.f;
    m_run = mn;
    uint4 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = dev::fast_exp2(fmaf(s[kb][8 * sh + e], a.scale_log2, neg));
        uint4 w;
        w.x = pack_bf16(p[0], p[1]);
        w.y = pack_bf16(p[2], p[3]);
        w.z = pack_bf16(p[4], p[5]);
        w.w = pack_bf16(p[6], p[7]);
        pb[2 * kb + sh] = w;
      }
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc_c[r] *= alpha;
        acc_d[r] *= alpha;
      }
    }

    // ---- A^T += C^V^T P^T, D^T += S^V^T P^T; step sp covers keys
    // 16sp + 8(e/4) + 4hh + e%4, stored at positions 16sp + 8hh + e
    const uint16_t* cvt = base + kCK + kSK + col * kVRow + 8 * hh;
    const uint16_t* svt = base + kCK + kSK + kCV + col * kVRow + 8 * hh;
#pragma unroll
    for (int sp = 0; sp < 4; ++sp) {
      const uint4 av = *reinterpret_cast<const uint4*>(cvt + 16 * sp);
      const uint4 ad = *reinterpret_cast<const uint4*>(svt + 16 * sp);
      acc_c = mfma32(av, pb[sp], acc_c);
      acc_d = mfma32(ad, pb[sp], acc_d);
    }
  };
  // pairs of tiles, then an odd last one: no conditional step inside the
  // loop, so the waits for each stage's loads see every load issued after it
  int t = 0;
  for (; t + 1 < n_tiles; t += 2) {
    tile_step(t, 0, sa);
    tile_step(t + 1, 1, sb);
  }
  if (t < n_tiles) tile_step(t, 0, sa);

  // ---- epilogue: bases of this KV head, transposed, into the page buffers
  __syncthreads();
  {
    const uint16_t* bvh = a.bv + (size_t)kvh * kR * HD;
    const uint16_t* uvh = a.uv + (size_t)kvh * kRM * HD;
    for (int idx = tid; idx < (kR + kRM) * HD / 8; idx += 256) {
      const int i = idx / (HD / 8), d0 = (idx % (HD / 8)) * 8;
      const uint4 v = *reinterpret_cast<const uint4*>(i < kR ? bvh + i * HD + d0 : uvh + (i - kR) * HD + d0);
      const int p = i < kR ? swz16(i) : kR + swz16(i - kR);
      uint16_t* dst = lds + d0 * kBRow + p;
      dst[0 * kBRow] = (uint16_t)(v.x & 0xffffu);
      dst[1 * kBRow] = (uint16_t)(v.x >> 16);
      dst[2 * kBRow] = (uint16_t)(v.y & 0xffffu);
      dst[3 * kBRow] = (uint16_t)(v.y >> 16);
      dst[4 * kBRow] = (uint16_t)(v.z & 0xffffu);
      dst[5 * kBRow] = (uint16_t)(v.z >> 16);
      dst[6 * kBRow] = (uint16_t)(v.w & 0xffffu);
      dst[7 * kBRow] = (uint16_t)(v.w >> 16);
    }
  }
  __syncthreads();

  uint4 chi[2], clo[2], dhi, dlo;
  split8(acc_c, 0, chi[0], clo[0]);
  split8(acc_c, 8, chi[1], clo[1]);
  split8(acc_d, 0, dhi, dlo);

  // the running sum: row 16 of D^T (register 8 of lanes 0..31; lanes
  // 32..63 hold row 20 there, a zero row)
  const float l_row = acc_d[8] + __shfl_xor(acc_d[8], 32);
  const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
  const size_t obase = (((size_t)b * n + (row_ok ? row : 0)) * a.n_q_heads + head) * HD;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const uint16_t* brow = lds + (32 * mb + col) * kBRow + 8 * hh;
    const uint4 b0 = *reinterpret_cast<const uint4*>(brow);
    const uint4 b1 = *reinterpret_cast<const uint4*>(brow + 16);
    const uint4 b2 = *reinterpret_cast<const uint4*>(brow + 32);
    f32x16_t o = mfma32(b0, chi[0], f32x16_t{});
    o = mfma32(b0, clo[0], o);
    o = mfma32(b1, chi[1], o);
    o = mfma32(b1, clo[1], o);
    o = mfma32(b2, dhi, o);
    o = mfma32(b2, dlo, o);
    if (row_ok) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * mb + 8 * g4 + 4 * hh;
        const float v0 = o[4 * g4 + 0] * inv, v1 = o[4 * g4 + 1] * inv;
        const float v2 = o[4 * g4 + 2] * inv, v3 = o[4 * g4 + 3] * inv;
        if (a.out_bf16) {
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + obase + d) =
              make_uint2(pack_bf16(v0, v1), pack_bf16(v2, v3));
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + obase + d) =
              make_float4(v0, v1, v2, v3);
        }
      }
    }
  }
}

template <int HD, int G>
int run_fact_prefill(FactPrefillParams p, int B, hipStream_t st, const KernelEvents& ev) {
  constexpr int HW = G < 4 ? G : 4;
  constexpr int PB = 4 / HW;
  p.head_groups = G / HW;
  p.n_pos_groups = (p.n + PB * kRows - 1) / (PB * kRows);
  dim3 grid(p.n_pos_groups * p.head_groups * p.n_kv_heads, B);
  launch_main(ev, fact_prefill_kernel<HD, G>, grid, dim3(256), st, p);
  return (int)hipGetLastError();
}

typedef int (*FactPrefillFn)(FactPrefillParams, int, hipStream_t, const KernelEvents&);

template <int HD>
FactPrefillFn pick_g(int G) {
  switch (G) {
    case 1: return run_fact_prefill<HD, 1>;
    case 2: return run_fact_prefill<HD, 2>;
    case 4: return run_fact_prefill<HD, 4>;
    case 8: return run_fact_prefill<HD, 8>;
    default: return nullptr;
  }
}

FactPrefillFn pick(int hd, int G) {
  if (hd == 64) return pick_g<64>(G);
  if (hd == 128) return pick_g<128>(G);
  return nullptr;
}

}  // namespace

bool fact_prefill_shape_supported(int32_t head_dim, int32_t group, int32_t basis_rank,
                                  int32_t resid_rank_max) {
  return basis_rank == kR && resid_rank_max == kRM && pick(head_dim, group) != nullptr;
}

int launch_fact_prefill(const FactPrefillLaunch& a, void* stream) {
  FactPrefillFn fn = pick(a.head_dim, a.n_q_heads / a.n_kv_heads);
  if (!fn) return (int)hipErrorInvalidValue;
  const size_t Hkv = a.n_kv_heads;
  FactPrefillParams p;
  p.ck = static_cast<const uint16_t*>(a.ck_pool) + (size_t)a.coef_slot * a.n_phys_pages * Hkv * kPage * kR;
  p.cv = static_cast<const uint16_t*>(a.cv_pool) + (size_t)a.coef_slot * a.n_phys_pages * Hkv * kPage * kR;
  p.dk = static_cast<const int8_t*>(a.dk_pool) + (size_t)a.layer * a.n_phys_pages * Hkv * kGranules * 8;
  p.dv = static_cast<const int8_t*>(a.dv_pool) + (size_t)a.layer * a.n_phys_pages * Hkv * kGranules * 8;
  p.sk = static_cast<const uint16_t*>(a.sk_pool) + (size_t)a.layer * a.n_phys_pages * Hkv * kPage;
  p.sv = static_cast<const uint16_t*>(a.sv_pool) + (size_t)a.layer * a.n_phys_pages * Hkv * kPage;
  p.meta = static_cast<const uint16_t*>(a.rank_pool);
  p.bk = static_cast<const uint16_t*>(a.basis_k) + (size_t)a.coef_slot * Hkv * kR * a.head_dim;
  p.bv = static_cast<const uint16_t*>(a.basis_v) + (size_t)a.coef_slot * Hkv * kR * a.head_dim;
  p.uk = static_cast<const uint16_t*>(a.ubasis_k) + (size_t)a.layer * Hkv * kRM * a.head_dim;
  p.uv = static_cast<const uint16_t*>(a.ubasis_v) + (size_t)a.layer * Hkv * kRM * a.head_dim;
  p.page_table = a.page_table;
  p.pages_per_seq = a.pages_per_seq;
  p.n_phys_pages = a.n_phys_pages;
  p.n_kv_heads = a.n_kv_heads;
  p.n_q_heads = a.n_q_heads;
  p.q = static_cast<const uint16_t*>(a.q);
  p.n = a.n;
  p.seq_len = a.seq_len;
  p.max_ctx = a.max_ctx;
  p.causal = a.causal;
  p.key_excl = a.key_excl;
  p.scale_log2 = a.scale_log2;
  p.out = a.out;
  p.out_bf16 = a.out_dtype == KVS_BF16;
  return fn(p, a.batch, static_cast<hipStream_t>(stream), a.ev);
}

}  // namespace kvs
