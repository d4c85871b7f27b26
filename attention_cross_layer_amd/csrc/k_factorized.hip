// Factorized cross-layer cache: writes, and decode attention that reads the
// factorized entries directly.
//
// The cache follows DepthWeave-KV ("DepthWeave-KV: Smarter KV Cache
// Compression by Sharing Across Layers and Adapting Per Token", Core
// Mechanism and Framework Shift): a layer pair shares a channel basis and
// per-token coefficients; each layer adds a low-rank residual whose int8
// codes carry an fp16 per-token scale; each token has its own residual rank.
// Per KV head:
//   K_l[t] = c[t] B_pair + s_l[t] * sum_{j < r_t} d_l[t, j] U_l[j]   (V alike)
// with c [R=32] bf16, B [R x hd] bf16, d [Rmax=16] int8, s fp16, U [Rmax x hd].
//
// Decode.  The attention of one query row over these keys/values is
//   z_t = q . K_t = c_t . (B q) + s_t * sum_{j<r_t} d_{t,j} (U_j . q)
//   out = sum_t p_t V_t = (sum_t p_t c^V_t) B^V + (sum_t p_t s^V_t d^V_t) U^V,
// the same values the explicit rebuild gives (up to rounding order).  A
// workgroup contracts the bases with its G queries once (q~ = B^K q,
// u~ = U^K q), streams each page's coefficients, codes and scales once for
// all G query heads, and accumulates in the 48-wide coefficient space;
// B^V / U^V are applied once per output row.  Per page of 64 tokens the two
// contractions are small dense products, [64 x 48] x [48 x G] for the scores
// and [G x 64] x [64 x 48] for the values.  Both run on the 4x4x4 bf16 MFMA
// (16 independent 4x4 blocks per instruction: a wave's lanes are 16 token
// quads x 4 heads), which keeps the whole chain in registers:
//   scores   A = coefficients or codes (lane = token, 4 per block),
//            B = q~ as a bf16 high part plus the bf16 rounding of the rest
//            (two products into one accumulator, exact to about 2^-17),
//            D = lane (quad q, head p): tokens 4q..4q+3 of head p;
//   values   A = those probabilities, straight from the score registers,
//            B = value coefficients / codes (lane (quad q, column j):
//            tokens 4q..4q+3), D accumulated per quad; the 16 quads are
//            summed once at the end.
//
// Page layouts (64 tokens per page and KV head):
//   cK  [4][64][8] bf16      coefficients 8cc..8cc+7 of token t at (cc*64 + t)*8
//   cV  [4][64][2][4] bf16   coefficient i of token t (m = i/4, lane = 4*(t/4) + i%4)
//                            at ((m/2)*64 + lane)*8 + (m%2)*4 + t%4
//   dK, dV  [128][8] int8    rank-packed: token t owns ceil(r_t/8) 8-byte granules
//                            from granule o_t = sum_{u<t} ceil(r_u/8); its codes
//                            j >= r_t inside them are zero
//   sK, sV  [64] fp16
//   meta    [64] uint16 per physical page, shared by all layers and heads:
//           r_t | o_t << 8
// so a decode reads ceil(r_t/8)*8 code bytes per token (exactly r_t for
// ranks that are multiples of 8), not a fixed 16.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "common.h"
#include "internal.h"

namespace kvs {
namespace {

using dev::dot2_bf16;

constexpr int kR = 32;             // basis rank (coefficients per token)
constexpr int kRM = 16;            // residual codes per token at most
constexpr int kW = kR + kRM;
constexpr int kGranules = 128;     // 8-byte code granules per page blob
constexpr int kMaxSplitsF = 64;

typedef __attribute__((ext_vector_type(4))) short s4_t;
typedef __attribute__((ext_vector_type(4))) float f4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf2_t;

struct FactParams {
  const uint16_t* ck; const uint16_t* cv;
  const int8_t* dk; const int8_t* dv;
  const uint16_t* sk; const uint16_t* sv;
  const uint16_t* meta;
  const uint16_t* bk; const uint16_t* bv;   // basis of the pair's slot: [Hkv][R][hd]
  const uint16_t* uk; const uint16_t* uv;   // residual directions of the layer: [Hkv][RM][hd]
  const int32_t* page_table;
  int32_t pages_per_seq;
  int32_t n_phys_pages;
  int32_t n_kv_heads;
  int32_t n_q_heads;
  int64_t coef_off;     // elements to the slot's cK/cV pages
  int64_t resid_off;    // bytes to the layer's dK/dV pages
  int64_t scale_off;    // elements to the layer's sK/sV pages
  const uint16_t* q;
  const int32_t* seq_len;
  int32_t max_ctx;
  int32_t key_excl;     // 1: keys 0..seq_len-2 only (source above the layer)
  int32_t n_splits;
  float scale_log2;
  float* ws_c;          // [B][Hq][S][48]
  float* ws_m;          // [B][Hq][S]
  float* ws_l;          // [B][Hq][S]
  float* ws_a;          // [B][Hq][S]: sum_t p_t (z_t - m) (statistics only)
  float* stats;         // [B][Hq][2]: entropy (nats), peak probability; or null
  void* out;
  int32_t out_bf16;
};

__device__ __forceinline__ void split_range(int n_pages, int s, int S, int& pb, int& pe) {
  pb = (int)(((long long)s * n_pages) / S);
  pe = (int)(((long long)(s + 1) * n_pages) / S);
}

__device__ __forceinline__ float half_to_float(uint16_t h) {
  return __half2float(__ushort_as_half(h));
}

__device__ __forceinline__ void store_out(void* out, size_t idx, float v, int bf16) {
  if (bf16)
    reinterpret_cast<uint16_t*>(out)[idx] = (uint16_t)dev::f32_to_bf16_bits(v);
  else
    reinterpret_cast<float*>(out)[idx] = v;
}

__device__ __forceinline__ f4_t mfma4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f4_t c) {
  const u2_t a = {a0, a1}, b = {b0, b1};
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s4_t, a),
                                                __builtin_bit_cast(s4_t, b), c, 0, 0, 0);
}

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;

__device__ __forceinline__ f4_t mfma16(const uint4& a, const uint4& b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// four int8 codes (the bytes of w) -> four bf16 values (exact: |d| <= 128)
__device__ __forceinline__ void codes_to_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = pack_bf16((float)(int8_t)(w & 0xffu), (float)(int8_t)((w >> 8) & 0xffu));
  hi = pack_bf16((float)(int8_t)((w >> 16) & 0xffu), (float)(int8_t)(w >> 24));
}

// Byte transpose inside a quad of lanes: lane p of the quad holds bytes
// b[p][0..3]; returns (b[0][p], b[1][p], b[2][p], b[3][p]).  Two exchange
// steps (16-bit halves with lane p^2, then bytes with lane p^1), each a DPP
// quad permutation and a byte permute; sel1 / sel2 are the lane's selectors.
__device__ __forceinline__ uint32_t quad_transpose(uint32_t x, uint32_t sel1, uint32_t sel2) {
  const uint32_t z = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xf, 0xf, true);
  const uint32_t w = __builtin_amdgcn_perm(z, x, sel1);
  const uint32_t z2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)w, 0xB1, 0xf, 0xf, true);
  return __builtin_amdgcn_perm(z2, w, sel2);
}

// Max over the 16 quads of a wave for each lane position p (the lanes l with
// l % 4 == p), returned to every such lane.
__device__ __forceinline__ float quad_column_max(float x) {
  x = dev::fmax_ieee(x, dev::dpp<0x124>(x));   // row_ror:4
  x = dev::fmax_ieee(x, dev::dpp<0x128>(x));   // row_ror:8: every lane holds its row's max
  // across the two halves, then across row pairs (v_permlane32_swap /
  // v_permlane16_swap with both operands x: the two results hold the two
  // partners' values)
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = dev::fmax_ieee(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return dev::fmax_ieee(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum over the 4 quads of each 16-lane row for each lane position p: lane
// 16*row + p (p < 4) then holds the row's sum.
__device__ __forceinline__ float quad_row_sum(float x) {
  x += dev::dpp<0x124>(x);
  x += dev::dpp<0x128>(x);
  return x;
}

using dev::kOOB;
using dev::ld16;
using dev::ld8;
using dev::ld2;
using dev::kStream;
using dev::rsrc;

// One page as loaded: cK, codes and meta with lane = token; cV with lane =
// (quad, coefficient); the scales with lane = quad.
struct PageRegs {
  uint4 ck[4];
  uint4 cv[4];
  uint2 dk[2];
  uint2 dv[2];
  uint2 sk, sv;
};

// out[h][d] = (C[h] . B^V[:, d] + D[h] . U^V[:, d]) / l[h] for the G heads of
// one (sequence, KV head); coef holds [G][48] (C then D), den [G].
template <int HD, int G>
__device__ void project_out(const FactParams& a, int b, int kvh, const float* coef, const float* den,
                            int tid, int nthreads) {
  const uint16_t* bv = a.bv + (size_t)kvh * kR * HD;
  const uint16_t* uv = a.uv + (size_t)kvh * kRM * HD;
  const size_t hq0 = (size_t)b * a.n_q_heads + (size_t)kvh * G;
  for (int e = tid; e < G * HD; e += nthreads) {
    const int h = e / HD, d = e % HD;
    float acc = 0.f;
#pragma unroll 8
    for (int i = 0; i < kR; ++i)
      acc = fmaf(coef[h * kW + i], __uint_as_float((uint32_t)bv[i * HD + d] << 16), acc);
#pragma unroll 8
    for (int j = 0; j < kRM; ++j)
      acc = fmaf(coef[h * kW + kR + j], __uint_as_float((uint32_t)uv[j * HD + d] << 16), acc);
    const float l = den[h];
    store_out(a.out, (hq0 + h) * HD + d, l > 0.f ? acc / l : 0.f, a.out_bf16);
  }
}

// grid (S, Hkv, B), 4 waves; wave w walks pages pb+w, pb+w+4, ... of its
// partition, with the next page's loads in flight while it computes one.
// entropy ln l - ln2 A / l (nats) and peak probability 1 / l of one query row
// from its softmax sum l and A = sum_t p_t (z_t - m); (0, 0) without keys
__device__ __forceinline__ void write_stats(float* stats, size_t row, float l, float A) {
  const bool any = l > 0.f;
  stats[2 * row] = any ? logf(l) - 0.69314718055994531f * A / l : 0.f;
  stats[2 * row + 1] = any ? 1.f / l : 0.f;
}

// STATS: also track A = sum_t p_t (z_t - m) beside the sum l = sum_t p_t
// (z in log2 units), so that the attention's entropy is ln l - ln2 A / l and
// its peak probability 1 / l (the largest p_t is 2^0 = 1).
template <int HD, int G, bool STATS>
__global__ __launch_bounds__(256) void fact_decode_kernel(FactParams a) {
  constexpr int NB = (G + 3) / 4;              // blocks of 4 query heads
  __shared__ float qt[NB * 4][kW];             // (B^K q, U^K q) * log2(e)/sqrt(hd)
  __shared__ float part[4][4][NB * 4][kW];     // [wave][16-lane row][head][coefficient]
  __shared__ float part_l[4][4][NB * 4];
  __shared__ float part_a[STATS ? 4 : 1][4][NB * 4];
  __shared__ float wave_m[4][NB * 4];
  __shared__ float fin_c[G * kW];
  __shared__ float fin_l[G];
  __shared__ float fin_a[G];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int quad = lane >> 2, pos = lane & 3;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int S = a.n_splits;

  const int n_keys = min(max(a.seq_len[b] - a.key_excl, 0), a.max_ctx);
  const int n_pages = (n_keys + kPage - 1) / kPage;
  int pb, pe;
  split_range(n_pages, split, S, pb, pe);
  const int32_t* pt = a.page_table + (size_t)b * a.pages_per_seq;
  const uint16_t* ck_base = a.ck + a.coef_off;
  const uint16_t* cv_base = a.cv + a.coef_off;
  const int8_t* dk_base = a.dk + a.resid_off;
  const int8_t* dv_base = a.dv + a.resid_off;
  const uint16_t* sk_base = a.sk + a.scale_off;
  const uint16_t* sv_base = a.sv + a.scale_off;

  // Buffer resources over this call's sub-pools: every page load below is
  // issued unconditionally, an absent page or granule with an offset past the
  // resource's end (the hardware returns zeros and moves no data), so the
  // loop holds a fixed number of loads and the next page stays in flight.
  const uint32_t P = (uint32_t)a.n_phys_pages, H = (uint32_t)a.n_kv_heads;
  const auto r_ck = rsrc(ck_base, P * H * (kPage * kR * 2));
  const auto r_cv = rsrc(cv_base, P * H * (kPage * kR * 2));
  const auto r_dk = rsrc(dk_base, P * H * (kGranules * 8));
  const auto r_dv = rsrc(dv_base, P * H * (kGranules * 8));
  const auto r_sk = rsrc(sk_base, P * H * (kPage * 2));
  const auto r_sv = rsrc(sv_base, P * H * (kPage * 2));
  const auto r_meta = rsrc(a.meta, P * (kPage * 2));
  const int pt_last = max(pe - 1, 0);

  // physical page of logical page pg, or -1 (past the partition, or a corrupt
  // entry, which is never read)
  auto phys_of = [&](int pg) {
    const int ph = pt[min(pg, pt_last)];
    return (pg < pe && (unsigned)ph < P) ? ph : -1;
  };
  // rank | granule offset << 8 of this lane's token; 0 when there is none
  auto load_meta = [&](int pg, int ph) -> uint32_t {
    const bool on = ph >= 0 && lane < n_keys - pg * kPage;
    return ld2<kStream>(r_meta, on ? (uint32_t)(ph * kPage + lane) * 2 : kOOB);
  };
  auto load_coefs = [&](int ph, PageRegs& r) {
    const uint32_t page_kv = (uint32_t)ph * H + kvh;
    const uint32_t cb = ph >= 0 ? page_kv * (kPage * kR * 2) : kOOB;
    const uint32_t sb = ph >= 0 ? page_kv * (kPage * 2) : kOOB;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.ck[i] = ld16<kStream>(r_ck, cb + (i * 64 + lane) * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.cv[i] = ld16<kStream>(r_cv, cb + (i * 64 + lane) * 16);
    r.sk = ld8<kStream>(r_sk, sb + quad * 8);
    r.sv = ld8<kStream>(r_sv, sb + quad * 8);
  };
  auto load_codes = [&](int ph, uint32_t meta, PageRegs& r) {
    const int rank = min((int)(meta & 0xffu), kRM);
    const int ng = (rank + 7) >> 3;                              // granules of this token
    const uint32_t g0 = min(meta >> 8, (uint32_t)(kGranules - 2));  // stays inside the blob
    // meta != 0 only for pages with ph >= 0
    const uint32_t blob = ((uint32_t)ph * H + kvh) * (kGranules * 8) + g0 * 8;
    const uint32_t o0 = ng >= 1 ? blob : kOOB, o1 = ng == 2 ? blob + 8 : kOOB;
    r.dk[0] = ld8<kStream>(r_dk, o0);
    r.dk[1] = ld8<kStream>(r_dk, o1);
    r.dv[0] = ld8<kStream>(r_dv, o0);
    r.dv[1] = ld8<kStream>(r_dv, o1);
  };

  // ---- absorbed query: qt[h][i] = (row i of [B^K; U^K]) . q_h for the 48
  // rows i and the G <= 8 heads h, on v_mfma_f32_16x16x32_bf16: waves 0..2
  // take one 16-row block each (A = 16 rows x 32 dims, B = 32 dims x 16
  // heads, the columns past G zero), HD/32 steps.  Products of bf16 values
  // are exact and summed in fp32.  Each lane requests its two 16-byte
  // operands per step before the first page, so the contraction waits only
  // for them; a workgroup reads the 12 KB of bases and its queries once.
  constexpr int KSQ = HD / 32;
  uint4 qa[KSQ], qb[KSQ];
  const int qh = lane & 15;              // head column of this lane
  const int qk = 8 * (lane >> 4);        // its first dim within each 32-dim step
  if (wave < 3) {
    const int r = 16 * wave + qh;        // row of [B^K; U^K]
    const uint16_t* row = r < kR ? a.bk + ((size_t)kvh * kR + r) * HD
                                 : a.uk + ((size_t)kvh * kRM + (r - kR)) * HD;
    const uint16_t* qr = a.q + ((size_t)b * a.n_q_heads + (size_t)kvh * G + min(qh, G - 1)) * HD;
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) {
      qa[ks] = *reinterpret_cast<const uint4*>(row + 32 * ks + qk);
      const uint4 y = *reinterpret_cast<const uint4*>(qr + 32 * ks + qk);
      qb[ks] = qh < G ? y : make_uint4(0, 0, 0, 0);
    }
  }

  // ---- the first page's requests
  const int pg0 = pb + wave;
  PageRegs bufA, bufB;
  const int ph0 = phys_of(pg0);
  const uint32_t meta0 = load_meta(pg0, ph0);
  int ph_b = phys_of(pg0 + 4);
  uint32_t meta_b = load_meta(pg0 + 4, ph_b);
  load_coefs(ph0, bufA);

  if (wave < 3) {
    f4_t d = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) d = mfma16(qa[ks], qb[ks], d);
    // lane: head qh, rows 16 * wave + 4 * (lane / 16) + j
    if (qh < NB * 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) qt[qh][16 * wave + 4 * (lane >> 4) + j] = d[j] * a.scale_log2;
    }
  }
  load_codes(ph0, meta0, bufA);
  __syncthreads();

  // score B operands: lane (quad, pos) supplies head 4*hb + pos, entries
  // 4m..4m+3 of q~ (m < 8) or u~ (m >= 8)
  uint32_t bq_hi[NB][12][2], bq_lo[NB][12][2];
#pragma unroll
  for (int hb = 0; hb < NB; ++hb)
#pragma unroll
    for (int m = 0; m < 12; ++m)
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        const float x0 = qt[hb * 4 + pos][4 * m + 2 * e2];
        const float x1 = qt[hb * 4 + pos][4 * m + 2 * e2 + 1];
        const uint32_t hi = pack_bf16(x0, x1);
        bq_hi[hb][m][e2] = hi;
        bq_lo[hb][m][e2] = pack_bf16(x0 - dev::bf16_lo(hi), x1 - dev::bf16_hi(hi));
      }

  // byte-transpose selectors of this lane
  const uint32_t sel1 = (pos & 2) ? 0x03020706u : 0x05040100u;
  const uint32_t sel2 = (pos & 1) ? 0x03070105u : 0x06020400u;

  float m_run[NB], l_run[NB], a_run[NB];
  f4_t acc[NB][12];
#pragma unroll
  for (int hb = 0; hb < NB; ++hb) {
    m_run[hb] = -INFINITY;
    l_run[hb] = 0.f;
    a_run[hb] = 0.f;
#pragma unroll
    for (int m = 0; m < 12; ++m) acc[hb][m] = f4_t{0.f, 0.f, 0.f, 0.f};
  }

  // ph < 0 here: the page's table entry is out of range; its keys get no
  // weight (its loads returned zeros)
  auto compute = [&](int pg, int ph, const PageRegs& r) {
    const int nvalid = ph >= 0 ? n_keys - pg * kPage : 0;
    const bool tail = nvalid < kPage;
    // score A operands of the codes (token = lane)
    uint32_t ad[4][2];
    {
      const uint32_t w4[4] = {r.dk[0].x, r.dk[0].y, r.dk[1].x, r.dk[1].y};
#pragma unroll
      for (int m = 0; m < 4; ++m) codes_to_bf16(w4[m], ad[m][0], ad[m][1]);
    }
    const uint32_t* cw = &r.ck[0].x;    // coefficient pairs 0..15 of token `lane`
    // value B operands of the codes: the quad's 4 tokens of code 4m + pos
    uint32_t bd[4][2];
    {
      const uint32_t w4[4] = {r.dv[0].x, r.dv[0].y, r.dv[1].x, r.dv[1].y};
#pragma unroll
      for (int m = 0; m < 4; ++m) codes_to_bf16(quad_transpose(w4[m], sel1, sel2), bd[m][0], bd[m][1]);
    }
    uint32_t bc[8][2];
    {
      const uint32_t* vw = &r.cv[0].x;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        bc[m][0] = vw[2 * m];
        bc[m][1] = vw[2 * m + 1];
      }
    }
    // which of the quad's tokens lie before the sequence end
    bool ok[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) ok[e] = !tail || quad * 4 + e < nvalid;
    const uint32_t mk0 = (ok[0] ? 0x0000ffffu : 0u) | (ok[1] ? 0xffff0000u : 0u);
    const uint32_t mk1 = (ok[2] ? 0x0000ffffu : 0u) | (ok[3] ? 0xffff0000u : 0u);
    if (tail) {
      // unwritten pool memory may hold NaN patterns: zero those tokens' values
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        bc[m][0] &= mk0;
        bc[m][1] &= mk1;
      }
    }
    float skf[4], svf[4];
    skf[0] = half_to_float((uint16_t)(r.sk.x & 0xffffu));
    skf[1] = half_to_float((uint16_t)(r.sk.x >> 16));
    skf[2] = half_to_float((uint16_t)(r.sk.y & 0xffffu));
    skf[3] = half_to_float((uint16_t)(r.sk.y >> 16));
    svf[0] = half_to_float((uint16_t)(r.sv.x & 0xffffu));
    svf[1] = half_to_float((uint16_t)(r.sv.x >> 16));
    svf[2] = half_to_float((uint16_t)(r.sv.y & 0xffffu));
    svf[3] = half_to_float((uint16_t)(r.sv.y >> 16));

#pragma unroll
    for (int hb = 0; hb < NB; ++hb) {
      // ---- scores: rows = the quads' tokens, columns = heads
      // six independent accumulator chains of four products each, so that
      // consecutive products never wait on each other's result
      f4_t zc[4], zd[2];
#pragma unroll
      for (int c = 0; c < 4; ++c) zc[c] = f4_t{0.f, 0.f, 0.f, 0.f};
      zd[0] = zd[1] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int m0 = 2 * k, m1 = 2 * k + 1;
        zc[0] = mfma4(cw[2 * m0], cw[2 * m0 + 1], bq_hi[hb][m0][0], bq_hi[hb][m0][1], zc[0]);
        zc[1] = mfma4(cw[2 * m1], cw[2 * m1 + 1], bq_hi[hb][m1][0], bq_hi[hb][m1][1], zc[1]);
        zc[2] = mfma4(cw[2 * m0], cw[2 * m0 + 1], bq_lo[hb][m0][0], bq_lo[hb][m0][1], zc[2]);
        zc[3] = mfma4(cw[2 * m1], cw[2 * m1 + 1], bq_lo[hb][m1][0], bq_lo[hb][m1][1], zc[3]);
        zd[0] = mfma4(ad[k][0], ad[k][1], bq_hi[hb][8 + k][0], bq_hi[hb][8 + k][1], zd[0]);
        zd[1] = mfma4(ad[k][0], ad[k][1], bq_lo[hb][8 + k][0], bq_lo[hb][8 + k][1], zd[1]);
      }
      const bool head_ok = hb * 4 + pos < G;
      float z[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = fmaf(skf[e], zd[0][e] + zd[1][e], (zc[0][e] + zc[1][e]) + (zc[2][e] + zc[3][e]));
        z[e] = (ok[e] && head_ok) ? v : -INFINITY;
      }
      // ---- online softmax with one running max per head (uniform over the wave)
      const float mt = quad_column_max(dev::fmax_ieee(dev::fmax3_ieee(z[0], z[1], z[2]), z[3]));
      const bool bump = mt > m_run[hb];
      const float mn = bump ? mt : m_run[hb];
      const float mu = mn == -INFINITY ? 0.f : mn;
      // 1 exactly while the max holds (also for heads past G, whose max stays -inf)
      const float alpha = bump ? dev::fast_exp2(m_run[hb] - mu) : 1.f;
      const float m_old = m_run[hb];
      m_run[hb] = mn;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
        // accumulator entry e of every lane belongs to head e of the block:
        // broadcast head e's factor from the quad
        const int ai = __float_as_int(alpha);
        const float a0 = __int_as_float(__builtin_amdgcn_mov_dpp(ai, 0x00, 0xf, 0xf, true));
        const float a1 = __int_as_float(__builtin_amdgcn_mov_dpp(ai, 0x55, 0xf, 0xf, true));
        const float a2 = __int_as_float(__builtin_amdgcn_mov_dpp(ai, 0xAA, 0xf, 0xf, true));
        const float a3 = __int_as_float(__builtin_amdgcn_mov_dpp(ai, 0xFF, 0xf, 0xf, true));
#pragma unroll
        for (int m = 0; m < 12; ++m) {
          acc[hb][m][0] *= a0;
          acc[hb][m][1] *= a1;
          acc[hb][m][2] *= a2;
          acc[hb][m][3] *= a3;
        }
        // A refers to the new maximum: alpha (A + (m_old - m_new) l)
        if (STATS) a_run[hb] = m_old == -INFINITY ? 0.f : alpha * fmaf(m_old - mu, l_run[hb], a_run[hb]);
        l_run[hb] *= alpha;
      }
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = dev::fast_exp2(z[e] - mu);
      const uint32_t ap0 = pack_bf16(p[0], p[1]), ap1 = pack_bf16(p[2], p[3]);
      // the bf16 probabilities enter both the numerator and the sum
      const float q0 = dev::bf16_lo(ap0), q1 = dev::bf16_hi(ap0);
      const float q2 = dev::bf16_lo(ap1), q3 = dev::bf16_hi(ap1);
      l_run[hb] += (q0 + q1) + (q2 + q3);
      if (STATS) {
        // masked tokens (z = -inf, p = 0) add nothing
        float dz[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) dz[e] = z[e] == -INFINITY ? 0.f : z[e] - mu;
        a_run[hb] = fmaf(q0, dz[0], fmaf(q1, dz[1], fmaf(q2, dz[2], fmaf(q3, dz[3], a_run[hb]))));
      }
      // p * s^V; masked tokens (p = 0) must not pick up a NaN scale
      const uint32_t as0 = pack_bf16(q0 * svf[0], q1 * svf[1]) & mk0;
      const uint32_t as1 = pack_bf16(q2 * svf[2], q3 * svf[3]) & mk1;
      // ---- values: rows = heads, columns = coefficients, k = the quad's tokens
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[hb][m] = mfma4(ap0, ap1, bc[m][0], bc[m][1], acc[hb][m]);
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[hb][8 + m] = mfma4(as0, as1, bd[m][0], bd[m][1], acc[hb][8 + m]);
    }
  };

  // ---- main loop over this wave's pages pg0, pg0+4, ...: two page buffers,
  // the next page's loads issued before the current page is computed, the
  // page after next's meta one step earlier still
  int ph_in_a = ph0;
  for (int pg = pg0; pg < pe; pg += 8) {
    const int ph_c = phys_of(pg + 8);
    const uint32_t meta_c = load_meta(pg + 8, ph_c);
    const int ph_in_b = ph_b;
    load_coefs(ph_b, bufB);
    load_codes(ph_b, meta_b, bufB);
    compute(pg, ph_in_a, bufA);
    if (pg + 4 >= pe) break;
    ph_b = phys_of(pg + 12);
    meta_b = load_meta(pg + 12, ph_b);
    ph_in_a = ph_c;
    load_coefs(ph_c, bufA);
    load_codes(ph_c, meta_c, bufA);
    compute(pg + 4, ph_in_b, bufB);
  }

  // ---- this wave's per-head (coefficient sums, m, l) to LDS
  const int row = lane >> 4;
  const bool writer = (lane & 15) < 4;          // lanes 16*row + pos
#pragma unroll
  for (int hb = 0; hb < NB; ++hb) {
    const float l = quad_row_sum(l_run[hb]);
#pragma unroll
    for (int m = 0; m < 12; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = quad_row_sum(acc[hb][m][e]);
        if (writer) part[wave][row][hb * 4 + e][4 * m + pos] = x;
      }
    if (writer) part_l[wave][row][hb * 4 + pos] = l;
    if (STATS) {
      const float aa = quad_row_sum(a_run[hb]);
      if (writer) part_a[wave][row][hb * 4 + pos] = aa;
    }
    if (lane < 4) wave_m[wave][hb * 4 + lane] = m_run[hb];
  }
  __syncthreads();

  // ---- merge the 4 waves; write the output (S == 1) or the partition
  const size_t hq0 = (size_t)b * a.n_q_heads + (size_t)kvh * G;
  for (int e = tid; e < G * kW; e += 256) {
    const int h = e / kW, i = e % kW;
    float M = wave_m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, wave_m[w][h]);
    float c = 0.f, l = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = dev::fast_exp2(wave_m[w][h] - M);
        const float cw = (part[w][0][h][i] + part[w][1][h][i]) + (part[w][2][h][i] + part[w][3][h][i]);
        const float lw = (part_l[w][0][h] + part_l[w][1][h]) + (part_l[w][2][h] + part_l[w][3][h]);
        c = fmaf(f, cw, c);
        l = fmaf(f, lw, l);
        if (STATS && i == 0 && wave_m[w][h] != -INFINITY) {
          const float aw = (part_a[w][0][h] + part_a[w][1][h]) + (part_a[w][2][h] + part_a[w][3][h]);
          A = fmaf(f, fmaf(wave_m[w][h] - M, lw, aw), A);
        }
      }
    }
    if (S == 1) {
      fin_c[e] = c;
      if (i == 0) {
        fin_l[h] = l;
        fin_a[h] = A;
      }
    } else {
      const size_t rw = (hq0 + h) * S + split;
      a.ws_c[rw * kW + i] = c;
      if (i == 0) {
        a.ws_m[rw] = M;
        a.ws_l[rw] = l;
        if (STATS) a.ws_a[rw] = A;
      }
    }
  }
  if (S != 1) return;
  __syncthreads();
  if (STATS && tid < G) write_stats(a.stats, hq0 + tid, fin_l[tid], fin_a[tid]);
  project_out<HD, G>(a, b, kvh, fin_c, fin_l, tid, 256);
}

// Merge of S partitions in coefficient space, then the basis projection.
// Every partition writes its row (an empty one as c = 0, m = -inf, l = 0), so
// a thread loads its S (m, l, c) triples 16 at a time with no dependence
// between them and folds each batch into a running (M, c, l); the basis
// column each thread projects with (its d is fixed: 256 is a multiple of HD)
// is loaded up front.  Partition order is fixed: deterministic.
template <int HD, int G, bool STATS>
__global__ __launch_bounds__(256) void fact_merge_kernel(FactParams a) {
  static_assert(256 % HD == 0, "a thread keeps one output column");
  __shared__ float den[G];
  __shared__ float num_a[G];
  __shared__ float coef[G * kW];
  const int tid = threadIdx.x;
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int S = a.n_splits;
  const size_t hq0 = (size_t)b * a.n_q_heads + (size_t)kvh * G;
  const int d = tid % HD;
  float col[kW];   // column d of B^V (rows 0..R-1) then U^V (rows R..R+RM-1)
  {
    const uint16_t* bv = a.bv + (size_t)kvh * kR * HD + d;
    const uint16_t* uv = a.uv + (size_t)kvh * kRM * HD + d;
#pragma unroll
    for (int i = 0; i < kR; ++i) col[i] = __uint_as_float((uint32_t)bv[i * HD] << 16);
#pragma unroll
    for (int j = 0; j < kRM; ++j) col[kR + j] = __uint_as_float((uint32_t)uv[j * HD] << 16);
  }
  for (int e = tid; e < G * kW; e += 256) {
    const int h = e / kW, i = e % kW;
    const float* mrow = a.ws_m + (hq0 + h) * S;
    const float* lrow = a.ws_l + (hq0 + h) * S;
    const float* crow = a.ws_c + (hq0 + h) * S * kW + i;
    const float* arow = a.ws_a + (hq0 + h) * S;
    const bool with_a = STATS && i == 0;
    float M = -INFINITY, c = 0.f, l = 0.f, A = 0.f;
    for (int s0 = 0; s0 < S; s0 += 16) {
      float mv[16], lv[16], cv[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int s = min(s0 + k, S - 1);
        mv[k] = s0 + k < S ? mrow[s] : -INFINITY;
        lv[k] = lrow[s];
        cv[k] = crow[(size_t)s * kW];
      }
      float Mn = M;
#pragma unroll
      for (int k = 0; k < 16; ++k) Mn = fmaxf(Mn, mv[k]);
      if (Mn != -INFINITY) {
        const float r = dev::fast_exp2(M - Mn);   // 0 while M is -inf
        if (with_a) A = M == -INFINITY ? 0.f : r * fmaf(M - Mn, l, A);
        c *= r;
        l *= r;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float f = dev::fast_exp2(mv[k] - Mn);   // 0 for empty or absent partitions
          c = fmaf(f, cv[k], c);
          l = fmaf(f, lv[k], l);
          if (with_a && mv[k] != -INFINITY) A = fmaf(f, fmaf(mv[k] - Mn, lv[k], arow[s0 + k]), A);
        }
        M = Mn;
      }
    }
    coef[e] = c;
    if (i == 0) den[h] = l;
    if (with_a) num_a[h] = A;
  }
  __syncthreads();
  if (STATS && tid < G) write_stats(a.stats, hq0 + tid, den[tid], num_a[tid]);
  for (int h = tid / HD; h < G; h += 256 / HD) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < kW; ++i) acc = fmaf(coef[h * kW + i], col[i], acc);
    const float l = den[h];
    store_out(a.out, (hq0 + h) * HD + d, l > 0.f ? acc / l : 0.f, a.out_bf16);
  }
}

template <int HD, int G, bool STATS>
int run_fact_t(const FactParams& p, int B, hipStream_t st, const KernelEvents& ev) {
  launch_main(ev, fact_decode_kernel<HD, G, STATS>, dim3(p.n_splits, p.n_kv_heads, B), dim3(256), st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_splits == 1) return (int)e;
  hipLaunchKernelGGL((fact_merge_kernel<HD, G, STATS>), dim3(p.n_kv_heads, B), dim3(256), 0, st, p);
  return (int)hipGetLastError();
}

template <int HD, int G>
int run_fact(const FactParams& p, int B, hipStream_t st, const KernelEvents& ev) {
  return p.stats ? run_fact_t<HD, G, true>(p, B, st, ev) : run_fact_t<HD, G, false>(p, B, st, ev);
}

typedef int (*FactFn)(const FactParams&, int, hipStream_t, const KernelEvents&);

FactFn pick(int hd, int G) {
  if (hd == 64) {
    switch (G) {
      case 1: return run_fact<64, 1>;
      case 2: return run_fact<64, 2>;
      case 4: return run_fact<64, 4>;
      case 8: return run_fact<64, 8>;
    }
  } else if (hd == 128) {
    switch (G) {
      case 1: return run_fact<128, 1>;
      case 2: return run_fact<128, 2>;
      case 4: return run_fact<128, 4>;
      case 8: return run_fact<128, 8>;
    }
  }
  return nullptr;
}

// ---------------------------------------------------------------- writes

// One wave per (page the append touches, KV head, sequence); lane t is
// token slot t of the page.  A token's granule offset is the exclusive
// prefix sum of ceil(r/8) over the page's earlier slots, taken across the
// wave: ranks of tokens this call writes come from `rank`, earlier ones from
// the page's meta entries.
__global__ __launch_bounds__(64) void fact_append_kernel(FactAppendLaunch a) {
  const int t = threadIdx.x;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int sp = a.start_pos[b];
  const int end = min(sp + a.n, a.max_ctx);            // positions [max(sp, 0), end) are written
  const int lp = max(sp, 0) / kPage + (int)blockIdx.x;  // logical page of this wave
  if (lp * kPage >= end) return;                        // uniform
  const int page = a.page_table[(size_t)b * a.pages_per_seq + lp];
  if (page < 0 || page >= a.n_phys_pages) return;       // uniform
  const int pos = lp * kPage + t;
  const bool fresh = pos >= sp && pos < end;
  const int i = pos - sp;
  const uint8_t* rk = a.rank + (size_t)b * a.n;
  uint16_t* meta = static_cast<uint16_t*>(a.rank_pool) + (size_t)page * kPage;
  const int r = fresh ? min((int)rk[i], kRM) : (pos < sp ? min((int)(meta[t] & 0xffu), kRM) : 0);
  const int ng = (r + 7) >> 3;
  int incl = ng;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (t >= off) incl += v;
  }
  const int g0 = incl - ng;
  if (!fresh) return;
  const size_t page_kv = (size_t)page * a.n_kv_heads + kvh;
  const size_t src_row = ((size_t)b * a.n + i) * a.n_kv_heads + kvh;
  if (a.coef_slot >= 0) {
    const size_t base = ((size_t)a.coef_slot * a.n_phys_pages * a.n_kv_heads + page_kv) * kPage * kR;
    const uint16_t* ck = static_cast<const uint16_t*>(a.ck) + src_row * kR;
    const uint16_t* cv = static_cast<const uint16_t*>(a.cv) + src_row * kR;
    uint16_t* dk = static_cast<uint16_t*>(a.ck_pool) + base;
    uint16_t* dv = static_cast<uint16_t*>(a.cv_pool) + base;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
      *reinterpret_cast<uint4*>(dk + (cc * 64 + t) * 8) = *reinterpret_cast<const uint4*>(ck + cc * 8);
#pragma unroll 8
    for (int e = 0; e < kR; ++e) {
      const int m = e >> 2, ln = ((t >> 2) << 2) | (e & 3);
      dv[((m >> 1) * 64 + ln) * 8 + (m & 1) * 4 + (t & 3)] = cv[e];
    }
  }
  {
    const size_t lbase = (size_t)a.layer * a.n_phys_pages * a.n_kv_heads + page_kv;
    // codes j >= r are stored as zero
    uint32_t keep[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int nb = min(max(r - 4 * w, 0), 4);
      keep[w] = nb == 4 ? 0xffffffffu : ((1u << (8 * nb)) - 1u);
    }
    const uint4 ck = *reinterpret_cast<const uint4*>(a.dk + src_row * kRM);
    const uint4 cv = *reinterpret_cast<const uint4*>(a.dv + src_row * kRM);
    int8_t* dk = static_cast<int8_t*>(a.dk_pool) + lbase * (kGranules * 8) + (size_t)g0 * 8;
    int8_t* dv = static_cast<int8_t*>(a.dv_pool) + lbase * (kGranules * 8) + (size_t)g0 * 8;
    if (ng >= 1) {
      *reinterpret_cast<uint2*>(dk) = make_uint2(ck.x & keep[0], ck.y & keep[1]);
      *reinterpret_cast<uint2*>(dv) = make_uint2(cv.x & keep[0], cv.y & keep[1]);
    }
    if (ng == 2) {
      *reinterpret_cast<uint2*>(dk + 8) = make_uint2(ck.z & keep[2], ck.w & keep[3]);
      *reinterpret_cast<uint2*>(dv + 8) = make_uint2(cv.z & keep[2], cv.w & keep[3]);
    }
    static_cast<uint16_t*>(a.sk_pool)[lbase * kPage + t] = static_cast<const uint16_t*>(a.sk)[src_row];
    static_cast<uint16_t*>(a.sv_pool)[lbase * kPage + t] = static_cast<const uint16_t*>(a.sv)[src_row];
  }
  if (kvh == 0) meta[t] = (uint16_t)(r | (g0 << 8));
}

}  // namespace

bool fact_shape_supported(int32_t head_dim, int32_t group, int32_t basis_rank,
                          int32_t resid_rank_max) {
  return basis_rank == kR && resid_rank_max == kRM && pick(head_dim, group) != nullptr;
}

int max_fact_splits() { return kMaxSplitsF; }

int launch_fact_decode(const FactDecodeLaunch& a, void* stream) {
  FactFn fn = pick(a.head_dim, a.n_q_heads / a.n_kv_heads);
  if (!fn || a.n_splits < 1 || a.n_splits > kMaxSplitsF) return (int)hipErrorInvalidValue;
  FactParams p;
  p.ck = static_cast<const uint16_t*>(a.ck_pool);
  p.cv = static_cast<const uint16_t*>(a.cv_pool);
  p.dk = static_cast<const int8_t*>(a.dk_pool);
  p.dv = static_cast<const int8_t*>(a.dv_pool);
  p.sk = static_cast<const uint16_t*>(a.sk_pool);
  p.sv = static_cast<const uint16_t*>(a.sv_pool);
  p.meta = static_cast<const uint16_t*>(a.rank_pool);
  const size_t Hkv = a.n_kv_heads;
  p.bk = static_cast<const uint16_t*>(a.basis_k) + (size_t)a.coef_slot * Hkv * kR * a.head_dim;
  p.bv = static_cast<const uint16_t*>(a.basis_v) + (size_t)a.coef_slot * Hkv * kR * a.head_dim;
  p.uk = static_cast<const uint16_t*>(a.ubasis_k) + (size_t)a.layer * Hkv * kRM * a.head_dim;
  p.uv = static_cast<const uint16_t*>(a.ubasis_v) + (size_t)a.layer * Hkv * kRM * a.head_dim;
  p.page_table = a.page_table;
  p.pages_per_seq = a.pages_per_seq;
  p.n_phys_pages = a.n_phys_pages;
  p.n_kv_heads = a.n_kv_heads;
  p.n_q_heads = a.n_q_heads;
  p.coef_off = (int64_t)a.coef_slot * a.n_phys_pages * a.n_kv_heads * kPage * kR;
  p.resid_off = (int64_t)a.layer * a.n_phys_pages * a.n_kv_heads * kGranules * 8;
  p.scale_off = (int64_t)a.layer * a.n_phys_pages * a.n_kv_heads * kPage;
  p.q = static_cast<const uint16_t*>(a.q);
  p.seq_len = a.seq_len;
  p.max_ctx = a.max_ctx;
  p.key_excl = a.key_excl;
  p.n_splits = a.n_splits;
  p.scale_log2 = a.scale_log2;
  const size_t rows = (size_t)a.batch * a.n_q_heads * a.n_splits;
  p.ws_c = a.ws;
  p.ws_m = a.ws + rows * kW;
  p.ws_l = p.ws_m + rows;
  p.ws_a = p.ws_l + rows;
  p.stats = a.stats;
  p.out = a.out;
  p.out_bf16 = a.out_dtype == KVS_BF16;
  return fn(p, a.batch, static_cast<hipStream_t>(stream), a.ev);
}

int launch_fact_append(const FactAppendLaunch& a, void* stream) {
  if (a.batch == 0 || a.n == 0) return 0;
  // pages a chunk of n positions can touch: one more than it fills when it
  // starts mid-page
  const unsigned pages = (unsigned)((a.n + kPage - 1) / kPage + 1);
  hipLaunchKernelGGL(fact_append_kernel, dim3(pages, a.n_kv_heads, a.batch), dim3(64), 0,
                     static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

}  // namespace kvs
