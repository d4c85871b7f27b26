// Split-K decode attention over a shared (paged, source-only) K/V cache, and
// the merge of the split-K partitions.
//
// One decode query per (sequence, q head) attends over keys 0..seq_len-1 of
// the layer's source slot(s): the CLA page ("Reducing Transformer Key-Value
// Cache Size with Cross-Layer Attention", Methodology) has reusing layers read
// the source layer's cached K/V; DepthGraft ("DepthGraft: Structural
// Regularization through Hierarchical Cross-Layer KV Reconstruction",
// Abstract) rebuilds a deep layer's K/V from two sources, here
// K~ = w0 K_s0 + w1 K_s1 (V alike).  Scores are linear in K~ and the output is
// linear in V~, so the kernel mixes scores and partial outputs instead of
// forming K~/V~: every product stays an exact bf16 x bf16 product.
//
// Work decomposition (gfx950, wave64):
//   grid (S, Hkv, B), 256 threads = 4 waves.  Workgroup s owns split-K
//   partition s of one (sequence, KV head): an even share of its 64-key
//   pages; wave w takes every 4th page of it.  All G query heads of the KV
//   head are served by the same pass, so each cached tile is read from HBM
//   once per (sequence, KV head), i.e. once for the whole query group.
//   Per page, per wave:
//     QK   eight lanes share a key: lane 8*k8 + w holds, in registers for
//          the whole launch, the query chunks 8*cc + w (E elements = 16
//          bytes each) of all G heads.  Pass j (0..7) scores keys 8j + k8:
//          the K page layout puts each (j, cc) slice of 64 lanes x 16 bytes
//          in one contiguous 1 KiB load; partial dot products
//          (v_dot2c_f32_bf16: bf16 x bf16 products, fp32 accumulation) are
//          completed by two quad_perm DPP adds and one ds_swizzle (xor 4).
//          Lane w then keeps the scores of pass w, i.e. key 8*w + k8.
//     softmax  per-head wave max over DPP, online rescaling; probabilities
//          are rounded to bf16 for the PV products and the running sum uses
//          the same rounded values.
//     PV   the V page is stored as token pairs [32][hd][2], so one 16-byte
//          load holds 4 dims x 2 keys; lane l owns 4 dims and every NPH-th
//          pair, each dword feeding v_dot2c_f32_bf16 with the pair's two
//          probabilities (read from LDS).
//   A page's K and V are requested together; the scores wait only for K.
//   Loads of other pages overlap through the other waves on the CU (a
//   register double buffer of whole pages measured slower: it spills).
//   Merge: the 4 waves' (O, m, l) meet in LDS.  With S = 1 the workgroup
//   writes the normalised output.  Otherwise it writes its partition to the
//   workspace and a small merge kernel on the same stream combines the S
//   partitions in fixed order, so results are deterministic for a fixed S.
//   (Merging inside the decode launch would need an agent-scope release per
//   workgroup, i.e. an L2 write-back per workgroup; that measured several
//   times slower than the second launch.)
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "common.h"
#include "internal.h"

namespace kvs {
namespace {

using dev::dot2_bf16;

constexpr int kMaxFusedSplits = 64;

struct DecodeParams {
  const char* k_pool;
  const char* v_pool;
  const int32_t* page_table;
  int32_t pages_per_seq;
  int32_t n_phys_pages;
  int32_t n_kv_heads;
  int32_t n_q_heads;
  int64_t slot_stride;   // elements
  int32_t slot0, slot1;
  float w0, w1;
  const char* q;
  const int32_t* seq_len;
  int32_t max_ctx;
  int32_t key_excl;      // 1: keys 0..seq_len-2 only (source above the layer)
  int32_t n_splits;
  float scale_log2;
  float* ws_o;           // [B][Hq][S][HD]
  float* ws_m;           // [B][Hq][S]
  float* ws_l;           // [B][Hq][S]
  void* out;             // [B][Hq][HD]
  int out_bf16;
};

// Storage traits.  bf16 elements are carried as raw 16-bit patterns.
template <typename T> struct Traits;
template <> struct Traits<uint16_t> {
  static constexpr int E = 8;      // elements per 16-byte chunk (K rows)
  static constexpr int DPL = 4;    // dims per 16-byte V load (4 dims x 2 keys)
  typedef uint32_t Pair;           // probabilities of a key pair, packed bf16
};
template <> struct Traits<float> {
  static constexpr int E = 4;
  static constexpr int DPL = 2;    // 2 dims x 2 keys
  typedef float2 Pair;
};

// Partition [pb, pe) of a sequence's pages for split s of S: an even share.
__device__ __forceinline__ void split_range(int n_pages, int s, int S, int& pb, int& pe) {
  pb = (int)(((long long)s * n_pages) / S);
  pe = (int)(((long long)(s + 1) * n_pages) / S);
}

__device__ __forceinline__ int clamp_len(int n, int cap) { return n < 0 ? 0 : (n > cap ? cap : n); }

// q chunk (16 B) . k chunk (16 B), accumulated into acc.
__device__ __forceinline__ float chunk_dot(const uint4& q, const uint4& k, float acc, uint16_t) {
  acc = dot2_bf16(q.x, k.x, acc);
  acc = dot2_bf16(q.y, k.y, acc);
  acc = dot2_bf16(q.z, k.z, acc);
  acc = dot2_bf16(q.w, k.w, acc);
  return acc;
}
__device__ __forceinline__ float chunk_dot(const uint4& q, const uint4& k, float acc, float) {
  acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
  acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
  acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
  acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  return acc;
}

// acc[dd] += p_pair . v(pair, dim dd) for the DPL dims of one 16-byte V load.
__device__ __forceinline__ void pair_fma(float* acc, uint32_t pp, const uint4& v, uint16_t) {
  acc[0] = dot2_bf16(pp, v.x, acc[0]);
  acc[1] = dot2_bf16(pp, v.y, acc[1]);
  acc[2] = dot2_bf16(pp, v.z, acc[2]);
  acc[3] = dot2_bf16(pp, v.w, acc[3]);
}
__device__ __forceinline__ void pair_fma(float* acc, float2 pp, const uint4& v, float) {
  acc[0] = fmaf(pp.x, __uint_as_float(v.x), fmaf(pp.y, __uint_as_float(v.y), acc[0]));
  acc[1] = fmaf(pp.x, __uint_as_float(v.z), fmaf(pp.y, __uint_as_float(v.w), acc[1]));
}

// Zero the entries of keys >= nvalid in a V pair load (pool memory past the
// sequence end may hold NaN patterns; p = 0 there, but 0 * NaN is NaN).
// Branch-free: the key index differs per lane.
__device__ __forceinline__ void mask_pair(uint4& v, int key0, int nvalid, uint16_t) {
  const uint32_t lo = key0 < nvalid ? 0x0000ffffu : 0u;
  const uint32_t hi = key0 + 1 < nvalid ? 0xffff0000u : 0u;
  const uint32_t mk = lo | hi;
  v.x &= mk; v.y &= mk; v.z &= mk; v.w &= mk;
}
__device__ __forceinline__ void mask_pair(uint4& v, int key0, int nvalid, float) {
  const uint32_t m0 = key0 < nvalid ? 0xffffffffu : 0u;
  const uint32_t m1 = key0 + 1 < nvalid ? 0xffffffffu : 0u;
  v.x &= m0; v.y &= m1; v.z &= m0; v.w &= m1;
}

__device__ __forceinline__ void store_prob(uint32_t* pl, int idx, int half, float p, float& used) {
  const uint32_t bits = dev::f32_to_bf16_bits(p);
  used = __uint_as_float(bits << 16);
  reinterpret_cast<uint16_t*>(pl)[idx * 2 + half] = (uint16_t)bits;
}
__device__ __forceinline__ void store_prob(float2* pl, int idx, int half, float p, float& used) {
  used = p;
  reinterpret_cast<float*>(pl)[idx * 2 + half] = p;
}

__device__ __forceinline__ void store_out(void* out, size_t idx, float v, int bf16) {
  if (bf16)
    reinterpret_cast<uint16_t*>(out)[idx] = (uint16_t)dev::f32_to_bf16_bits(v);
  else
    reinterpret_cast<float*>(out)[idx] = v;
}

template <typename T, int HD, int NSRC>
__device__ __forceinline__ void load_k(uint4 (&kr)[NSRC][HD / Traits<T>::E], const T* const (&kt)[NSRC],
                                       int lane) {
  constexpr int E = Traits<T>::E;
#pragma unroll
  for (int s = 0; s < NSRC; ++s)
#pragma unroll
    for (int c = 0; c < HD / E; ++c)
      kr[s][c] = dev::ld16_stream(kt[s] + c * (kPage * E) + lane * E);
}

template <typename T, int HD, int NSRC, int PPL, int NPH, int DPL>
__device__ __forceinline__ void load_v(uint4 (&vr)[NSRC][PPL], const T* const (&vt)[NSRC], int ph,
                                       int quad) {
#pragma unroll
  for (int s = 0; s < NSRC; ++s)
#pragma unroll
    for (int j = 0; j < PPL; ++j)
      vr[s][j] = dev::ld16_stream(vt[s] + (ph + NPH * j) * (HD * 2) + quad * (DPL * 2));
}

template <typename T, int HD, int G, int NSRC>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams a) {
  typedef Traits<T> Tr;
  typedef typename Tr::Pair Pair;
  constexpr int E = Tr::E;
  constexpr int NCH = HD / E;        // 16-byte chunks per key row
  constexpr int DPL = Tr::DPL;
  constexpr int NQ = HD / DPL;       // lanes across the head dim in PV
  constexpr int NPH = 64 / NQ;       // pair phases
  constexpr int PPL = 32 / NPH;      // pairs per lane per page

  constexpr int NCW = NCH / kWays;   // chunks of a key row per lane (an eighth)

  // probabilities of key pair i, head h at i * PSTR + h; the padded row stride
  // spreads the 32 pairs over the LDS banks
  constexpr int PSTR = G + 2;
  __shared__ Pair p_lds[4][32 * PSTR];
  __shared__ float mrg_o[4][G][HD];
  __shared__ float mrg_m[4][G];
  __shared__ float mrg_l[4][G];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index as a scalar, so page loop control stays in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int S = a.n_splits;

  // QK lane roles: 8 lanes share a key; lane (k8, way) = 8*k8 + way holds the
  // query chunks 8*cc + way of every head in registers for the whole launch.
  const int way = lane & (kWays - 1);
  const int k8 = lane >> 3;
  uint4 qreg[G][NCW];
  {
    const uint4* qsrc = reinterpret_cast<const uint4*>(
        a.q + ((size_t)b * a.n_q_heads + (size_t)kvh * G) * HD * sizeof(T));
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int cc = 0; cc < NCW; ++cc) qreg[h][cc] = qsrc[h * NCH + kWays * cc + way];
  }
  // after the 8-lane reduction each lane keeps the scores of one key of the
  // page: pass `way`, i.e. key 8*way + k8
  const int my_key = 8 * way + k8;

  const int n_keys = clamp_len(a.seq_len[b] - a.key_excl, a.max_ctx);
  const int n_pages = (n_keys + kPage - 1) / kPage;
  int pb, pe;
  split_range(n_pages, split, S, pb, pe);

  const int quad = lane % NQ;
  const int ph = lane / NQ;
  Pair* pl = p_lds[wave];

  float m[G], lsum[G];
  float acc[NSRC][G][DPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int s = 0; s < NSRC; ++s)
#pragma unroll
      for (int d = 0; d < DPL; ++d) acc[s][h][d] = 0.f;
  }

  const int64_t slot_off[2] = {(int64_t)a.slot0 * a.slot_stride, (int64_t)a.slot1 * a.slot_stride};
  const int32_t* pt = a.page_table + (size_t)b * a.pages_per_seq;
  const T* kbase = reinterpret_cast<const T*>(a.k_pool);
  const T* vbase = reinterpret_cast<const T*>(a.v_pool);

  // next page of this wave whose page-table entry is valid (corrupt entries
  // are skipped, never read)
  auto next_page = [&](int from) {
    int p = from;
    while (p < pe && (unsigned)pt[p] >= (unsigned)a.n_phys_pages) p += 4;
    return p;
  };
  auto tiles = [&](int p, const T* (&kt)[NSRC], const T* (&vt)[NSRC]) {
    const int64_t tile = ((int64_t)pt[p] * a.n_kv_heads + kvh) * (kPage * HD);
#pragma unroll
    for (int s = 0; s < NSRC; ++s) {
      kt[s] = kbase + slot_off[s] + tile;
      vt[s] = vbase + slot_off[s] + tile;
    }
  };

  // One page: scores, online softmax and P V for the K/V already loaded in
  // (kr, vr).
  auto compute = [&](int pg, uint4 (&kr)[NSRC][NCH], uint4 (&vr)[NSRC][PPL]) {
    // ---- scores: pass j covers keys 8j..8j+7, an eighth of the head dim
    // per lane; quad_perm and row_half_mirror DPP adds complete the dot
    // products across the 8 lanes of a key
    const int nvalid = n_keys - pg * kPage;   // >= 1
    float sc[G];
#pragma unroll
    for (int j = 0; j < kWays; ++j) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int cc = 0; cc < NCW; ++cc) {
          d0 = chunk_dot(qreg[h][cc], kr[0][j * NCW + cc], d0, T());
          if (NSRC == 2) d1 = chunk_dot(qreg[h][cc], kr[NSRC - 1][j * NCW + cc], d1, T());
        }
        float s = (NSRC == 2) ? fmaf(a.w0, d0, a.w1 * d1) : d0;
        s = dev::add_dpp<0xB1>(s);    // quad_perm [1,0,3,2]
        s = dev::add_dpp<0x4E>(s);    // quad_perm [2,3,0,1]
        // the other quad of the 8: lane ^ 4 through ds_swizzle (bitmask mode,
        // xor 4), which keeps the VALU free
        s += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(s), (4 << 10) | 0x1f));
        if (j == 0) sc[h] = s;
        else sc[h] = (way == j) ? s : sc[h];
      }
    }
    const bool key_ok = my_key < nvalid;
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = key_ok ? sc[h] * a.scale_log2 : -INFINITY;

    // ---- online softmax
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mt = dev::wave_max(sc[h]);
      const float mn = fmaxf(m[h], mt);
      const float alpha = dev::fast_exp2(m[h] - mn);
      m[h] = mn;
      float used;
      store_prob(pl, (my_key >> 1) * PSTR + h, my_key & 1, dev::fast_exp2(sc[h] - mn), used);
      lsum[h] = fmaf(lsum[h], alpha, used);
#pragma unroll
      for (int s = 0; s < NSRC; ++s)
#pragma unroll
        for (int d = 0; d < DPL; ++d) acc[s][h][d] *= alpha;
    }
    __builtin_amdgcn_wave_barrier();

    // ---- P V, lane = (dims quad, pair phase)
    if (nvalid < kPage) {
#pragma unroll
      for (int s = 0; s < NSRC; ++s)
#pragma unroll
        for (int j = 0; j < PPL; ++j) mask_pair(vr[s][j], 2 * (ph + NPH * j), nvalid, T());
    }
#pragma unroll
    for (int j = 0; j < PPL; ++j) {
      const int i = ph + NPH * j;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const Pair pp = pl[i * PSTR + h];
#pragma unroll
        for (int s = 0; s < NSRC; ++s) pair_fma(acc[s][h], pp, vr[s][j], T());
      }
    }
    __builtin_amdgcn_wave_barrier();
  };
  auto load = [&](int pg, uint4 (&kr)[NSRC][NCH], uint4 (&vr)[NSRC][PPL]) {
    const T* kt[NSRC];
    const T* vt[NSRC];
    tiles(pg, kt, vt);
    load_k<T, HD, NSRC>(kr, kt, lane);
    load_v<T, HD, NSRC, PPL, NPH, DPL>(vr, vt, ph, quad);
  };

  for (int pg = next_page(pb + wave); pg < pe; pg = next_page(pg + 4)) {
    // both halves of the page are requested up front; the scores wait only
    // for K, while V is still in flight
    uint4 kr[NSRC][NCH];
    uint4 vr[NSRC][PPL];
    load(pg, kr, vr);
    compute(pg, kr, vr);
  }

  // ---- this wave's (O, m, l) to LDS
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float l = dev::wave_sum(lsum[h]);
#pragma unroll
    for (int d = 0; d < DPL; ++d) {
      float x0 = acc[0][h][d];
#pragma unroll
      for (int off = NQ; off < 64; off <<= 1) x0 += __shfl_xor(x0, off);
      if (NSRC == 2) {
        float x1 = acc[NSRC - 1][h][d];
#pragma unroll
        for (int off = NQ; off < 64; off <<= 1) x1 += __shfl_xor(x1, off);
        x0 = fmaf(a.w0, x0, a.w1 * x1);
      }
      if (lane < NQ) mrg_o[wave][h][quad * DPL + d] = x0;
    }
    if (lane == 0) {
      mrg_m[wave][h] = m[h];
      mrg_l[wave][h] = l;
    }
  }
  __syncthreads();

  // ---- merge the 4 waves; write the output (S == 1) or the partition
  const size_t hq0 = (size_t)b * a.n_q_heads + (size_t)kvh * G;
  for (int e = tid; e < G * HD; e += 256) {
    const int h = e / HD, d = e % HD;
    float M = mrg_m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, mrg_m[w][h]);
    float o = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = dev::fast_exp2(mrg_m[w][h] - M);
        o = fmaf(f, mrg_o[w][h][d], o);
        l = fmaf(f, mrg_l[w][h], l);
      }
    }
    if (S == 1) {
      store_out(a.out, (hq0 + h) * HD + d, l > 0.f ? o / l : 0.f, a.out_bf16);
    } else {
      const size_t row = (hq0 + h) * S + split;
      a.ws_o[row * HD + d] = o;
      if (d == 0) {
        a.ws_m[row] = M;
        a.ws_l[row] = l;
      }
    }
  }
}

// Merge of the S partitions of one (sequence, KV head): for each of its G
// query heads, out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s with
// M = max_s m_s.  Every partition writes its row, an empty one as
// (O = 0, m = -inf, l = 0), so a thread loads its S (m, l, O) triples 16 at
// a time with no dependence between them and folds each batch into a running
// (M, num, den); the order is fixed, so the result is deterministic.
// grid (Hkv, B), 256 threads.
template <int G, int HD>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams a) {
  const int tid = threadIdx.x;
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int S = a.n_splits;
  const size_t hq0 = (size_t)b * a.n_q_heads + (size_t)kvh * G;
  for (int e = tid; e < G * HD; e += 256) {
    const int h = e / HD, d = e % HD;
    const float* mrow = a.ws_m + (hq0 + h) * S;
    const float* lrow = a.ws_l + (hq0 + h) * S;
    const float* orow = a.ws_o + (hq0 + h) * S * HD + d;
    float M = -INFINITY, num = 0.f, den = 0.f;
    for (int s0 = 0; s0 < S; s0 += 16) {
      float mv[16], lv[16], ov[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int s = min(s0 + k, S - 1);
        mv[k] = s0 + k < S ? mrow[s] : -INFINITY;
        lv[k] = lrow[s];
        ov[k] = orow[(size_t)s * HD];
      }
      float Mn = M;
#pragma unroll
      for (int k = 0; k < 16; ++k) Mn = fmaxf(Mn, mv[k]);
      if (Mn != -INFINITY) {
        const float r = dev::fast_exp2(M - Mn);   // 0 while M is -inf
        num *= r;
        den *= r;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float f = dev::fast_exp2(mv[k] - Mn);   // 0 for empty or absent partitions
          num = fmaf(f, ov[k], num);
          den = fmaf(f, lv[k], den);
        }
        M = Mn;
      }
    }
    store_out(a.out, (hq0 + h) * HD + d, den > 0.f ? num / den : 0.f, a.out_bf16);
  }
}

// ---------------------------------------------------------------- MFMA path
// bf16, one source, hd 64 with G <= 32 or hd 128 with G = 16: both products
// of a page on v_mfma_f32_16x16x32_bf16 (A: lane l holds row l%16,
// k = 8(l/16)..+7; B: column l%16, same k; result register r of lane l is
// row 4(l/16)+r, column l%16), reading the cache in its stored layouts:
//   scores  S[keys][heads] = K q^T per block of 16 heads: A = 16 keys x 32
//           dims, one 16-byte load of a K row chunk per lane; B = 16 queries of the
//           group (columns past G zero), in registers for the whole launch.
//           Lane (g = l/16, h = l%16) ends with keys 16kb + 4g + r (kb =
//           0..3, r = 0..3) of head h of each block.
//   values  O[heads][dims] = P^T V over 32 keys per step, the keys of step ps
//           taken in the order those registers hold them:
//           k = 8g + e  ->  key 32ps + 16(e/4) + 4g + e%4,
//           so P^T is the lane's own (bf16) probabilities and the matching V
//           operand is 4 dwords of the pair-interleaved V page (each dword =
//           one dim of two consecutive keys).
// Every K and V tile is loaded once for all G heads: a group of 32 (hd 64)
// runs two 16-head blocks over the same page registers.
// The online softmax keeps one running maximum per head (raw scores; the
// positive scale is applied inside the exponent), so only heads whose
// maximum moved rescale their accumulators.
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_pk_t;

__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  const bf16x2_pk_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// max over the 4 rows of 16 lanes (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float row_max4(float x) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int HD>
struct MfmaPage {
  uint4 k[4][HD / 32];   // [kb][ks]: key 16kb + l%16, dims 8(l/16) + 32ks .. +7
  uint4 v[2][HD / 16];   // [ps][db]: 4 dwords (pairs) of dim 16db + l%16
};

// Waves per workgroup (one workgroup per (partition, KV head, sequence)).
// Each wave loads one page and computes it before loading the next.  With
// 256 workgroups of 4 waves that keeps 16 MB in flight, and the streaming
// rate is higher than with a second page in flight per wave (26.7 vs
// 28.4 us per tinyllama_cla2 layer) or with 8 or 2 waves (27.4, 30.4 us):
// more requests in flight lower the HBM efficiency, fewer leave it idle.
// Unsplit launches of at least one workgroup per CU stream faster still
// with three waves (batch 64 x 2K: 26.0-26.5 vs 26.6-26.9 us; 128 x 2K:
// 49.5 vs 51.1-51.4; 128 x 512: 16.2-16.4 vs 17.4-17.5), while smaller
// grids (8 x 512: 7.6-7.7 vs 6.5-6.7) and split ones (32 x 2K at S = 2:
// 18.2 vs 17.5; 16 x 1K at S = 4: 8.4-8.5 vs 7.5-7.7) lose with three, so
// the launcher takes NW = 3 for unsplit grids of at least 256 workgroups
// and 4 otherwise.
constexpr int kMfmaWavesSmall = 4;
constexpr int kMfmaWavesLarge = 3;
constexpr int kMfmaLargeGrid = 256;

template <int G, int HD, int NW>
__global__ __launch_bounds__(64 * NW) void decode_mfma_kernel(DecodeParams a) {
  constexpr int GB = (G + 15) / 16;          // 16-head blocks
  constexpr int KS = HD / 32;                // 32-dim steps of the scores
  constexpr int DB = HD / 16;                // 16-dim blocks of the values
  static_assert(G <= 32 && (HD == 64 || HD == 128), "shapes of the MFMA decode");
  __shared__ float mrg_o[NW][G][HD];
  __shared__ float mrg_m[NW][G];
  __shared__ float mrg_l[NW][G];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int S = a.n_splits;
  const int col = lane & 15, g = lane >> 4;

  // B operands of the scores: head 16gb + col, dims 8g + 32ks .. +7
  uint4 qf[GB][KS];
#pragma unroll
  for (int gb = 0; gb < GB; ++gb) {
    const int h = 16 * gb + col;
    const uint16_t* qh = reinterpret_cast<const uint16_t*>(a.q) +
                         ((size_t)b * a.n_q_heads + (size_t)kvh * G + (h < G ? h : 0)) * HD;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 x = *reinterpret_cast<const uint4*>(qh + 8 * g + 32 * ks);
      qf[gb][ks] = h < G ? x : make_uint4(0, 0, 0, 0);
    }
  }

  const int n_keys = clamp_len(a.seq_len[b] - a.key_excl, a.max_ctx);
  const int n_pages = (n_keys + kPage - 1) / kPage;
  int pb, pe;
  split_range(n_pages, split, S, pb, pe);
  const int32_t* pt = a.page_table + (size_t)b * a.pages_per_seq;
  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k_pool) + (int64_t)a.slot0 * a.slot_stride;
  const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.v_pool) + (int64_t)a.slot0 * a.slot_stride;

  auto next_page = [&](int from) {
    int p = from;
    while (p < pe && (unsigned)pt[p] >= (unsigned)a.n_phys_pages) p += NW;
    return p;
  };
  const int k_lane = ((col / 8) * (HD / 64) * kPage + (col % 8) * 8 + g) * 8;
  auto load = [&](int pg, MfmaPage<HD>& r) {
    const int64_t tile = ((int64_t)pt[pg] * a.n_kv_heads + kvh) * (kPage * HD);
    const uint16_t* kt = kbase + tile;
    const uint32_t* vt = reinterpret_cast<const uint32_t*>(vbase + tile);   // [32 pairs][HD dims]
    // 16-byte chunk c = g + 4ks of key t = 16kb + col at its place in the K
    // page layout, k_chunk_offset(t, c, HD/8, 8) split into this lane's part
    // and a constant per (kb, ks) (row-major at hd 64)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        r.k[kb][ks] = *reinterpret_cast<const uint4*>(
            kt + k_lane + ((2 * kb * (HD / 64) + ks / 2) * kPage + 4 * (ks % 2)) * 8);
#pragma unroll
    for (int ps = 0; ps < 2; ++ps)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = 16 * db + col;
        const int p0 = 16 * ps + 2 * g, p1 = p0 + 8;           // pairs of keys 32ps+4g.., 32ps+16+4g..
        r.v[ps][db] = make_uint4(vt[p0 * HD + d], vt[(p0 + 1) * HD + d], vt[p1 * HD + d],
                                 vt[(p1 + 1) * HD + d]);
      }
  };

  float m_run[GB], l_run[GB];   // for head 16gb + col, over this lane's keys
  f32x4_t o[GB][DB];
#pragma unroll
  for (int gb = 0; gb < GB; ++gb) {
    m_run[gb] = -INFINITY;
    l_run[gb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[gb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const uint32_t ones = 0x3F803F80u;       // (1.0, 1.0) in bf16

  auto compute = [&](int pg, MfmaPage<HD>& r) {
    const int nvalid = n_keys - pg * kPage;
#pragma unroll
    for (int gb = 0; gb < GB; ++gb) {
      f32x4_t s[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = mfma16(r.k[kb][0], qf[gb][0], f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int ks = 1; ks < KS; ++ks) s[kb] = mfma16(r.k[kb][ks], qf[gb][ks], s[kb]);
      }
      if (nvalid < kPage || 16 * gb + 16 > G) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s[kb][e] = (16 * gb + col < G && 16 * kb + 4 * g + e < nvalid) ? s[kb][e] : -INFINITY;
      }
      float mt = fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3]));
#pragma unroll
      for (int kb = 1; kb < 4; ++kb) mt = fmaxf(mt, fmaxf(fmaxf(s[kb][0], s[kb][1]), fmaxf(s[kb][2], s[kb][3])));
      mt = row_max4(mt);
      const float mn = fmaxf(m_run[gb], mt);
      const float neg = mn == -INFINITY ? 0.f : -mn * a.scale_log2;
      const float alpha = m_run[gb] == mn ? 1.f : dev::fast_exp2(fmaf(m_run[gb], a.scale_log2, neg));
      m_run[gb] = mn;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
        // accumulator entry rr of lane l belongs to head 16gb + 4(l/16) + rr
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float f = __shfl(alpha, 4 * g + rr);
#pragma unroll
          for (int db = 0; db < DB; ++db) o[gb][db][rr] *= f;
        }
        l_run[gb] *= alpha;
      }
      uint4 pf[2];
#pragma unroll
      for (int ps = 0; ps < 2; ++ps) {
        const f32x4_t& s0 = s[2 * ps];
        const f32x4_t& s1 = s[2 * ps + 1];
        pf[ps].x = pack_bf16_rne(dev::fast_exp2(fmaf(s0[0], a.scale_log2, neg)), dev::fast_exp2(fmaf(s0[1], a.scale_log2, neg)));
        pf[ps].y = pack_bf16_rne(dev::fast_exp2(fmaf(s0[2], a.scale_log2, neg)), dev::fast_exp2(fmaf(s0[3], a.scale_log2, neg)));
        pf[ps].z = pack_bf16_rne(dev::fast_exp2(fmaf(s1[0], a.scale_log2, neg)), dev::fast_exp2(fmaf(s1[1], a.scale_log2, neg)));
        pf[ps].w = pack_bf16_rne(dev::fast_exp2(fmaf(s1[2], a.scale_log2, neg)), dev::fast_exp2(fmaf(s1[3], a.scale_log2, neg)));
        // the running sum adds the same bf16-rounded probabilities
        l_run[gb] = dot2_bf16(pf[ps].x, ones, l_run[gb]);
        l_run[gb] = dot2_bf16(pf[ps].y, ones, l_run[gb]);
        l_run[gb] = dot2_bf16(pf[ps].z, ones, l_run[gb]);
        l_run[gb] = dot2_bf16(pf[ps].w, ones, l_run[gb]);
      }
      if (gb == 0 && nvalid < kPage) {
        // keys past the sequence end: p = 0, but unwritten V memory may hold
        // NaN patterns and 0 * NaN is NaN.  Masked here, after the scores,
        // so that the scores wait only for K while V is still in flight.
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
          const int k0 = 32 * ps + 4 * g, k1 = k0 + 16;
          const uint32_t m0 = (k0 < nvalid ? 0x0000ffffu : 0u) | (k0 + 1 < nvalid ? 0xffff0000u : 0u);
          const uint32_t m1 = (k0 + 2 < nvalid ? 0x0000ffffu : 0u) | (k0 + 3 < nvalid ? 0xffff0000u : 0u);
          const uint32_t m2 = (k1 < nvalid ? 0x0000ffffu : 0u) | (k1 + 1 < nvalid ? 0xffff0000u : 0u);
          const uint32_t m3 = (k1 + 2 < nvalid ? 0x0000ffffu : 0u) | (k1 + 3 < nvalid ? 0xffff0000u : 0u);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            r.v[ps][db].x &= m0;
            r.v[ps][db].y &= m1;
            r.v[ps][db].z &= m2;
            r.v[ps][db].w &= m3;
          }
        }
      }
#pragma unroll
      for (int ps = 0; ps < 2; ++ps)
#pragma unroll
        for (int db = 0; db < DB; ++db) o[gb][db] = mfma16(pf[ps], r.v[ps][db], o[gb][db]);
    }
  };

  MfmaPage<HD> bufA;
  for (int pg = next_page(pb + wave); pg < pe; pg = next_page(pg + NW)) {
    load(pg, bufA);
    compute(pg, bufA);
  }

  // ---- this wave's (O, m, l) to LDS; m in log2 units as the merge expects
#pragma unroll
  for (int gb = 0; gb < GB; ++gb) {
    float l = l_run[gb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int hc = 16 * gb + col;
    if (g == 0 && hc < G) {
      mrg_m[wave][hc] = m_run[gb] == -INFINITY ? -INFINITY : m_run[gb] * a.scale_log2;
      mrg_l[wave][hc] = l;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int h = 16 * gb + 4 * g + rr;
        if (h < G) mrg_o[wave][h][16 * db + col] = o[gb][db][rr];
      }
  }
  __syncthreads();

  const size_t hq0 = (size_t)b * a.n_q_heads + (size_t)kvh * G;
  for (int e = tid; e < G * HD; e += 64 * NW) {
    const int h = e / HD, d = e % HD;
    float M = mrg_m[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, mrg_m[w][h]);
    float ov = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = dev::fast_exp2(mrg_m[w][h] - M);
        ov = fmaf(f, mrg_o[w][h][d], ov);
        l = fmaf(f, mrg_l[w][h], l);
      }
    }
    if (S == 1) {
      store_out(a.out, (hq0 + h) * HD + d, l > 0.f ? ov / l : 0.f, a.out_bf16);
    } else {
      const size_t row = (hq0 + h) * S + split;
      a.ws_o[row * HD + d] = ov;
      if (d == 0) {
        a.ws_m[row] = M;
        a.ws_l[row] = l;
      }
    }
  }
}

template <int G, int HD>
int run_decode_mfma(const DecodeParams& p, int B, hipStream_t st, const KernelEvents& ev) {
  dim3 grid(p.n_splits, p.n_kv_heads, B);
  if (p.n_splits == 1 && (long long)p.n_kv_heads * B >= kMfmaLargeGrid)
    launch_main(ev, decode_mfma_kernel<G, HD, kMfmaWavesLarge>, grid, dim3(64 * kMfmaWavesLarge), st, p);
  else
    launch_main(ev, decode_mfma_kernel<G, HD, kMfmaWavesSmall>, grid, dim3(64 * kMfmaWavesSmall), st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_splits == 1) return (int)e;
  hipLaunchKernelGGL((decode_merge_kernel<G, HD>), dim3(p.n_kv_heads, B), dim3(256), 0, st, p);
  return (int)hipGetLastError();
}

// Which single-source bf16 calls take the MFMA decode: hd 64 up to G = 32,
// hd 128 at G = 16 (the dot-product kernel would hold 16 heads' queries
// beside a page: 512 registers and spills).  Smaller hd-128 groups stream
// faster through the dot-product kernel.
template <typename T, int HD, int G, int NSRC>
constexpr bool use_mfma_decode() {
  return sizeof(T) == 2 && NSRC == 1 && ((HD == 64 && G <= 32) || (HD == 128 && G == 16));
}

template <typename T, int HD, int G, int NSRC>
int run_decode(const DecodeParams& p, int B, hipStream_t st, const KernelEvents& ev) {
  if constexpr (use_mfma_decode<T, HD, G, NSRC>()) {
    return run_decode_mfma<G, HD>(p, B, st, ev);
  } else {
    dim3 grid(p.n_splits, p.n_kv_heads, B);
    launch_main(ev, decode_kernel<T, HD, G, NSRC>, grid, dim3(256), st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_splits == 1) return (int)e;
    hipLaunchKernelGGL((decode_merge_kernel<G, HD>), dim3(p.n_kv_heads, B), dim3(256), 0, st, p);
    return (int)hipGetLastError();
  }
}

typedef int (*DecodeFn)(const DecodeParams&, int, hipStream_t, const KernelEvents&);

template <typename T, int HD, int NSRC>
DecodeFn pick_group(int G) {
  switch (G) {
    case 1: return run_decode<T, HD, 1, NSRC>;
    case 2: return run_decode<T, HD, 2, NSRC>;
    case 4: return run_decode<T, HD, 4, NSRC>;
    case 8: return run_decode<T, HD, 8, NSRC>;
    default: break;
  }
  // large query groups (MQA-style): one source only, bf16 only
  if constexpr (NSRC == 1 && sizeof(T) == 2) {
    if (G == 16) return run_decode<T, HD, 16, 1>;
    if constexpr (HD == 64) {
      if (G == 32) return run_decode<T, 64, 32, 1>;
    }
  }
  return nullptr;
}

DecodeFn pick(int dtype, int hd, int G, int nsrc) {
  if (dtype == KVS_BF16) {
    if (hd == 64) return nsrc == 1 ? pick_group<uint16_t, 64, 1>(G) : pick_group<uint16_t, 64, 2>(G);
    if (hd == 128) return nsrc == 1 ? pick_group<uint16_t, 128, 1>(G) : pick_group<uint16_t, 128, 2>(G);
  } else {
    if (hd == 64) return nsrc == 1 ? pick_group<float, 64, 1>(G) : pick_group<float, 64, 2>(G);
    if (hd == 128) return nsrc == 1 ? pick_group<float, 128, 1>(G) : pick_group<float, 128, 2>(G);
  }
  return nullptr;
}

}  // namespace

int max_decode_splits() { return kMaxFusedSplits; }

bool decode_shape_supported(int32_t dtype, int32_t head_dim, int32_t group, int32_t n_src) {
  return pick(dtype, head_dim, group, n_src) != nullptr;
}

int launch_decode(const DecodeLaunch& a, void* stream) {
  DecodeFn fn = pick(a.dtype, a.head_dim, a.group, a.n_src);
  if (!fn || a.n_splits < 1 || a.n_splits > kMaxFusedSplits) return (int)hipErrorInvalidValue;
  DecodeParams p;
  p.k_pool = static_cast<const char*>(a.k_pool);
  p.v_pool = static_cast<const char*>(a.v_pool);
  p.page_table = a.page_table;
  p.pages_per_seq = a.pages_per_seq;
  p.n_phys_pages = a.n_phys_pages;
  p.n_kv_heads = a.n_kv_heads;
  p.n_q_heads = a.n_q_heads;
  p.slot_stride = a.slot_stride;
  p.slot0 = a.slot[0];
  p.slot1 = a.n_src == 2 ? a.slot[1] : a.slot[0];
  p.w0 = a.weight[0];
  p.w1 = a.n_src == 2 ? a.weight[1] : 0.f;
  p.q = static_cast<const char*>(a.q);
  p.seq_len = a.seq_len;
  p.max_ctx = a.max_ctx;
  p.key_excl = a.key_excl;
  p.n_splits = a.n_splits;
  p.scale_log2 = a.scale_log2;
  const size_t rows = (size_t)a.batch * a.n_q_heads * a.n_splits;
  p.ws_o = a.ws;
  p.ws_m = a.ws + rows * a.head_dim;
  p.ws_l = p.ws_m + rows;
  p.out = a.out;
  p.out_bf16 = a.out_dtype == KVS_BF16;
  return fn(p, a.batch, static_cast<hipStream_t>(stream), a.ev);
}

const char* hip_error_name(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace kvs
