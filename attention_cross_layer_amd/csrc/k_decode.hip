// Split-K decode attention over a shared (paged, source-only) K/V cache, and
// the combine of the per-partition partial results.
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
//   grid (ceil(n_splits / 4), Hkv, B), 256 threads = 4 independent waves.
//   Each wave owns one split-K partition: a run of whole 64-key pages of one
//   (sequence, KV head).  All G query heads of that KV head are served by
//   the same pass, so every cached tile is read from HBM once per
//   (sequence, KV head) -- once for the whole query group.
//   Per page:
//     QK   lane t owns key t.  The K page is stored as [hd/E][64][E] (E
//          elements = 16 bytes), so chunk c of all 64 keys is one contiguous
//          1 KiB load.  The G query rows are broadcast from LDS; scores use
//          v_dot2c_f32_bf16 (fp32 accumulate).
//     softmax  wave-wide max per head over DPP, running max/sum rescaling
//          (online softmax); probabilities are rounded to bf16 for the PV
//          products and the running sum uses the same rounded values.
//     PV   the V page is stored as token pairs [32][hd][2], so a 16-byte load
//          holds 4 dims x 2 keys; lane l owns dims 4*(l % (hd/4)) and every
//          NPH-th pair; each dword feeds v_dot2c_f32_bf16 with the pair's two
//          probabilities read from LDS.
//   A partition's result (unnormalised O, running max m, running sum l; log2
//   domain) goes to the workspace; the combine kernel merges partitions in
//   fixed order, so results are deterministic for a fixed split count.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "common.cuh"
#include "internal.h"

namespace kvs {
namespace {

using dev::dot2_bf16;

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
  int32_t n_splits;
  float scale_log2;
  float* ws_o;           // [B][Hq][S][HD]
  float* ws_m;           // [B][Hq][S]
  float* ws_l;           // [B][Hq][S]
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
// sequence end is unwritten and may hold NaN patterns; p = 0 there, but
// 0 * NaN is NaN).
__device__ __forceinline__ void mask_pair(uint4& v, int key0, int nvalid, uint16_t) {
  if (key0 >= nvalid) {
    v = make_uint4(0, 0, 0, 0);
  } else if (key0 + 1 >= nvalid) {
    v.x &= 0xffffu; v.y &= 0xffffu; v.z &= 0xffffu; v.w &= 0xffffu;
  }
}
__device__ __forceinline__ void mask_pair(uint4& v, int key0, int nvalid, float) {
  if (key0 >= nvalid) {
    v = make_uint4(0, 0, 0, 0);
  } else if (key0 + 1 >= nvalid) {
    v.y = 0; v.w = 0;
  }
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

template <typename T, int HD, int G, int NSRC>
__global__ __launch_bounds__(256) void decode_partial_kernel(DecodeParams a) {
  typedef Traits<T> Tr;
  typedef typename Tr::Pair Pair;
  constexpr int E = Tr::E;
  constexpr int NCH = HD / E;        // 16-byte chunks per key row
  constexpr int DPL = Tr::DPL;
  constexpr int NQ = HD / DPL;       // lanes across the head dim in PV
  constexpr int NPH = 64 / NQ;       // pair phases
  constexpr int PPL = 32 / NPH;      // pairs per lane per page

  __shared__ uint4 q_lds[G * NCH];
  __shared__ Pair p_lds[4][32 * G];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.z;
  const int kvh = blockIdx.y;
  const int split = blockIdx.x * 4 + wave;

  {
    const uint4* qsrc = reinterpret_cast<const uint4*>(
        a.q + ((size_t)b * a.n_q_heads + (size_t)kvh * G) * HD * sizeof(T));
    for (int i = threadIdx.x; i < G * NCH; i += 256) q_lds[i] = qsrc[i];
  }
  __syncthreads();
  if (split >= a.n_splits) return;

  const int n_keys = clamp_len(a.seq_len[b], a.max_ctx);
  const int n_pages = (n_keys + kPage - 1) / kPage;
  int pb, pe;
  split_range(n_pages, split, a.n_splits, pb, pe);
  if (pb >= pe) return;

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

  for (int pg = pb; pg < pe; ++pg) {
    const int phys = pt[pg];
    if ((unsigned)phys >= (unsigned)a.n_phys_pages) continue;   // corrupt entry: never read
    const int64_t tile = ((int64_t)phys * a.n_kv_heads + kvh) * (kPage * HD);
    uint4 kr[NSRC][NCH];
    uint4 vr[NSRC][PPL];
#pragma unroll
    for (int s = 0; s < NSRC; ++s) {
      const T* kt = reinterpret_cast<const T*>(a.k_pool) + slot_off[s] + tile;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        kr[s][c] = *reinterpret_cast<const uint4*>(kt + c * (kPage * E) + lane * E);
    }
#pragma unroll
    for (int s = 0; s < NSRC; ++s) {
      const T* vt = reinterpret_cast<const T*>(a.v_pool) + slot_off[s] + tile;
#pragma unroll
      for (int j = 0; j < PPL; ++j)
        vr[s][j] = *reinterpret_cast<const uint4*>(vt + (ph + NPH * j) * (HD * 2) + quad * (DPL * 2));
    }

    // ---- scores, lane = key
    const int nvalid = n_keys - pg * kPage;   // >= 1
    const bool key_ok = lane < nvalid;
    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float d0 = 0.f, d1 = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint4 qc = q_lds[h * NCH + c];
        d0 = chunk_dot(qc, kr[0][c], d0, T());
        if (NSRC == 2) d1 = chunk_dot(qc, kr[NSRC - 1][c], d1, T());
      }
      const float s = (NSRC == 2) ? fmaf(a.w0, d0, a.w1 * d1) : d0;
      sc[h] = key_ok ? s * a.scale_log2 : -INFINITY;
    }

    // ---- online softmax
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mt = dev::wave_max(sc[h]);
      const float mn = fmaxf(m[h], mt);
      const float alpha = dev::fast_exp2(m[h] - mn);
      m[h] = mn;
      float used;
      store_prob(pl, (lane >> 1) * G + h, lane & 1, dev::fast_exp2(sc[h] - mn), used);
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
        const Pair pp = pl[i * G + h];
#pragma unroll
        for (int s = 0; s < NSRC; ++s) pair_fma(acc[s][h], pp, vr[s][j], T());
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- write the partition's partial result
  const int S = a.n_splits;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float l = dev::wave_sum(lsum[h]);
    float o[DPL];
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
      o[d] = x0;
    }
    const size_t row = ((size_t)b * a.n_q_heads + (size_t)kvh * G + h) * S + split;
    if (lane < NQ) {
      float* dst = a.ws_o + row * HD + quad * DPL;
#pragma unroll
      for (int d = 0; d < DPL; ++d) dst[d] = o[d];
    }
    if (lane == 0) {
      a.ws_m[row] = m[h];
      a.ws_l[row] = l;
    }
  }
}

// Merge the partitions of one (sequence, q head): out = sum_s 2^(m_s - M) O_s /
// sum_s 2^(m_s - M) l_s, M = max_s m_s, in split order.  grid (Hq, B), 64 threads.
template <int HD>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* ws_o, const float* ws_m,
                                                            const float* ws_l,
                                                            const int32_t* seq_len, int max_ctx,
                                                            int n_q_heads, int S, void* out,
                                                            int out_bf16) {
  constexpr int DPT = HD / 64;
  const int hq = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int n_keys = clamp_len(seq_len[b], max_ctx);
  const int n_pages = (n_keys + kPage - 1) / kPage;
  const size_t row0 = ((size_t)b * n_q_heads + hq) * S;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) {
    int pb, pe;
    split_range(n_pages, s, S, pb, pe);
    if (pb < pe) M = fmaxf(M, ws_m[row0 + s]);
  }
  float den = 0.f, num[DPT];
#pragma unroll
  for (int d = 0; d < DPT; ++d) num[d] = 0.f;
  for (int s = 0; s < S; ++s) {
    int pb, pe;
    split_range(n_pages, s, S, pb, pe);
    if (pb >= pe) continue;
    const float f = dev::fast_exp2(ws_m[row0 + s] - M);
    den = fmaf(f, ws_l[row0 + s], den);
    const float* o = ws_o + (row0 + s) * HD;
#pragma unroll
    for (int d = 0; d < DPT; ++d) num[d] = fmaf(f, o[lane + 64 * d], num[d]);
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const size_t orow = ((size_t)b * n_q_heads + hq) * HD;
#pragma unroll
  for (int d = 0; d < DPT; ++d) {
    const float r = num[d] * inv;
    if (out_bf16)
      reinterpret_cast<uint16_t*>(out)[orow + lane + 64 * d] = (uint16_t)dev::f32_to_bf16_bits(r);
    else
      reinterpret_cast<float*>(out)[orow + lane + 64 * d] = r;
  }
}

template <typename T, int HD, int G, int NSRC>
int run_decode(const DecodeParams& p, int B, int S, int Hkv, const int32_t* seq_len, int max_ctx,
               void* out, int out_bf16, hipStream_t st) {
  dim3 grid((S + 3) / 4, Hkv, B);
  hipLaunchKernelGGL((decode_partial_kernel<T, HD, G, NSRC>), grid, dim3(256), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL((decode_combine_kernel<HD>), dim3(p.n_q_heads, B), dim3(64), 0, st, p.ws_o,
                     p.ws_m, p.ws_l, seq_len, max_ctx, p.n_q_heads, S, out, out_bf16);
  return (int)hipGetLastError();
}

typedef int (*DecodeFn)(const DecodeParams&, int, int, int, const int32_t*, int, void*, int,
                        hipStream_t);

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

bool decode_shape_supported(int32_t dtype, int32_t head_dim, int32_t group, int32_t n_src) {
  return pick(dtype, head_dim, group, n_src) != nullptr;
}

int launch_decode(const DecodeLaunch& a, void* stream) {
  DecodeFn fn = pick(a.dtype, a.head_dim, a.group, a.n_src);
  if (!fn) return (int)hipErrorInvalidValue;
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
  p.n_splits = a.n_splits;
  p.scale_log2 = a.scale_log2;
  const size_t rows = (size_t)a.batch * a.n_q_heads * a.n_splits;
  p.ws_o = a.ws;
  p.ws_m = a.ws + rows * a.head_dim;
  p.ws_l = p.ws_m + rows;
  return fn(p, a.batch, a.n_splits, a.n_kv_heads, a.seq_len, a.max_ctx, a.out,
            a.out_dtype == KVS_BF16, static_cast<hipStream_t>(stream));
}

const char* hip_error_name(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace kvs
