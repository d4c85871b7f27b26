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
// the same values the explicit rebuild gives (up to rounding order).  The
// kernel therefore contracts the bases with the query once per workgroup
// (q~ = B^K q, u~ = U^K q), streams the coefficients, codes, scales and ranks
// once per (sequence, KV head) for all G query heads, accumulates in the
// 48-wide coefficient space, and applies B^V / U^V once per output row.
// Per token it moves 64+64 B of coefficients, 16+16 B of codes, 4 B of scales
// and the rank byte, and spends about 0.6 KFLOP instead of the 24.6 KFLOP an
// explicit 64x128 tile rebuild would cost.
//
// Page layouts (64 tokens per page and KV head):
//   cK  [4][64][8] bf16     coefficient chunk cc (8 values) of token t at
//                            (cc*64 + t)*8: a 1 KiB contiguous load per chunk
//   cV  [32][32][2] bf16    token pairs: (t, i) at (t/2)*64 + i*2 + t%2
//   dK  [64][16] int8        16 codes of token t at t*16
//   dV  [32][16][2] int8     token pairs: (t, j) at (t/2)*32 + j*2 + t%2
//   sK, sV [64] fp16; rank [64] uint8 per physical page (shared by all heads
//   and layers)
// Decomposition: grid (S, Hkv, B) of 4-wave workgroups, split-K over pages
// as in the dense decode, with the same LDS merge of the 4 waves and the
// same second-kernel merge across partitions (in coefficient space).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "common.cuh"
#include "internal.h"

namespace kvs {
namespace {

using dev::dot2_bf16;

constexpr int kR = 32;      // basis rank (coefficients per token)
constexpr int kRM = 16;     // residual codes per token
constexpr int kW = kR + kRM;
constexpr int kMaxSplitsF = 64;

struct FactParams {
  const uint16_t* ck; const uint16_t* cv;
  const int8_t* dk; const int8_t* dv;
  const uint16_t* sk; const uint16_t* sv;
  const uint8_t* rank;
  const uint16_t* bk; const uint16_t* bv;   // basis of the pair's slot: [Hkv][R][hd]
  const uint16_t* uk; const uint16_t* uv;   // residual directions of the layer: [Hkv][RM][hd]
  const int32_t* page_table;
  int32_t pages_per_seq;
  int32_t n_phys_pages;
  int32_t n_kv_heads;
  int32_t n_q_heads;
  int64_t coef_off;     // elements to the slot's cK/cV pages
  int64_t resid_off;    // elements to the layer's dK/dV pages
  int64_t scale_off;    // elements to the layer's sK/sV pages
  const uint16_t* q;
  const int32_t* seq_len;
  int32_t max_ctx;
  int32_t n_splits;
  float scale_log2;
  float* ws_c;          // [B][Hq][S][48]
  float* ws_m;          // [B][Hq][S]
  float* ws_l;          // [B][Hq][S]
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

// int8 code -> bf16 bits (exact: |d| <= 128 needs at most 8 significant bits)
__device__ __forceinline__ uint32_t i8_to_bf16(int v) { return __float_as_uint((float)v) >> 16; }

__device__ __forceinline__ void store_out(void* out, size_t idx, float v, int bf16) {
  if (bf16)
    reinterpret_cast<uint16_t*>(out)[idx] = (uint16_t)dev::f32_to_bf16_bits(v);
  else
    reinterpret_cast<float*>(out)[idx] = v;
}

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

template <int HD, int G>
__global__ __launch_bounds__(256) void fact_decode_kernel(FactParams a) {
  __shared__ float qt[G][kW];                  // (B^K q, U^K q) * log2(e)/sqrt(hd)
  __shared__ uint32_t p_lds[4][32 * G];        // p of a key pair, packed bf16
  __shared__ uint32_t ps_lds[4][32 * G];       // p * s^V of a key pair, packed bf16
  __shared__ float mrg_c[4][G][kW];
  __shared__ float mrg_m[4][G];
  __shared__ float mrg_l[4][G];
  __shared__ float fin_c[G * kW];
  __shared__ float fin_l[G];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int S = a.n_splits;

  // ---- absorbed query: qt[h][i] = (row i of B^K, or U^K for i >= R) . q_h
  for (int e = tid; e < G * kW; e += 256) {
    const int h = e / kW, i = e % kW;
    const uint16_t* row = i < kR ? a.bk + ((size_t)kvh * kR + i) * HD
                                 : a.uk + ((size_t)kvh * kRM + (i - kR)) * HD;
    const uint16_t* qr = a.q + ((size_t)b * a.n_q_heads + (size_t)kvh * G + h) * HD;
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < HD / 8; ++c) {
      const uint4 x = *reinterpret_cast<const uint4*>(row + c * 8);
      const uint4 y = *reinterpret_cast<const uint4*>(qr + c * 8);
      acc = dot2_bf16(x.x, y.x, acc);
      acc = dot2_bf16(x.y, y.y, acc);
      acc = dot2_bf16(x.z, y.z, acc);
      acc = dot2_bf16(x.w, y.w, acc);
    }
    qt[h][i] = acc * a.scale_log2;
  }
  __syncthreads();

  const int n_keys = min(max(a.seq_len[b], 0), a.max_ctx);
  const int n_pages = (n_keys + kPage - 1) / kPage;
  int pb, pe;
  split_range(n_pages, split, S, pb, pe);
  const int32_t* pt = a.page_table + (size_t)b * a.pages_per_seq;

  // V-side lane roles: C part lane (q8 = coefs 4*q8.., ph8 = pair phase),
  // D part lane (jq = codes 8*jq.., dp = key pair)
  const int q8 = lane & 7, ph8 = lane >> 3;
  const int jq = lane & 1, dp = lane >> 1;

  float m[G], lsum[G], acc_c[G][4], acc_d[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc_c[h][i] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc_d[h][j] = 0.f;
  }

  for (int pg = pb + wave; pg < pe; pg += 4) {
    const int phys = pt[pg];
    if ((unsigned)phys >= (unsigned)a.n_phys_pages) continue;   // corrupt entry: never read
    const size_t page_kv = (size_t)phys * a.n_kv_heads + kvh;
    const uint16_t* ckp = a.ck + a.coef_off + page_kv * 64 * kR;
    const uint16_t* cvp = a.cv + a.coef_off + page_kv * 64 * kR;
    const int8_t* dkp = a.dk + a.resid_off + page_kv * 64 * kRM;
    const int8_t* dvp = a.dv + a.resid_off + page_kv * 64 * kRM;
    const uint16_t* skp = a.sk + a.scale_off + page_kv * 64;
    const uint16_t* svp = a.sv + a.scale_off + page_kv * 64;
    const uint8_t* rkp = a.rank + (size_t)phys * 64;

    // all loads of the page up front
    uint4 ckr[4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) ckr[cc] = *reinterpret_cast<const uint4*>(ckp + (cc * 64 + lane) * 8);
    const uint4 dkr = *reinterpret_cast<const uint4*>(dkp + lane * 16);
    const uint16_t skr = skp[lane];
    const uint16_t svr = svp[lane];
    const int r_t = rkp[lane];
    uint4 cvr[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      cvr[k] = *reinterpret_cast<const uint4*>(cvp + (ph8 + 8 * k) * (kR * 2) + q8 * 8);
    const uint4 dvr = *reinterpret_cast<const uint4*>(dvp + dp * (kRM * 2) + jq * 16);
    const uint16_t rpair = *reinterpret_cast<const uint16_t*>(rkp + 2 * dp);

    const int nvalid = n_keys - pg * kPage;
    const bool key_ok = lane < nvalid;

    // ---- scores, lane = token
    float cf[kR], df[kRM];
    {
      const uint32_t* cw = &ckr[0].x;
#pragma unroll
      for (int w = 0; w < 16; ++w) {
        cf[2 * w] = dev::bf16_lo(cw[w]);
        cf[2 * w + 1] = dev::bf16_hi(cw[w]);
      }
      const uint32_t* dw = &dkr.x;
#pragma unroll
      for (int j = 0; j < kRM; ++j) {
        const int v = (int)(int8_t)((dw[j / 4] >> (8 * (j % 4))) & 0xff);
        df[j] = j < r_t ? (float)v : 0.f;
      }
    }
    const float sKf = half_to_float(skr);
    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float zc = 0.f, zd = 0.f;
#pragma unroll
      for (int i = 0; i < kR; ++i) zc = fmaf(cf[i], qt[h][i], zc);
#pragma unroll
      for (int j = 0; j < kRM; ++j) zd = fmaf(df[j], qt[h][kR + j], zd);
      const float z = fmaf(sKf, zd, zc);
      sc[h] = key_ok ? z : -INFINITY;
    }

    // ---- online softmax; p and p*s^V to LDS as bf16 key pairs
    const float sVf = key_ok ? half_to_float(svr) : 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mt = dev::wave_max(sc[h]);
      const float mn = fmaxf(m[h], mt);
      const float alpha = dev::fast_exp2(m[h] - mn);
      m[h] = mn;
      const uint32_t pbits = dev::f32_to_bf16_bits(dev::fast_exp2(sc[h] - mn));
      const float p = __uint_as_float(pbits << 16);
      lsum[h] = fmaf(lsum[h], alpha, p);
      reinterpret_cast<uint16_t*>(p_lds[wave])[((lane >> 1) * G + h) * 2 + (lane & 1)] = (uint16_t)pbits;
      reinterpret_cast<uint16_t*>(ps_lds[wave])[((lane >> 1) * G + h) * 2 + (lane & 1)] =
          (uint16_t)dev::f32_to_bf16_bits(p * sVf);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc_c[h][i] *= alpha;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc_d[h][j] *= alpha;
    }
    __builtin_amdgcn_wave_barrier();

    // ---- coefficient-space accumulation
    if (nvalid < kPage) {   // unwritten pool memory past the sequence end may hold NaN patterns
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int key0 = 2 * (ph8 + 8 * k);
        const uint32_t mk = (key0 < nvalid ? 0x0000ffffu : 0u) | (key0 + 1 < nvalid ? 0xffff0000u : 0u);
        cvr[k].x &= mk; cvr[k].y &= mk; cvr[k].z &= mk; cvr[k].w &= mk;
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = ph8 + 8 * k;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint32_t pp = p_lds[wave][p * G + h];
        acc_c[h][0] = dot2_bf16(pp, cvr[k].x, acc_c[h][0]);
        acc_c[h][1] = dot2_bf16(pp, cvr[k].y, acc_c[h][1]);
        acc_c[h][2] = dot2_bf16(pp, cvr[k].z, acc_c[h][2]);
        acc_c[h][3] = dot2_bf16(pp, cvr[k].w, acc_c[h][3]);
      }
    }
    {
      const int r0 = rpair & 0xff, r1 = rpair >> 8;     // ranks of keys 2dp, 2dp+1
      const uint32_t* dw = &dvr.x;
      uint32_t dpair[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int j = 8 * jq + jj;
        const uint32_t two = (dw[jj / 2] >> (16 * (jj % 2))) & 0xffffu;   // (key 2dp, key 2dp+1)
        const int v0 = (int)(int8_t)(two & 0xff), v1 = (int)(int8_t)(two >> 8);
        dpair[jj] = (j < r0 ? i8_to_bf16(v0) : 0u) | ((j < r1 ? i8_to_bf16(v1) : 0u) << 16);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint32_t pp = ps_lds[wave][dp * G + h];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) acc_d[h][jj] = dot2_bf16(pp, dpair[jj], acc_d[h][jj]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- this wave's (coefficient sums, m, l) to LDS
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float l = dev::wave_sum(lsum[h]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = acc_c[h][i];
      x += __shfl_xor(x, 8);
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      if (lane < 8) mrg_c[wave][h][4 * q8 + i] = x;
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      float x = acc_d[h][jj];
#pragma unroll
      for (int off = 2; off < 64; off <<= 1) x += __shfl_xor(x, off);
      if (lane < 2) mrg_c[wave][h][kR + 8 * jq + jj] = x;
    }
    if (lane == 0) {
      mrg_m[wave][h] = m[h];
      mrg_l[wave][h] = l;
    }
  }
  __syncthreads();

  const size_t hq0 = (size_t)b * a.n_q_heads + (size_t)kvh * G;
  for (int e = tid; e < G * kW; e += 256) {
    const int h = e / kW, i = e % kW;
    float M = mrg_m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, mrg_m[w][h]);
    float c = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = dev::fast_exp2(mrg_m[w][h] - M);
        c = fmaf(f, mrg_c[w][h][i], c);
        l = fmaf(f, mrg_l[w][h], l);
      }
    }
    if (S == 1) {
      fin_c[e] = c;
      if (i == 0) fin_l[h] = l;
    } else {
      const size_t row = (hq0 + h) * S + split;
      a.ws_c[row * kW + i] = c;
      if (i == 0) {
        a.ws_m[row] = M;
        a.ws_l[row] = l;
      }
    }
  }
  if (S != 1) return;
  __syncthreads();
  project_out<HD, G>(a, b, kvh, fin_c, fin_l, tid, 256);
}

// Merge of S partitions in coefficient space, then the basis projection.
// Every partition writes its row (an empty one as c = 0, m = -inf, l = 0).
// Loads that do not depend on each other are issued together: the maxima and
// sums to LDS, each thread's basis column (its d is fixed: 256 is a multiple
// of HD) into registers, then the S coefficient partials.
template <int HD, int G>
__global__ __launch_bounds__(256) void fact_merge_kernel(FactParams a) {
  static_assert(256 % HD == 0, "a thread keeps one output column");
  __shared__ float m_lds[G * kMaxSplitsF];
  __shared__ float l_lds[G * kMaxSplitsF];
  __shared__ float den[G];
  __shared__ float coef[G * kW];
  const int tid = threadIdx.x;
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int S = a.n_splits;
  const size_t hq0 = (size_t)b * a.n_q_heads + (size_t)kvh * G;
  for (int i = tid; i < G * S; i += 256) {
    m_lds[i] = a.ws_m[hq0 * S + i];
    l_lds[i] = a.ws_l[hq0 * S + i];
  }
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
  __syncthreads();
  for (int e = tid; e < G * kW; e += 256) {
    const int h = e / kW, i = e % kW;
    const float* ml = m_lds + h * S;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, ml[s]);
    const float* c = a.ws_c + (hq0 + h) * S * kW + i;
    float acc = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll 8
      for (int s = 0; s < S; ++s) {
        const float f = dev::fast_exp2(ml[s] - M);   // 0 for an empty partition
        acc = fmaf(f, c[(size_t)s * kW], acc);
        l = fmaf(f, l_lds[h * S + s], l);
      }
    }
    coef[e] = acc;
    if (i == 0) den[h] = l;
  }
  __syncthreads();
  for (int h = tid / HD; h < G; h += 256 / HD) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < kW; ++i) acc = fmaf(coef[h * kW + i], col[i], acc);
    const float l = den[h];
    store_out(a.out, (hq0 + h) * HD + d, l > 0.f ? acc / l : 0.f, a.out_bf16);
  }
}

template <int HD, int G>
int run_fact(const FactParams& p, int B, hipStream_t st) {
  hipLaunchKernelGGL((fact_decode_kernel<HD, G>), dim3(p.n_splits, p.n_kv_heads, B), dim3(256), 0,
                     st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_splits == 1) return (int)e;
  hipLaunchKernelGGL((fact_merge_kernel<HD, G>), dim3(p.n_kv_heads, B), dim3(256), 0, st, p);
  return (int)hipGetLastError();
}

typedef int (*FactFn)(const FactParams&, int, hipStream_t);

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

__global__ __launch_bounds__(256) void fact_append_kernel(FactAppendLaunch a) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)a.batch * a.n * a.n_kv_heads;
  if (idx >= total) return;
  const int kvh = (int)(idx % a.n_kv_heads);
  const long long bi = idx / a.n_kv_heads;
  const int i = (int)(bi % a.n);
  const int b = (int)(bi / a.n);
  const int pos = a.start_pos[b] + i;
  if (pos < 0 || pos >= a.max_ctx) return;
  const int page = a.page_table[(size_t)b * a.pages_per_seq + pos / kPage];
  if (page < 0 || page >= a.n_phys_pages) return;
  const int t = pos % kPage;
  const size_t page_kv = (size_t)page * a.n_kv_heads + kvh;
  const size_t src_row = ((size_t)b * a.n + i) * a.n_kv_heads + kvh;
  if (a.coef_slot >= 0) {
    const size_t base = ((size_t)a.coef_slot * a.n_phys_pages * a.n_kv_heads + page_kv) * 64 * kR;
    const uint16_t* ck = static_cast<const uint16_t*>(a.ck) + src_row * kR;
    const uint16_t* cv = static_cast<const uint16_t*>(a.cv) + src_row * kR;
    uint16_t* dk = static_cast<uint16_t*>(a.ck_pool) + base;
    uint16_t* dv = static_cast<uint16_t*>(a.cv_pool) + base;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
      *reinterpret_cast<uint4*>(dk + (cc * 64 + t) * 8) = *reinterpret_cast<const uint4*>(ck + cc * 8);
#pragma unroll 8
    for (int e = 0; e < kR; ++e) dv[(t >> 1) * (kR * 2) + e * 2 + (t & 1)] = cv[e];
  }
  {
    const size_t lbase = (size_t)a.layer * a.n_phys_pages * a.n_kv_heads + page_kv;
    int8_t* dk = static_cast<int8_t*>(a.dk_pool) + lbase * 64 * kRM;
    int8_t* dv = static_cast<int8_t*>(a.dv_pool) + lbase * 64 * kRM;
    *reinterpret_cast<uint4*>(dk + t * kRM) = *reinterpret_cast<const uint4*>(a.dk + src_row * kRM);
    const int8_t* sv = a.dv + src_row * kRM;
#pragma unroll
    for (int j = 0; j < kRM; ++j) dv[(t >> 1) * (kRM * 2) + j * 2 + (t & 1)] = sv[j];
    static_cast<uint16_t*>(a.sk_pool)[lbase * 64 + t] = static_cast<const uint16_t*>(a.sk)[src_row];
    static_cast<uint16_t*>(a.sv_pool)[lbase * 64 + t] = static_cast<const uint16_t*>(a.sv)[src_row];
  }
  if (a.rank && kvh == 0) {
    const uint8_t r = a.rank[(size_t)b * a.n + i];
    static_cast<uint8_t*>(a.rank_pool)[(size_t)page * 64 + t] = r > kRM ? (uint8_t)kRM : r;
  }
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
  p.rank = static_cast<const uint8_t*>(a.rank_pool);
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
  p.coef_off = (int64_t)a.coef_slot * a.n_phys_pages * a.n_kv_heads * 64 * kR;
  p.resid_off = (int64_t)a.layer * a.n_phys_pages * a.n_kv_heads * 64 * kRM;
  p.scale_off = (int64_t)a.layer * a.n_phys_pages * a.n_kv_heads * 64;
  p.q = static_cast<const uint16_t*>(a.q);
  p.seq_len = a.seq_len;
  p.max_ctx = a.max_ctx;
  p.n_splits = a.n_splits;
  p.scale_log2 = a.scale_log2;
  const size_t rows = (size_t)a.batch * a.n_q_heads * a.n_splits;
  p.ws_c = a.ws;
  p.ws_m = a.ws + rows * kW;
  p.ws_l = p.ws_m + rows;
  p.out = a.out;
  p.out_bf16 = a.out_dtype == KVS_BF16;
  return fn(p, a.batch, static_cast<hipStream_t>(stream));
}

int launch_fact_append(const FactAppendLaunch& a, void* stream) {
  const long long total = (long long)a.batch * a.n * a.n_kv_heads;
  if (total == 0) return 0;
  hipLaunchKernelGGL(fact_append_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

}  // namespace kvs
