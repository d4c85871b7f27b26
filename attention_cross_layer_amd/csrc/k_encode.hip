// Write side of the factorized cache: the encoder that turns a layer's K/V
// rows into pair coefficients and int8 residual codes, and the basis builder
// (pair basis, per-layer residual directions).
//
// The cache follows DepthWeave-KV ("DepthWeave-KV: Smarter KV Cache
// Compression by Sharing Across Layers and Adapting Per Token", Core
// Mechanism): a low-rank channel basis B shared by a pair of neighbouring
// layers, computed from their own K/V without training, plus a small
// low-rank quantized residual per layer.  The page gives no numerical recipe;
// this file implements the readings
//   c_t  = bf16(B x^o_t)                  x^o: the pair's coefficient-writing layer
//   y_t  = U_l (x_t - c_t B)              the residual on the layer's directions
//   s_t  = fp16(max_{j<r_t} |y_tj| / 127),  d_tj = clamp(rne(y_tj / s_t), +-127)
//   B    = R leading right singular vectors of the pair's stacked token rows
//   U_l  = Rmax leading right singular vectors of the layer's residual rows
// (rows sign-normalised: largest-magnitude entry positive).
//
// Encoder (one wave per 32 tokens of one KV head and one of K / V, four
// waves per workgroup sharing the basis staged in LDS;
// v_mfma_f32_32x32x16_bf16, lane l of A/B holding row or column l%32 and
// k = 8(l/32)+e, result register r of lane l = row 8(r/4)+4(l/32)+r%4,
// column l%32):
//   C^T  = B X_o^T                 hd/16 MFMAs; rounded to bf16, the result
//                                  registers are the next product's B operand
//                                  (coefficient order 8(r/4)+4(l/32)+r%4)
//   R^T  = B^T C^T, E^T = X^T - R^T  B^T staged in LDS with each 16-wide group's
//                                  quads 1 and 2 swapped to match that order
//   Y^T  = [U; 0] E^T              E^T split into a bf16 high part and the
//                                  bf16 rounding of the rest (two products per
//                                  step), so y carries about 16 bits
//   quantize per token (the two lane halves of a token combine their maxima)
// and writes the coefficients / codes / scales in the input format of the
// factorized append, which places them in the paged layout.
//
// Basis builder: Gram matrices of the rows (fp32, one workgroup per 32x32
// block pair and KV head), then one workgroup per Gram matrix runs cyclic
// Jacobi rotations in LDS (parallel round-robin ordering: 64 disjoint pairs
// per round) until the off-diagonal mass is negligible, and writes the
// leading eigenvectors (largest eigenvalue first) as bf16 rows.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "common.h"
#include "internal.h"

namespace kvs {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

constexpr int kR = 32;
constexpr int kRM = 16;
constexpr int kBT = kR + 8;       // transposed basis row pitch (coefficients)

__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ int swz16(int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); }

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

struct EncodeSide {
  const uint16_t* x;        // [B][n][Hkv][hd] bf16: the layer's rows
  const uint16_t* xo;       // the coefficient-writing layer's rows (may be x)
  const uint16_t* basis;    // [Hkv][R][hd] bf16
  const uint16_t* ubasis;   // [Hkv][RM][hd] bf16 (codes mode)
  uint16_t* c_out;          // [B][n][Hkv][R] bf16, or null
  int8_t* d_out;            // [B][n][Hkv][RM]
  uint16_t* s_out;          // [B][n][Hkv] fp16
  float* e_out;             // residual mode: [B][n][Hkv][hd] fp32
};

struct EncodeParams {
  EncodeSide side[2];       // K, V
  const uint8_t* rank;      // [B][n]
  const int32_t* n_tokens;  // residual mode: rows t >= n_tokens[b] are not written
  int32_t n;
  int32_t n_kv_heads;
  int32_t residual_mode;
};

constexpr int kEncWaves = 4;      // waves per workgroup, 32 tokens each, sharing the staged B^T

// grid (ceil(n / (32 kEncWaves)), 2 Hkv, B), kEncWaves waves
template <int HD>
__global__ __launch_bounds__(64 * kEncWaves) void encode_kernel(EncodeParams a) {
  constexpr int KS = HD / 16;
  constexpr int MB = HD / 32;
  __shared__ __attribute__((aligned(16))) uint16_t bt[HD * kBT];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, col = lane & 31;
  const int kvh = blockIdx.y >> 1, kv = blockIdx.y & 1, b = blockIdx.z;
  const EncodeSide& s = a.side[kv];
  const int i = (blockIdx.x * kEncWaves + wave) * 32 + col;
  const bool ok = i < a.n;
  const size_t row = ((size_t)b * a.n + (ok ? i : a.n - 1)) * a.n_kv_heads + kvh;
  const uint16_t* xr = s.x + row * HD;
  const uint16_t* xo = s.xo + row * HD;
  const uint16_t* bh = s.basis + (size_t)kvh * kR * HD;

  // B^T into LDS: position swz16(i) of row d holds B[i][d]
  for (int idx = tid; idx < kR * HD / 8; idx += 64 * kEncWaves) {
    const int ci = idx / (HD / 8), d0 = (idx % (HD / 8)) * 8;
    const uint4 v = *reinterpret_cast<const uint4*>(bh + ci * HD + d0);
    uint16_t* dst = bt + d0 * kBT + swz16(ci);
    dst[0 * kBT] = (uint16_t)(v.x & 0xffffu);
    dst[1 * kBT] = (uint16_t)(v.x >> 16);
    dst[2 * kBT] = (uint16_t)(v.y & 0xffffu);
    dst[3 * kBT] = (uint16_t)(v.y >> 16);
    dst[4 * kBT] = (uint16_t)(v.z & 0xffffu);
    dst[5 * kBT] = (uint16_t)(v.z >> 16);
    dst[6 * kBT] = (uint16_t)(v.w & 0xffffu);
    dst[7 * kBT] = (uint16_t)(v.w >> 16);
  }

  // ---- C^T = B X_o^T, rounded to the stored bf16 coefficients
  f32x16_t c = f32x16_t{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint4 ab = *reinterpret_cast<const uint4*>(bh + col * HD + (2 * ks + hh) * 8);
    const uint4 xv = *reinterpret_cast<const uint4*>(xo + (2 * ks + hh) * 8);
    c = mfma32(ab, xv, c);
  }
  uint4 cb[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    cb[ks] = make_uint4(pack_bf16(c[8 * ks + 0], c[8 * ks + 1]), pack_bf16(c[8 * ks + 2], c[8 * ks + 3]),
                        pack_bf16(c[8 * ks + 4], c[8 * ks + 5]), pack_bf16(c[8 * ks + 6], c[8 * ks + 7]));
  __syncthreads();

  // ---- E^T = X^T - B^T C^T; register r of block mb: dim 32mb + 8(r/4) + 4hh + r%4
  f32x16_t e[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const uint16_t* brow = bt + (32 * mb + col) * kBT + 8 * hh;
    f32x16_t o = mfma32(*reinterpret_cast<const uint4*>(brow), cb[0], f32x16_t{});
    o = mfma32(*reinterpret_cast<const uint4*>(brow + 16), cb[1], o);
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const uint2 xv = *reinterpret_cast<const uint2*>(xr + 32 * mb + 8 * g4 + 4 * hh);
      e[mb][4 * g4 + 0] = dev::bf16_lo(xv.x) - o[4 * g4 + 0];
      e[mb][4 * g4 + 1] = dev::bf16_hi(xv.x) - o[4 * g4 + 1];
      e[mb][4 * g4 + 2] = dev::bf16_lo(xv.y) - o[4 * g4 + 2];
      e[mb][4 * g4 + 3] = dev::bf16_hi(xv.y) - o[4 * g4 + 3];
    }
  }

  if (a.residual_mode) {
    if (!ok || i >= a.n_tokens[b]) return;
    float* er = s.e_out + row * HD;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<float4*>(er + 32 * mb + 8 * g4 + 4 * hh) =
            make_float4(e[mb][4 * g4 + 0], e[mb][4 * g4 + 1], e[mb][4 * g4 + 2], e[mb][4 * g4 + 3]);
    return;
  }

  // ---- Y^T = [U; 0] E^T; step (mb, h2) covers dims 32mb + 16h2 + 8(e/4) + 4hh + e%4
  const uint16_t* urow = s.ubasis + ((size_t)kvh * kRM + (col & 15)) * HD;
  f32x16_t y = f32x16_t{};
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      uint4 hi, lo;
      split8(e[mb], 8 * h2, hi, lo);
      const int d = 32 * mb + 16 * h2 + 4 * hh;
      const uint2 u0 = *reinterpret_cast<const uint2*>(urow + d);
      const uint2 u1 = *reinterpret_cast<const uint2*>(urow + d + 8);
      const uint4 au = col < kRM ? make_uint4(u0.x, u0.y, u1.x, u1.y) : make_uint4(0, 0, 0, 0);
      y = mfma32(au, hi, y);
      y = mfma32(au, lo, y);
    }

  // ---- quantize: this lane holds codes 8(rr/4) + 4hh + rr%4, rr < 8
  const int r = ok ? min((int)a.rank[(size_t)b * a.n + i], kRM) : 0;
  float amax = 0.f;
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const int j = 8 * (rr / 4) + 4 * hh + (rr % 4);
    if (j < r) amax = fmaxf(amax, fabsf(y[rr]));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  const __half s16 = __float2half_rn(amax / 127.f);
  const float sf = __half2float(s16);
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const int j = 8 * (rr / 4) + 4 * hh + (rr % 4);
    int q = 0;
    if (j < r && sf > 0.f) q = (int)fminf(fmaxf(rintf(y[rr] / sf), -127.f), 127.f);
    packed[rr / 4] |= ((uint32_t)q & 0xffu) << (8 * (rr % 4));
  }
  if (!ok) return;
  int8_t* dr = s.d_out + row * kRM;
  *reinterpret_cast<uint32_t*>(dr + 4 * hh) = packed[0];
  *reinterpret_cast<uint32_t*>(dr + 8 + 4 * hh) = packed[1];
  if (hh == 0) s.s_out[row] = __half_as_ushort(s16);
  if (s.c_out) {
    uint16_t* cr = s.c_out + row * kR;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      *reinterpret_cast<uint2*>(cr + 16 * ks + 4 * hh) = make_uint2(cb[ks].x, cb[ks].y);
      *reinterpret_cast<uint2*>(cr + 16 * ks + 8 + 4 * hh) = make_uint2(cb[ks].z, cb[ks].w);
    }
  }
}

// ------------------------------------------------------------ Gram matrices

struct GramParams {
  const void* x[kMaxBasisSets][2];   // [matrix set][source] rows ([B][n][Hkv][hd]); source 1 may be null
  int32_t rows_f32;         // 1: fp32 rows, 0: bf16 rows
  const int32_t* n_tokens;  // [B]
  int32_t n;
  int32_t batch;
  int32_t n_kv_heads;
  float* gram;              // [set][Hkv][hd][hd]
};

// grid (NB (NB+1) / 2 block pairs, Hkv, matrix sets), 256 threads; a set is
// one of K / V of one basis; thread (ti, tj) owns
// G[32bi + ti][32bj + 4tj .. +3]
template <int HD>
__global__ __launch_bounds__(256) void gram_kernel(GramParams a) {
  constexpr int NB = HD / 32;
  __shared__ float xs[2][64][33];
  const int tid = threadIdx.x;
  const int h = blockIdx.y, side = blockIdx.z;   // side: the matrix set
  int pr = blockIdx.x, bi = 0;
  while (pr >= NB - bi) {
    pr -= NB - bi;
    ++bi;
  }
  const int bj = bi + pr;
  const int ti = tid >> 3, tj = tid & 7;
  // staging role: token tid/4 of the tile, 8 dims 8*(tid%4).. of each block
  const int st = tid >> 2, sd = (tid & 3) * 8;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int src = 0; src < 2; ++src) {
    if (!a.x[side][src]) continue;
    for (int b = 0; b < a.batch; ++b) {
      const int cnt = min(max(a.n_tokens[b], 0), a.n);
      for (int t0 = 0; t0 < cnt; t0 += 64) {
        const int t = t0 + st;
        float vi[8], vj[8];
        if (t < cnt) {
          const size_t rowoff = (((size_t)b * a.n + t) * a.n_kv_heads + h) * HD;
          if (a.rows_f32) {
            const float* xr = static_cast<const float*>(a.x[side][src]) + rowoff;
#pragma unroll
            for (int e = 0; e < 8; e += 4) {
              const float4 p = *reinterpret_cast<const float4*>(xr + 32 * bi + sd + e);
              const float4 q = *reinterpret_cast<const float4*>(xr + 32 * bj + sd + e);
              vi[e] = p.x; vi[e + 1] = p.y; vi[e + 2] = p.z; vi[e + 3] = p.w;
              vj[e] = q.x; vj[e + 1] = q.y; vj[e + 2] = q.z; vj[e + 3] = q.w;
            }
          } else {
            const uint16_t* xr = static_cast<const uint16_t*>(a.x[side][src]) + rowoff;
            const uint4 p = *reinterpret_cast<const uint4*>(xr + 32 * bi + sd);
            const uint4 q = *reinterpret_cast<const uint4*>(xr + 32 * bj + sd);
            const uint32_t pw[4] = {p.x, p.y, p.z, p.w}, qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              vi[2 * w] = dev::bf16_lo(pw[w]);
              vi[2 * w + 1] = dev::bf16_hi(pw[w]);
              vj[2 * w] = dev::bf16_lo(qw[w]);
              vj[2 * w + 1] = dev::bf16_hi(qw[w]);
            }
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) vi[e] = vj[e] = 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xs[0][st][sd + e] = vi[e];
          xs[1][st][sd + e] = vj[e];
        }
        __syncthreads();
        const int tn = min(64, cnt - t0);
        for (int u = 0; u < tn; ++u) {
          const float p = xs[0][u][ti];
#pragma unroll
          for (int m = 0; m < 4; ++m) acc[m] = fmaf(p, xs[1][u][4 * tj + m], acc[m]);
        }
      }
    }
  }
  float* g = a.gram + ((size_t)side * a.n_kv_heads + h) * HD * HD;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int r = 32 * bi + ti, cc = 32 * bj + 4 * tj + m;
    g[(size_t)r * HD + cc] = acc[m];
    g[(size_t)cc * HD + r] = acc[m];
  }
}

// --------------------------------------------------- symmetric eigenvectors

struct EigParams {
  const float* gram;        // [set][Hkv][hd][hd]
  int32_t k_out;            // leading eigenvectors to write
  int32_t n_kv_heads;
  uint16_t* out[kMaxBasisSets];   // per set [Hkv][k_out][hd] bf16
  float* evals;             // [set][Hkv][hd] eigenvalues, descending
  int32_t max_sweeps;
};

// one workgroup of 1024 threads per matrix: blockIdx.x = set * Hkv + head.
// Each round rotates 64 disjoint index pairs at once: every 2x2 block
// A[{p_i,q_i}, {p_j,q_j}] becomes J_i^T A J_j (one read and one write of the
// block), and V's columns p_i, q_i rotate.  A pair is rotated only while its
// coupling is above 1e-6 sqrt(a_pp a_qq) and above 2e-7 of the matrix's
// Frobenius norm (about the fp32 rounding level of the entries, so the
// eigenvectors of well-separated leading eigenvalues come out to ~1e-5); the
// sweeps stop after one without a rotation.
template <int HD>
__global__ __launch_bounds__(1024) void eig_kernel(EigParams a) {
  constexpr int NP = HD / 2;           // disjoint pairs per round
  constexpr int LD = HD + 1;
  __shared__ float A[HD * LD];
  __shared__ float V[HD * LD];
  __shared__ float2 rot[NP];           // (c, s) of each pair this round
  __shared__ int2 pq[NP];              // (p, q)
  __shared__ float red[16];
  __shared__ int order[HD];
  __shared__ float sgn[HD];
  __shared__ int rotated;
  __shared__ float floor_abs;

  const int tid = threadIdx.x;
  const int side = blockIdx.x / a.n_kv_heads, h = blockIdx.x % a.n_kv_heads;
  const float* g = a.gram + (size_t)blockIdx.x * HD * HD;
  float ss = 0.f;
  for (int idx = tid; idx < HD * HD; idx += 1024) {
    const int r = idx / HD, c = idx % HD;
    const float v = g[idx];
    A[r * LD + c] = v;
    V[r * LD + c] = r == c ? 1.f : 0.f;
    ss += v * v;
  }
  ss = dev::wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int w = 0; w < 16; ++w) t += red[w];
    floor_abs = 2e-7f * sqrtf(t);
  }
  __syncthreads();

  for (int sweep = 0; sweep < a.max_sweeps; ++sweep) {
    if (tid == 0) rotated = 0;
    for (int round = 0; round < HD - 1; ++round) {
      // round-robin pairing: index HD-1 is fixed, the others rotate
      if (tid < NP) {
        int p, q;
        if (tid == 0) {
          p = round;
          q = HD - 1;
        } else {
          p = (round + tid) % (HD - 1);
          q = (round - tid + (HD - 1)) % (HD - 1);
        }
        const float apq = A[p * LD + q];
        const float app = A[p * LD + p], aqq = A[q * LD + q];
        float c = 1.f, s = 0.f;
        if (fabsf(apq) > fmaxf(1e-6f * sqrtf(fabsf(app * aqq)), floor_abs)) {
          const float tau = (aqq - app) / (2.f * apq);
          const float at = fabsf(tau);
          const float t = (at > 1e15f ? 0.5f / at : 1.f / (at + sqrtf(1.f + tau * tau))) *
                          (tau >= 0.f ? 1.f : -1.f);
          c = 1.f / sqrtf(1.f + t * t);
          s = t * c;
          rotated = 1;
        }
        rot[tid] = make_float2(c, s);
        pq[tid] = make_int2(p, q);
      }
      __syncthreads();
      // A <- J^T A J, one 2x2 block per (i, j); this thread's j is fixed
      // (1024 is a multiple of NP), a wave shares i
      const int j = tid % NP;
      const float2 rj = rot[j];
      const int2 ij = pq[j];
      const float cj = rj.x, sj = rj.y;
      const int pj = ij.x, qj = ij.y;
      for (int i = tid / NP; i < NP; i += 1024 / NP) {
        const float2 ri = rot[i];
        const int2 ii = pq[i];
        const float ci = ri.x, si = ri.y;
        const int pi = ii.x, qi = ii.y;
        const float a00 = A[pi * LD + pj], a01 = A[pi * LD + qj];
        const float a10 = A[qi * LD + pj], a11 = A[qi * LD + qj];
        const float m00 = cj * a00 - sj * a01, m01 = sj * a00 + cj * a01;
        const float m10 = cj * a10 - sj * a11, m11 = sj * a10 + cj * a11;
        // the rotated pair's own coupling is zero by construction; storing
        // the rounded remainder instead would keep a tiny eigenvalue paired
        // with a large one above the relative threshold
        const bool own = i == j && si != 0.f;
        A[pi * LD + pj] = ci * m00 - si * m10;
        A[pi * LD + qj] = own ? 0.f : ci * m01 - si * m11;
        A[qi * LD + pj] = own ? 0.f : si * m00 + ci * m10;
        A[qi * LD + qj] = si * m01 + ci * m11;
      }
      // V <- V J: columns p_j, q_j of every row
      for (int r = tid / NP; r < HD; r += 1024 / NP) {
        const float vp = V[r * LD + pj], vq = V[r * LD + qj];
        V[r * LD + pj] = cj * vp - sj * vq;
        V[r * LD + qj] = sj * vp + cj * vq;
      }
      __syncthreads();
    }
    if (!rotated) break;
    __syncthreads();
  }

  // ---- order by eigenvalue, largest first (ties: lower index first)
  if (tid < HD) {
    const float l = A[tid * LD + tid];
    int pos = 0;
    for (int j = 0; j < HD; ++j) {
      const float lj = A[j * LD + j];
      pos += (lj > l) || (lj == l && j < tid);
    }
    order[pos] = tid;
  }
  __syncthreads();
  if (tid < a.k_out) {
    const int col = order[tid];
    float best = -1.f, v = 0.f;
    for (int d = 0; d < HD; ++d) {
      const float x = V[d * LD + col];
      if (fabsf(x) > best) {
        best = fabsf(x);
        v = x;
      }
    }
    sgn[tid] = v < 0.f ? -1.f : 1.f;
  }
  if (tid < HD) a.evals[(size_t)blockIdx.x * HD + tid] = A[order[tid] * LD + order[tid]];
  __syncthreads();
  uint16_t* o = a.out[side] + (size_t)h * a.k_out * HD;
  for (int idx = tid; idx < a.k_out * HD; idx += 1024) {
    const int k = idx / HD, d = idx % HD;
    const float x = sgn[k] * V[d * LD + order[k]];
    o[idx] = __builtin_bit_cast(uint16_t, (__bf16)x);
  }
}

template <int HD>
int run_encode(const EncodeParams& p, int batch, hipStream_t st) {
  dim3 grid((p.n + 32 * kEncWaves - 1) / (32 * kEncWaves), 2 * p.n_kv_heads, batch);
  hipLaunchKernelGGL(encode_kernel<HD>, grid, dim3(64 * kEncWaves), 0, st, p);
  return (int)hipGetLastError();
}

template <int HD>
int run_gram(const GramParams& p, int n_sets, hipStream_t st) {
  constexpr int NB = HD / 32;
  hipLaunchKernelGGL(gram_kernel<HD>, dim3(NB * (NB + 1) / 2, p.n_kv_heads, n_sets), dim3(256), 0, st, p);
  return (int)hipGetLastError();
}

template <int HD>
int run_eig(const EigParams& p, int n_sets, hipStream_t st) {
  hipLaunchKernelGGL(eig_kernel<HD>, dim3(n_sets * p.n_kv_heads), dim3(1024), 0, st, p);
  return (int)hipGetLastError();
}

}  // namespace

bool encode_shape_supported(int32_t head_dim, int32_t basis_rank, int32_t resid_rank_max) {
  return (head_dim == 64 || head_dim == 128) && basis_rank == kR && resid_rank_max == kRM;
}

int launch_encode(const EncodeLaunch& a, void* stream) {
  EncodeParams p;
  for (int kv = 0; kv < 2; ++kv) {
    EncodeSide& s = p.side[kv];
    s.x = static_cast<const uint16_t*>(a.x[kv]);
    s.xo = static_cast<const uint16_t*>(a.xo[kv]);
    s.basis = static_cast<const uint16_t*>(a.basis[kv]);
    s.ubasis = static_cast<const uint16_t*>(a.ubasis[kv]);
    s.c_out = static_cast<uint16_t*>(a.c_out[kv]);
    s.d_out = static_cast<int8_t*>(a.d_out[kv]);
    s.s_out = static_cast<uint16_t*>(a.s_out[kv]);
    s.e_out = static_cast<float*>(a.e_out[kv]);
  }
  p.rank = a.rank;
  p.n_tokens = a.n_tokens;
  p.n = a.n;
  p.n_kv_heads = a.n_kv_heads;
  p.residual_mode = a.residual_mode;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.head_dim == 64) return run_encode<64>(p, a.batch, st);
  if (a.head_dim == 128) return run_encode<128>(p, a.batch, st);
  return (int)hipErrorInvalidValue;
}

int launch_basis(const BasisLaunch& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.n_sets < 1 || a.n_sets > kMaxBasisSets) return (int)hipErrorInvalidValue;
  GramParams g;
  for (int m = 0; m < a.n_sets; ++m)
    for (int src = 0; src < 2; ++src) g.x[m][src] = a.x[m][src];
  g.rows_f32 = a.rows_f32;
  g.n_tokens = a.n_tokens;
  g.n = a.n;
  g.batch = a.batch;
  g.n_kv_heads = a.n_kv_heads;
  g.gram = a.gram;
  EigParams e;
  e.gram = a.gram;
  e.k_out = a.k_out;
  e.n_kv_heads = a.n_kv_heads;
  for (int m = 0; m < a.n_sets; ++m) e.out[m] = static_cast<uint16_t*>(a.out[m]);
  e.evals = a.evals;
  e.max_sweeps = 20;
  int err;
  if (a.head_dim == 64) {
    if ((err = run_gram<64>(g, a.n_sets, st)) != 0) return err;
    return run_eig<64>(e, a.n_sets, st);
  }
  if (a.head_dim == 128) {
    if ((err = run_gram<128>(g, a.n_sets, st)) != 0) return err;
    return run_eig<128>(e, a.n_sets, st);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace kvs
