// Causal (or full) prefill-chunk attention over the shared paged K/V cache,
// on bf16 MFMA with fp32 accumulation.
//
// A chunk of n queries per sequence sits at the last n positions: query i of
// sequence b is at P = seq_len[b] - n + i and, causal, sees keys 0..P.  The
// keys of the chunk itself were appended first, so the whole key range comes
// from the cache of the layer's source slot(s) (CLA page, "Reducing
// Transformer Key-Value Cache Size with Cross-Layer Attention", Methodology:
// reusing layers read the source layer's K/V).  A two-source layer reads the
// DepthGraft mix K~ = w0 K_s0 + w1 K_s1 ("DepthGraft: Structural
// Regularization through Hierarchical Cross-Layer KV Reconstruction",
// Abstract), formed in fp32 while a tile is staged and rounded to fp16 (11
// significant bits); such a layer's products run on the fp16 MFMA, with its
// queries (bf16, converted exactly) and probabilities in fp16 as well.
// DepthGraft's owner layers are the only ones that need prefill for all
// prompt tokens (the Abstract's "prefill early completion").
//
// Decomposition (gfx950, v_mfma_f32_32x32x16_bf16; lane l of A/B holds row or
// column l%32 and k = 8*(l/32)+e; result register r of lane l is row
// 8*(r/4) + 4*(l/32) + r%4, column l%32):
//   workgroup = NW = 8 waves sharing one KV head (one workgroup per CU, two
//   waves per SIMD, every staged tile serving 256 query rows): HW = min(G, 4)
//   query heads x NW/HW blocks of 32 consecutive query positions; each wave
//   owns 32 query rows of one head.  Per 64-key tile (one cache page):
//     staging  all threads copy the K page into LDS as [64 keys][hd]
//              (16-byte chunks XOR-swizzled by key) and the V page as V^T
//              [hd][64+4 keys]; keys past the sequence end are zeroed (cache
//              memory there is unwritten).  Two register stages hold the
//              global loads of the next two tiles while the current tile is
//              computed; one barrier per tile (double-buffered LDS).
//     S^T = K Q^T   16 MFMAs (2 blocks of 32 keys x hd/16 steps): each lane
//              ends up with 32 scores of one query row (its column).
//     softmax  online, per query row, in registers; the two lanes of a row
//              exchange their tile maximum with one cross-half shuffle.
//     O^T += V^T P^T   the probabilities, rounded to bf16, are the B operand
//              straight from the S^T registers; the MFMA's k index runs over
//              keys in the order those registers hold them, and V^T is read
//              from LDS in the same order.
//   Work order: workgroups with later query positions (more causal keys)
//   are dispatched first; the KV head is the fastest-varying index so each
//   XCD's L2 serves the K/V of one head.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "common.h"
#include "internal.h"

namespace kvs {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int kRows = 32;        // query rows per wave
constexpr int kVRow = 64 + 8;    // V^T row pitch in keys (144 B: an odd number of 16-byte units)

// Key position inside V^T rows: each 16-key group has its quads 1 and 2
// swapped, so a lane's 8 keys 16sp + 8(e/4) + 4hh + e%4 (the order of the
// probabilities in its B operand) are one 16-byte read.
__device__ __forceinline__ int swz16(int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); }
// LDS row of dim d in V^T: d with its low 3 bits flipped by bits 3..5, so
// that the staging writes of 8 consecutive threads (dims 4L + i) and the
// reads of 8 consecutive lanes (dims 32mb + col) land in 8 different 16-byte
// bank groups (row pitch 9 units).
__device__ __forceinline__ int vrow_of(int d) { return d ^ ((d >> 3) & 7); }

struct PrefillParams {
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* page_table;
  int32_t pages_per_seq;
  int32_t n_phys_pages;
  int32_t n_kv_heads;
  int32_t n_q_heads;
  int64_t slot_stride;  // elements
  int32_t slot0, slot1;
  float w0, w1;
  const uint16_t* q;    // [B][n][Hq][hd]
  int32_t n;
  const int32_t* seq_len;
  int32_t max_ctx;
  int32_t causal;
  int32_t key_excl;     // 1: query at P sees keys 0..P-1 (source above the layer)
  float scale_log2;
  void* out;            // [B][n][Hq][hd]
  int32_t out_bf16;
  int32_t n_pos_groups; // workgroups along query positions
  int32_t head_groups;  // G / HW
};

__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;

__device__ __forceinline__ f32x16_t mfma32h(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                0, 0, 0);
}

// two floats -> packed fp16 pair, round to nearest even
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  const f16x2_t v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// a.lo*b.lo + a.hi*b.hi + c for two fp16 pairs (v_dot2_f32_f16)
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}

// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;   // (1.0, 1.0) in bf16
constexpr uint32_t kOnesF16x2 = 0x3C003C00u;    // (1.0, 1.0) in fp16
constexpr float kBumpLog2 = 8.f;                // lazy-maximum slack (log2 units)

// w0*a + w1*b per bf16 element of two 16-byte chunks, formed in fp32 and
// rounded to fp16 (11 significant bits against bf16's 8).
__device__ __forceinline__ uint4 mix_chunk_f16(const uint4& a, const uint4& b, float w0, float w1) {
  uint4 r;
  const uint32_t* pa = &a.x;
  const uint32_t* pb = &b.x;
  uint32_t* pr = &r.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = fmaf(w0, dev::bf16_lo(pa[i]), w1 * dev::bf16_lo(pb[i]));
    const float hi = fmaf(w0, dev::bf16_hi(pa[i]), w1 * dev::bf16_hi(pb[i]));
    pr[i] = pack_f16(lo, hi);
  }
  return r;
}

// eight bf16 values -> eight fp16 values (exact for magnitudes in
// [2^-14, 65504]; smaller ones keep fp16's subnormal precision)
__device__ __forceinline__ uint4 bf16x8_to_f16(const uint4& x) {
  auto cv = [](uint32_t w) { return pack_f16(dev::bf16_lo(w), dev::bf16_hi(w)); };
  return make_uint4(cv(x.x), cv(x.y), cv(x.z), cv(x.w));
}

// One MFMA of the kernel: bf16 operands for one-source layers, fp16 for
// two-source layers (whose tiles are the fp16 mix).
template <int NSRC>
__device__ __forceinline__ f32x16_t mfma_op(const uint4& a, const uint4& b, f32x16_t c) {
  if constexpr (NSRC == 2)
    return mfma32h(a, b, c);
  else
    return mfma32(a, b, c);
}

// Waves per workgroup.  Eight waves sharing each staged tile halve the
// staging loads and LDS writes per MFMA against two 4-wave workgroups per CU
// (hd 128: 395 vs 427 us per DepthGraft chunk layer; hd 64: 144 vs 159 us
// for a 2048-query chunk of the 1.1B shape).
constexpr int kWaves = 8;

template <int HD, int G, int NSRC>
__global__ __launch_bounds__(64 * kWaves, 1) void prefill_kernel(PrefillParams a) {
  constexpr int NW = kWaves;
  constexpr int NT = 64 * NW;
  constexpr int HW = G < 4 ? G : 4;          // heads per workgroup
  constexpr int PB = NW / HW;                // 32-row position blocks per workgroup
  constexpr int NCH = HD / 8;                // 16-byte chunks per key row
  constexpr int KS = HD / 16;                // MFMA k-steps over the head dim
  constexpr int MB = HD / 32;                // 32-dim blocks of O^T
  constexpr int KCH = 64 * NCH / NT;         // K chunks staged per thread per source
  constexpr int VCH = KCH;                   // V chunks staged per thread per source
  static_assert(VCH >= 1 && VCH <= 4, "V staging stores 1 to 4 dwords per dim row");

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][64 * HD];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][HD * kVRow];
  // Two sources: the tiles hold the fp32 mix rounded to fp16, and the
  // queries and probabilities enter those products as fp16 too.  Rounding
  // the mixed tiles to bf16 moved single outputs by up to 1e-2 where a few
  // keys dominate a row (mostly through the scores), at the edge of the
  // error bound; fp16 keeps 3 more bits in one product per step.

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

  // ---- this lane's query row (MFMA column) and its key limit
  const int row = i0 + col;
  const bool row_ok = row < n;
  const int pos = T - n + row;                               // absolute position
  const int row_kend = !row_ok ? 0 : (a.causal ? max(min(T, pos + 1 - a.key_excl), 0) : T);
  // tiles below this one need no key mask in any row of the wave (the wave's
  // first row has the smallest key limit; rows past n make the wave masked)
  const int wave_kend = (i0 + kRows <= n) ? (a.causal ? max(min(T, T - n + i0 + 1 - a.key_excl), 0) : T) : 0;
  const int unmasked_tiles = wave_kend / 64;

  uint4 qreg[KS];
  {
    const int qrow = row_ok ? row : (n - 1);                 // stay in bounds
    const uint16_t* qp = a.q + (((size_t)b * n + qrow) * a.n_q_heads + head) * HD;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qreg[ks] = *reinterpret_cast<const uint4*>(qp + (2 * ks + hh) * 8);
      if constexpr (NSRC == 2) qreg[ks] = bf16x8_to_f16(qreg[ks]);
    }
  }

  const int32_t* pt = a.page_table + (size_t)b * a.pages_per_seq;
  const int64_t so0 = (int64_t)a.slot0 * a.slot_stride;
  const int64_t so1 = (int64_t)a.slot1 * a.slot_stride;

  struct Stage {
    uint4 k[NSRC][KCH], v[NSRC][VCH];
    int entry;                               // page-table entry of the staged tile
  };
  Stage sa, sb;                              // register stages of alternate tiles
  // V chunk u of this thread: key pair (tid / (HD/4)) * VCH + u, dims
  // 4 * (tid % (HD/4)) .. +3 (16-byte unit pair * HD/4 + dim group)
  auto v_chunk = [&](int u) { return ((tid / (HD / 4)) * VCH + u) * (HD / 4) + tid % (HD / 4); };
  auto load_tile = [&](int entry, Stage& st) {
    st.entry = entry;
    // an entry outside [0, n_phys_pages) reads page 0 in its place; store_tile
    // zeroes that tile's values and tile_step gives its keys no weight, so the
    // keys of such a page are skipped, as the decode skips them
    const int page = (unsigned)entry < (unsigned)a.n_phys_pages ? entry : 0;
    const int64_t tile = ((int64_t)page * a.n_kv_heads + kvh) * (64 * HD);
#pragma unroll
    for (int s = 0; s < NSRC; ++s) {
      const uint16_t* kp = a.k_pool + (s == 0 ? so0 : so1) + tile;
      const uint16_t* vp = a.v_pool + (s == 0 ? so0 : so1) + tile;
#pragma unroll
      for (int u = 0; u < KCH; ++u) st.k[s][u] = *reinterpret_cast<const uint4*>(kp + (tid + NT * u) * 8);
#pragma unroll
      for (int u = 0; u < VCH; ++u) st.v[s][u] = *reinterpret_cast<const uint4*>(vp + v_chunk(u) * 8);
    }
  };
  auto store_tile = [&](int t, int entry, int buf, const Stage& st) {
    const int key0 = t * 64;
    const bool page_ok = (unsigned)entry < (unsigned)a.n_phys_pages;
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      // cache layout chunk index -> (key, chunk)
      const int qi = tid + NT * u;
      constexpr int NCW = NCH / kWays, KPP = 64 / kWays;   // chunks per lane, keys per pass
      const int j = qi / (NCW * 64), cc = (qi / 64) % NCW, kk = (qi % 64) / kWays, w = qi % kWays;
      const int key = KPP * j + kk, c = kWays * cc + w;
      uint4 v = NSRC == 2 ? mix_chunk_f16(st.k[0][u], st.k[NSRC - 1][u], a.w0, a.w1) : st.k[0][u];
      *reinterpret_cast<uint4*>(&k_lds[buf][key * HD + ((c ^ (key & (NCH - 1))) * 8)]) = v;
    }
    // V^T: this thread holds VCH consecutive key pairs of its 4 dims (a
    // dword = one dim of a key pair), so each dim row takes one VCH-dword
    // store, pairs in key order
    {
      const int L = tid % (HD / 4), q = tid / (HD / 4);
      uint32_t w[4][VCH];
#pragma unroll
      for (int u = 0; u < VCH; ++u) {
        const uint4 v = NSRC == 2 ? mix_chunk_f16(st.v[0][u], st.v[NSRC - 1][u], a.w0, a.w1) : st.v[0][u];
        w[0][u] = v.x;
        w[1][u] = v.y;
        w[2][u] = v.z;
        w[3][u] = v.w;
      }
      if (!(page_ok && key0 + 64 <= T)) {                       // a page not wholly in range (uniform)
#pragma unroll
        for (int u = 0; u < VCH; ++u) {
          const int k0 = key0 + 2 * (q * VCH + u);              // keys k0, k0+1
          const uint32_t mk = (page_ok && k0 < T ? 0x0000ffffu : 0u) | (page_ok && k0 + 1 < T ? 0xffff0000u : 0u);
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i][u] &= mk;
        }
      }
      // one dword store per (dim row, key pair); pairs in key order, each
      // group of two at swz16 of its first key
      uint16_t* dst = &v_lds[buf][0];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t* row = reinterpret_cast<uint32_t*>(dst + vrow_of(4 * L + i) * kVRow);
        const int k0 = 2 * VCH * q;                          // first of this thread's keys
#pragma unroll
        for (int u = 0; u < VCH; ++u) row[swz16(k0 + 2 * u) / 2] = w[i][u];
      }
    }
  };

  f32x16_t o[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) o[mb] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;
  const float bump_gap = kBumpLog2 / a.scale_log2;   // in raw score units

  // Register stages: tile t's loads were issued two tiles before its LDS
  // stores (two stages, the loop unrolled by two so each is static).
  // Page-table entries are read a tile before the loads that use them.
  int pt_a = n_tiles > 2 ? pt[2] : 0;
  if (n_tiles > 0) load_tile(pt[0], sa);
  if (n_tiles > 1) load_tile(pt[1], sb);
  auto tile_step = [&](int t, Stage& st) {
    const int buf = t & 1;
    const int pt_b = pt[min(t + 3, n_tiles - 1)];
    const bool tile_ok = (unsigned)st.entry < (unsigned)a.n_phys_pages;   // uniform
    store_tile(t, st.entry, buf, st);
    if (t + 2 < n_tiles) load_tile(pt_a, st);
    pt_a = pt_b;
    __syncthreads();
    // ---- S^T = K Q^T: two 32-key blocks
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16_t{};
      const int key = 32 * kb + col;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = 2 * ks + hh;
        const uint4 kv = *reinterpret_cast<const uint4*>(&k_lds[buf][key * HD + ((c ^ (key & (NCH - 1))) * 8)]);
        s[kb] = mfma_op<NSRC>(kv, qreg[ks], s[kb]);
      }
    }
    // the K operand reads run four ahead of the MFMAs that take them (two
    // ahead with two sources, whose tile stages hold twice the registers)
    constexpr int NQK = 2 * KS;               // score MFMAs (and K reads) per tile
    constexpr int AHEAD = NSRC == 2 ? 2 : 4;
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
    for (int i = 0; i < NQK - AHEAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);

    // ---- online softmax for this lane's query row, on raw scores (the
    // positive scale commutes with the max); keys past the row's limit are
    // masked only in tiles that reach a limit, and every key of a tile whose
    // page-table entry is out of range
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
    float lt = 0.f;
    uint4 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = dev::fast_exp2(fmaf(s[kb][8 * sh + e], a.scale_log2, neg));
        uint4 w;
        if constexpr (NSRC == 2) {
          // p <= 2^kBumpLog2: in fp16 range
          w.x = pack_f16(p[0], p[1]);
          w.y = pack_f16(p[2], p[3]);
          w.z = pack_f16(p[4], p[5]);
          w.w = pack_f16(p[6], p[7]);
          lt = dot2_f16(w.x, kOnesF16x2, lt);
          lt = dot2_f16(w.y, kOnesF16x2, lt);
          lt = dot2_f16(w.z, kOnesF16x2, lt);
          lt = dot2_f16(w.w, kOnesF16x2, lt);
        } else {
          w.x = pack_bf16(p[0], p[1]);
          w.y = pack_bf16(p[2], p[3]);
          w.z = pack_bf16(p[4], p[5]);
          w.w = pack_bf16(p[6], p[7]);
          // the running sum adds the same rounded probabilities (dot with ones)
          lt = dev::dot2_bf16(w.x, kOnesBf16x2, lt);
          lt = dev::dot2_bf16(w.y, kOnesBf16x2, lt);
          lt = dev::dot2_bf16(w.z, kOnesBf16x2, lt);
          lt = dev::dot2_bf16(w.w, kOnesBf16x2, lt);
        }
        pb[2 * kb + sh] = w;
      }
    l_run = fmaf(l_run, alpha, lt);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[mb][r] *= alpha;
    }

    // ---- O^T += V^T P^T; step sp covers keys 16sp + 8(e/4) + 4hh + e%4
#pragma unroll
    for (int sp = 0; sp < 4; ++sp)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int d = 32 * mb + col;
        const uint16_t* vrow = &v_lds[buf][vrow_of(d) * kVRow + 16 * sp + 8 * hh];
        o[mb] = mfma_op<NSRC>(*reinterpret_cast<const uint4*>(vrow), pb[sp], o[mb]);
      }
  };
  for (int t = 0; t < n_tiles; t += 2) {
    tile_step(t, sa);
    if (t + 1 < n_tiles) tile_step(t + 1, sb);
  }

  // ---- normalise and store this lane's row: dims 32mb + 8(r/4) + 4hh + r%4
  const float l_row = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
  const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
  const size_t obase = (((size_t)b * n + row) * a.n_q_heads + head) * HD;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = 32 * mb + 8 * g4 + 4 * hh;
      const float v0 = o[mb][4 * g4 + 0] * inv, v1 = o[mb][4 * g4 + 1] * inv;
      const float v2 = o[mb][4 * g4 + 2] * inv, v3 = o[mb][4 * g4 + 3] * inv;
      if (a.out_bf16) {
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + obase + d) =
            make_uint2(pack_bf16(v0, v1), pack_bf16(v2, v3));
      } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + obase + d) =
            make_float4(v0, v1, v2, v3);
      }
    }
}

template <int HD, int G, int NSRC>
int run_prefill(PrefillParams p, int B, hipStream_t st, const KernelEvents& ev) {
  constexpr int HW = G < 4 ? G : 4;
  constexpr int PB = kWaves / HW;
  p.head_groups = G / HW;
  p.n_pos_groups = (p.n + PB * kRows - 1) / (PB * kRows);
  dim3 grid(p.n_pos_groups * p.head_groups * p.n_kv_heads, B);
  launch_main(ev, prefill_kernel<HD, G, NSRC>, grid, dim3(64 * kWaves), st, p);
  return (int)hipGetLastError();
}

typedef int (*PrefillFn)(PrefillParams, int, hipStream_t, const KernelEvents&);

// Group sizes a plan can reach: the decode kernels take two sources up to
// G = 8 and one source up to G = 16 (G = 32 at hd 64 only), so the prefill
// is built for the same shapes and no others.
template <int HD, int NSRC>
PrefillFn pick_g(int G) {
  switch (G) {
    case 1: return run_prefill<HD, 1, NSRC>;
    case 2: return run_prefill<HD, 2, NSRC>;
    case 4: return run_prefill<HD, 4, NSRC>;
    case 8: return run_prefill<HD, 8, NSRC>;
    case 16:
      if constexpr (NSRC == 1) return run_prefill<HD, 16, 1>;
      return nullptr;
    case 32:
      if constexpr (NSRC == 1 && HD == 64) return run_prefill<64, 32, 1>;
      return nullptr;
    default: return nullptr;
  }
}

PrefillFn pick(int hd, int G, int nsrc) {
  if (hd == 64) return nsrc == 1 ? pick_g<64, 1>(G) : pick_g<64, 2>(G);
  if (hd == 128) return nsrc == 1 ? pick_g<128, 1>(G) : pick_g<128, 2>(G);
  return nullptr;
}

}  // namespace

bool prefill_shape_supported(int32_t head_dim, int32_t group, int32_t n_src) {
  return pick(head_dim, group, n_src) != nullptr;
}

int launch_prefill(const PrefillLaunch& a, void* stream) {
  PrefillFn fn = pick(a.head_dim, a.n_q_heads / a.n_kv_heads, a.n_src);
  if (!fn) return (int)hipErrorInvalidValue;
  PrefillParams p;
  p.k_pool = static_cast<const uint16_t*>(a.k_pool);
  p.v_pool = static_cast<const uint16_t*>(a.v_pool);
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
