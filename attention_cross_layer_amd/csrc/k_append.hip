// Cache writes: scatter new tokens' K/V of an owner layer into its paged
// slot.  Only owner layers write (CLA page, "Reducing Transformer Key-Value
// Cache Size with Cross-Layer Attention", Methodology: some layers compute
// new K/V, the others reuse it), so the pools hold source layers only.
//
// Page layouts (64 tokens per page, per KV head):
//   K  [8][NCW][8][8][E]   E = elements per 16 bytes, NCW = hd/(8E): chunk
//                          c = 8*cc + w of token t = 8*j + k8 sits at
//                          ((j*NCW + cc)*64 + 8*k8 + w)*E, so the decode's
//                          lane 8*k8 + w loads one contiguous 1 KiB per
//                          (j, cc) and holds an eighth of 8 keys' rows
//   V  [32][hd][2]         token pairs: element (t, d) at (t/2)*hd*2 + d*2 + t%2
// One thread moves one 16-byte chunk of the input row; byte copy, no
// arithmetic on the values.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace kvs {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void append_kernel(AppendLaunch a) {
  constexpr int E = 16 / sizeof(T);
  const int hd = a.head_dim;
  const int nch = hd / E;
  const long long total = (long long)a.batch * a.n * a.n_kv_heads * nch;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int c = (int)(idx % nch);
  long long r = idx / nch;
  const int kvh = (int)(r % a.n_kv_heads);
  r /= a.n_kv_heads;
  const int i = (int)(r % a.n);
  const int b = (int)(r / a.n);
  const int pos = a.start_pos[b] + i;
  if (pos < 0 || pos >= a.max_ctx) return;
  const int page = a.page_table[(size_t)b * a.pages_per_seq + pos / kPage];
  if (page < 0 || page >= a.n_phys_pages) return;
  const int t = pos % kPage;
  const size_t tile = ((size_t)page * a.n_kv_heads + kvh) * kPage * hd + a.slot_offset;
  const size_t src = (((size_t)b * a.n + i) * a.n_kv_heads + kvh) * hd + (size_t)c * E;

  const size_t kdst = (size_t)k_chunk_offset(t, c, nch, E);
  const uint4 kv = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.k) + src);
  *reinterpret_cast<uint4*>(static_cast<T*>(a.k_pool) + tile + kdst) = kv;

  const T* vs = static_cast<const T*>(a.v) + src;
  T* vd = static_cast<T*>(a.v_pool) + tile + (size_t)(t >> 1) * hd * 2 + (t & 1);
#pragma unroll
  for (int e = 0; e < E; ++e) vd[(size_t)(c * E + e) * 2] = vs[e];
}

}  // namespace

int launch_append(const AppendLaunch& a, void* stream) {
  const int E = a.dtype == KVS_F32 ? 4 : 8;
  const long long total = (long long)a.batch * a.n * a.n_kv_heads * (a.head_dim / E);
  if (total == 0) return 0;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.dtype == KVS_F32)
    hipLaunchKernelGGL(append_kernel<float>, dim3(blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(append_kernel<uint16_t>, dim3(blocks), dim3(256), 0, st, a);
  return (int)hipGetLastError();
}

}  // namespace kvs
