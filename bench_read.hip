// Plain streaming read of a device buffer, the ceiling against which bench.py
// sets the decode kernels: every byte read once, nothing computed.  Not part
// of the attention library; bench.py loads it on its own.
//
// Workgroup i reads the contiguous bytes [i*chunk, (i+1)*chunk) of the buffer
// with 16-byte non-temporal loads, U of them per thread in flight; the loaded
// words are folded into one value per thread that is stored only if it
// equals a sentinel, so the loads cannot be dropped.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u4_t;

template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u4_t* __restrict__ p, size_t n16,
                                                          size_t chunk16, uint32_t* sink) {
  const size_t b0 = (size_t)blockIdx.x * chunk16;
  const size_t b1 = b0 + chunk16 < n16 ? b0 + chunk16 : n16;
  uint32_t acc = 0;
  for (size_t i = b0 + threadIdx.x; i < b1; i += (size_t)256 * U) {
    u4_t v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const size_t j = i + (size_t)k * 256;
      v[k] = j < b1 ? __builtin_nontemporal_load(p + j) : u4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int k = 0; k < U; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  if (acc == 0x9E3779B9u) sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) at device pointer `p` with `blocks`
// workgroups of 256 threads and `unroll` (4, 8 or 16) loads in flight per
// thread.  `sink` is device memory of at least blocks * 256 uint32.  With
// `start` / `stop` (hipEvent_t, or both null) the launch records them at the
// kernel's own start and end.  Returns 0, -1 for an unsupported argument, or
// the launch's HIP error code.
template <int U>
static void launch(const u4_t* q, size_t n16, size_t chunk16, uint32_t* sink, int blocks, hipStream_t st,
                   hipEvent_t start, hipEvent_t stop) {
  if (start || stop)
    hipExtLaunchKernelGGL(stream_read_kernel<U>, dim3(blocks), dim3(256), 0, st, start, stop, 0, q, n16,
                          chunk16, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<U>, dim3(blocks), dim3(256), 0, st, q, n16, chunk16, sink);
}

extern "C" __attribute__((visibility("default"))) int stream_read(const void* p, size_t bytes,
                                                                  uint32_t* sink, int blocks,
                                                                  int unroll, void* stream,
                                                                  void* start, void* stop) {
  if (!p || !sink || blocks <= 0 || bytes % 16 != 0) return -1;
  const size_t n16 = bytes / 16;
  const size_t chunk16 = (n16 + blocks - 1) / blocks;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = static_cast<hipEvent_t>(start), e1 = static_cast<hipEvent_t>(stop);
  const u4_t* q = static_cast<const u4_t*>(p);
  switch (unroll) {
    case 4: launch<4>(q, n16, chunk16, sink, blocks, st, e0, e1); break;
    case 8: launch<8>(q, n16, chunk16, sink, blocks, st, e0, e1); break;
    case 16: launch<16>(q, n16, chunk16, sink, blocks, st, e0, e1); break;
    default: return -1;
  }
  return (int)hipGetLastError();
}
