// Token router of the factorized cache: a residual rank per sequence from the
// attention statistics of its current decode query.
//
// DepthWeave-KV ("DepthWeave-KV: Smarter KV Cache Compression by Sharing
// Across Layers and Adapting Per Token", Core Mechanism and Key Concepts):
// the router reads attention entropy and peak scores and gives focused
// (low-entropy, peaked) tokens a higher residual rank, generic ones a lower
// one.  Reading taken here: h = mean over the statistic sets and query heads
// of entropy / ln(n) (n = keys the query saw; h = 0 when n <= 1), p = the
// largest peak probability; rank_focused if h < entropy_focused or
// p >= peak_focused, rank_mid if h < entropy_diffuse, else rank_diffuse.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"

namespace kvs {
namespace {

// one thread per sequence; heads and sets summed in a fixed order
__global__ __launch_bounds__(64) void route_kernel(RouteLaunch a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.batch) return;
  float hsum = 0.f, peak = 0.f;
  for (int s = 0; s < a.n_sets; ++s) {
    const float* row = a.stats + ((size_t)s * a.batch + b) * a.n_q_heads * 2;
    for (int h = 0; h < a.n_q_heads; ++h) {
      hsum += row[2 * h];
      peak = fmaxf(peak, row[2 * h + 1]);
    }
  }
  const int n = a.n_keys[b];
  const float h = n > 1 ? hsum / ((float)(a.n_sets * a.n_q_heads) * logf((float)n)) : 0.f;
  int r;
  if (h < a.entropy_focused || peak >= a.peak_focused)
    r = a.rank_focused;
  else if (h < a.entropy_diffuse)
    r = a.rank_mid;
  else
    r = a.rank_diffuse;
  a.rank_out[b] = (uint8_t)r;
}

}  // namespace

int launch_route(const RouteLaunch& a, void* stream) {
  hipLaunchKernelGGL(route_kernel, dim3((a.batch + 63) / 64), dim3(64), 0,
                     static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

}  // namespace kvs
