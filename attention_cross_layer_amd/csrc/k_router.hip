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

#include "common.h"
#include "internal.h"

namespace kvs {
namespace {

// one workgroup per sequence: threads take (set, head) entries in a fixed
// stride, then a fixed-order reduction (wave DPP, then the 4 waves)
__global__ __launch_bounds__(256) void route_kernel(RouteLaunch a) {
  __shared__ float part_h[4], part_p[4];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int per_set = a.n_q_heads;
  const int total = a.n_sets * per_set;
  float hsum = 0.f, peak = 0.f;
  for (int e = tid; e < total; e += 256) {
    const int s = e / per_set, h = e % per_set;
    const float* row = a.stats + (((size_t)s * a.batch + b) * a.n_q_heads + h) * 2;
    hsum += row[0];
    peak = fmaxf(peak, row[1]);
  }
  hsum = dev::wave_sum(hsum);
  peak = dev::wave_max(peak);
  if ((tid & 63) == 0) {
    part_h[tid >> 6] = hsum;
    part_p[tid >> 6] = peak;
  }
  __syncthreads();
  if (tid != 0) return;
  hsum = (part_h[0] + part_h[1]) + (part_h[2] + part_h[3]);
  peak = fmaxf(fmaxf(part_p[0], part_p[1]), fmaxf(part_p[2], part_p[3]));
  const int n = a.n_keys[b];
  const float h = n > 1 ? hsum / ((float)total * logf((float)n)) : 0.f;
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
  hipLaunchKernelGGL(route_kernel, dim3(a.batch), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

}  // namespace kvs
