// Device helpers shared by the gfx950 kernels: bf16 packing, packed bf16 dot
// products, wave64 reductions over DPP.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvs {
namespace dev {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// a.lo*b.lo + a.hi*b.hi + c for two bf16 pairs (v_dot2c_f32_bf16); bf16
// products are exact in fp32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp(float x) {
  // lanes the control leaves without a source keep x itself
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL,
                                                    ROW_MASK, 0xf, false));
}

// x + (x from the lane CTRL selects), for controls under which every lane has
// a source (quad_perm, row_half_mirror, row_ror): written as a bound_ctrl
// mov_dpp so the compiler folds it into a single v_add_f32_dpp.
template <int CTRL>
__device__ __forceinline__ float add_dpp(float x) {
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Max over the 64 lanes, returned to every lane (uniform).
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));        // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp<0x4E>(x));        // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp<0x124>(x));       // row_ror:4
  x = fmaxf(x, dpp<0x128>(x));       // row_ror:8  -> every lane holds its row's max
  x = fmaxf(x, dpp<0x142, 0xA>(x));  // row_bcast:15 into rows 1 and 3
  x = fmaxf(x, dpp<0x143, 0xC>(x));  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// Sum over the 64 lanes, returned to every lane.
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x124>(x);
  x += dpp<0x128>(x);
  x += dpp<0x142, 0xA>(x);
  x += dpp<0x143, 0xC>(x);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace dev
}  // namespace kvs
