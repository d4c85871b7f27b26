// Device helpers shared by the gfx950 kernels: bf16 packing, packed bf16 dot
// products, wave64 reductions over DPP.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace kvs {

// Launch of a main attention kernel: with the caller's timing events
// attached (hipExtLaunchKernel records them at the kernel's start and end)
// when kvs_time_next_launch armed them, else a plain launch.
template <typename F, typename... Args>
inline void launch_main(const KernelEvents& ev, F kernel, dim3 grid, dim3 block, hipStream_t st,
                        Args... args) {
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, static_cast<hipEvent_t>(ev.start),
                          static_cast<hipEvent_t>(ev.stop), 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}

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

// IEEE 754-2019 maximum (a NaN operand gives NaN, -0 < +0).  gfx950 has it as
// v_maximum3_f32, which needs none of the quieting copies that fmaxf takes
// under IEEE mode; max3(m, a, b) is one instruction.
__device__ __forceinline__ float fmax_ieee(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float fmax3_ieee(float m, float a, float b) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, a), b);
}

// Buffer loads through a resource over [base, base + bytes): an offset at or
// past the end returns zeros and moves no data, so a load that may be absent
// is issued unconditionally with offset kOOB instead of under a branch.
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Cache policy of a load: kCached, or kStream (the non-temporal bit) for
// data a kernel reads exactly once, such as the pages a decode streams, so
// that their lines do not displace what is reused.  Measured on the decode
// kernels (one box, cache flushed): the 64K-context hd-128 layer call 174 ->
// 158 us, the factorized 64K call 32.6 -> 30.1 us.  Loads that gather
// 4-byte pieces of lines that neighbouring lanes read later (the hd-64 MFMA
// decode's V operand) stay cached: streaming them measured slower.
constexpr int kCached = 0;
constexpr int kStream = 2;

template <int CPOL = kCached>
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u4_t;
  const u4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, CPOL);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <int CPOL = kCached>
__device__ __forceinline__ uint2 ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef __attribute__((ext_vector_type(2))) uint32_t u2v_t;
  const u2v_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, CPOL);
  return make_uint2(v.x, v.y);
}
template <int CPOL = kCached>
__device__ __forceinline__ uint32_t ld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, CPOL);
}
template <int CPOL = kCached>
__device__ __forceinline__ uint32_t ld2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, CPOL);
}
// 16 bytes through a plain pointer with the non-temporal policy
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u4_t;
  const u4_t v = __builtin_nontemporal_load(reinterpret_cast<const u4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace dev
}  // namespace kvs
