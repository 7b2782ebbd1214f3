// Device-side helpers for the gfx950 kernels of libmoe.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// SiLU(g) * u of the SwiGLU epilogues, g / (1 + e^-g) * u, with the hardware
// exponential and reciprocal (each within a few ulp in fp32: far below the
// bf16 or e4m3 rounding of h that follows, and of the fp32 tolerance).
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Order-preserving map of an fp32 to uint32 (larger float -> larger uint).
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_from_order_key(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  lo = __shfl_xor(lo, m, 64);
  hi = __shfl_xor(hi, m, 64);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Largest of non-negative floats across lanes, by DPP moves inside each
// 16-lane row (quad xor 1, quad xor 2, half-row mirror, row mirror: no LDS
// round trip), then lane reads across rows.  Non-negative floats order as
// their bit patterns, so the cross-row maximum is an integer one.
template <int CTRL>
__device__ __forceinline__ float dpp_fmax(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false)));
}
// every lane gets the maximum over its 16-lane row
__device__ __forceinline__ float row16_fmax(float v) {
  v = dpp_fmax<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_fmax<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_fmax<0x141>(v);  // row_half_mirror
  return dpp_fmax<0x140>(v);  // row_mirror
}
// every lane gets the maximum over its half wave (lanes 0-31 or 32-63); v >= 0
__device__ __forceinline__ float half_wave_fmax_nonneg(float v) {
  const int r = __float_as_int(row16_fmax(v));
  const uint32_t lo = max(static_cast<uint32_t>(__builtin_amdgcn_readlane(r, 0)),
                          static_cast<uint32_t>(__builtin_amdgcn_readlane(r, 16)));
  const uint32_t hi = max(static_cast<uint32_t>(__builtin_amdgcn_readlane(r, 32)),
                          static_cast<uint32_t>(__builtin_amdgcn_readlane(r, 48)));
  return __uint_as_float((threadIdx.x & 32) ? hi : lo);
}
// the maximum over the wave, the same in every lane; v >= 0
__device__ __forceinline__ float wave_fmax_nonneg(float v) {
  const int r = __float_as_int(row16_fmax(v));
  const uint32_t m = max(max(static_cast<uint32_t>(__builtin_amdgcn_readlane(r, 0)),
                             static_cast<uint32_t>(__builtin_amdgcn_readlane(r, 16))),
                         max(static_cast<uint32_t>(__builtin_amdgcn_readlane(r, 32)),
                             static_cast<uint32_t>(__builtin_amdgcn_readlane(r, 48))));
  return __uint_as_float(m);
}

// Four fp32 -> four OCP e4m3 codes (round to nearest even), packed little-endian.
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return static_cast<uint32_t>(r);
}

}  // namespace moe
