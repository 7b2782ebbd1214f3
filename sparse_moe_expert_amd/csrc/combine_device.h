// Combine of one token: the fixed-order weighted sum of its k expert rows
// plus the shared experts (and the residual in a block forward).  Shared by
// the combine kernel (combine.hip) and the single-launch layer (fused.hip);
// the method and its sources are described in combine.hip.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// Columns [c0, c1) of token t (multiples of 4), by one workgroup (every
// thread of it calls this; it holds one workgroup barrier).  ws / rs:
// kMaxTopK entries of LDS each.  Each output element is summed by one thread
// in the fixed order (residual, shared experts, slots j ascending), so the
// column split does not change the result.
template <int OK>
__device__ __forceinline__ void combine_token(const float* __restrict__ y,
                                              const float* __restrict__ ysh,
                                              const float* __restrict__ w,
                                              const int32_t* __restrict__ inv,
                                              const void* __restrict__ residual,
                                              void* __restrict__ out, int T, int H, int k, int S,
                                              int t, float* ws, long long* rs, int c0, int c1) {
  if (threadIdx.x < k) {
    ws[threadIdx.x] = w[static_cast<long long>(t) * k + threadIdx.x];
    rs[threadIdx.x] = inv[static_cast<long long>(t) * k + threadIdx.x];
  }
  __syncthreads();
  for (int c = c0 + threadIdx.x * 4; c < c1; c += blockDim.x * 4) {
    float4 acc = float4{0.f, 0.f, 0.f, 0.f};
    if (residual) {
      // decoder block: the residual stream comes first
      if constexpr (OK == K_BF16) {
        const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(residual) +
                                                        static_cast<long long>(t) * H + c);
        acc = float4{bf16_to_f32(static_cast<uint16_t>(r.x & 0xFFFF)),
                     bf16_to_f32(static_cast<uint16_t>(r.x >> 16)),
                     bf16_to_f32(static_cast<uint16_t>(r.y & 0xFFFF)),
                     bf16_to_f32(static_cast<uint16_t>(r.y >> 16))};
      } else {
        acc = *reinterpret_cast<const float4*>(static_cast<const float*>(residual) +
                                               static_cast<long long>(t) * H + c);
      }
    }
    for (int s = 0; s < S; ++s) {
      const f32x4 vv = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4*>(ysh + (static_cast<long long>(s) * T + t) * H + c));
      const float4 v = float4{vv[0], vv[1], vv[2], vv[3]};
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    for (int j = 0; j < k; ++j) {
      const float wj = ws[j];
      // y is read exactly once: a nontemporal load keeps it from evicting
      // the rest of the stream from the caches (measured: combine 7% faster)
      const f32x4 vv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y + rs[j] * H + c));
      const float4 v = float4{vv[0], vv[1], vv[2], vv[3]};
      acc.x = fmaf(wj, v.x, acc.x);
      acc.y = fmaf(wj, v.y, acc.y);
      acc.z = fmaf(wj, v.z, acc.z);
      acc.w = fmaf(wj, v.w, acc.w);
    }
    if constexpr (OK == K_BF16) {
      uint2 o;
      o.x = f32_to_bf16(acc.x) | (static_cast<uint32_t>(f32_to_bf16(acc.y)) << 16);
      o.y = f32_to_bf16(acc.z) | (static_cast<uint32_t>(f32_to_bf16(acc.w)) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + static_cast<long long>(t) * H + c) = o;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(out) + static_cast<long long>(t) * H + c) = acc;
    }
  }
}

}  // namespace moe
