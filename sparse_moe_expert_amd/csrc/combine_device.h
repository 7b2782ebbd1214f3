// Combine of one token: the fixed-order weighted sum of its k expert rows
// plus the shared experts (and the residual in a block forward).  Shared by
// the combine kernel (combine.hip) and the single-launch layer (fused.hip);
// the method and its sources are described in combine.hip.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// Columns [c0, c1) of token t (multiples of 8), by one workgroup (every
// thread of it calls this; it holds one workgroup barrier).  ws / rs:
// kMaxTopK entries of LDS each.  Each output element is summed by one thread
// in the fixed order (residual, shared experts, slots j ascending), so the
// column split does not change the result.
// YF16: y and ysh hold fp16 codes, value = code * 2^e with e from yexp
// [T*k + S*T rows, ceil(H / kHBlock)] (row of the sorted row space).
template <int OK, bool YF16 = false>
__device__ __forceinline__ void combine_token(const void* __restrict__ y_,
                                              const void* __restrict__ ysh_,
                                              const float* __restrict__ w,
                                              const int32_t* __restrict__ inv,
                                              const void* __restrict__ residual,
                                              void* __restrict__ out, int T, int H, int k, int S,
                                              int t, float* ws, long long* rs, int c0, int c1,
                                              const int32_t* __restrict__ yexp = nullptr) {
  const int yeb = (H + kHBlock - 1) / kHBlock;
  const long long R = static_cast<long long>(T) * k;
  // 4 values of row `row` at column c (c % 4 == 0: one exponent block)
  auto load4 = [&](const void* base, long long row, long long drow, int c) __attribute__((always_inline)) {
    if constexpr (YF16) {
      typedef _Float16 h4 __attribute__((ext_vector_type(4)));
      const h4 u = __builtin_nontemporal_load(
          reinterpret_cast<const h4*>(static_cast<const uint16_t*>(base) + drow * H + c));
      const int e = yexp[row * yeb + c / kHBlock];
      const h4 a = u, b = h4{u[2], u[3], u[2], u[3]};
      return float4{ldexpf(static_cast<float>(a[0]), e), ldexpf(static_cast<float>(a[1]), e),
                    ldexpf(static_cast<float>(b[0]), e), ldexpf(static_cast<float>(b[1]), e)};
    } else {
      const f32x4 vv = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + drow * H + c));
      return float4{vv[0], vv[1], vv[2], vv[3]};
    }
  };
  if (threadIdx.x < k) {
    ws[threadIdx.x] = w[static_cast<long long>(t) * k + threadIdx.x];
    rs[threadIdx.x] = inv[static_cast<long long>(t) * k + threadIdx.x];
  }
  __syncthreads();
  if constexpr (YF16) {
    // scaled fp16 y (bf16 layers): 8 columns per thread, so each row is read
    // with one 16-byte load (8 codes inside one exponent block; c0 and c1
    // are multiples of 8).  Same terms in the same order as below.
    static_assert(!YF16 || OK == K_BF16, "scaled fp16 y belongs to bf16 layers");
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    auto add8 = [&](float* acc, const void* base, long long row, long long drow, int c, float wj,
                    bool fma) __attribute__((always_inline)) {
      const h8 u = __builtin_nontemporal_load(
          reinterpret_cast<const h8*>(static_cast<const uint16_t*>(base) + drow * H + c));
      const int e = yexp[row * yeb + c / kHBlock];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = ldexpf(static_cast<float>(u[i]), e);
        acc[i] = fma ? fmaf(wj, v, acc[i]) : acc[i] + v;
      }
    };
    for (int c = c0 + threadIdx.x * 8; c < c1; c += blockDim.x * 8) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (residual) {
        const uint4 r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(residual) +
                                                        static_cast<long long>(t) * H + c);
        const uint32_t r4[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = bf16_to_f32(static_cast<uint16_t>(r4[i] & 0xFFFF));
          acc[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(r4[i] >> 16));
        }
      }
      for (int s = 0; s < S; ++s) {
        const long long srow = static_cast<long long>(s) * T + t;
        add8(acc, ysh_, R + srow, srow, c, 1.f, false);
      }
      for (int j = 0; j < k; ++j) add8(acc, y_, rs[j], rs[j], c, ws[j], true);
      uint4 o;
      o.x = f32_to_bf16(acc[0]) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
      o.y = f32_to_bf16(acc[2]) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
      o.z = f32_to_bf16(acc[4]) | (static_cast<uint32_t>(f32_to_bf16(acc[5])) << 16);
      o.w = f32_to_bf16(acc[6]) | (static_cast<uint32_t>(f32_to_bf16(acc[7])) << 16);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + static_cast<long long>(t) * H + c) = o;
    }
    return;
  }
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
      const long long srow = static_cast<long long>(s) * T + t;
      const float4 v = load4(ysh_, R + srow, srow, c);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    for (int j = 0; j < k; ++j) {
      const float wj = ws[j];
      // y is read exactly once: a nontemporal load keeps it from evicting
      // the rest of the stream from the caches (measured: combine 7% faster)
      const float4 v = load4(y_, rs[j], rs[j], c);
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
