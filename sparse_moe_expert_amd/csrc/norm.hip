// RMSNorm of the decoder block around the MoE layer (gfx950).
//
// out[t, c] = gamma[c] * h[t, c] / sqrt(mean_c' h[t, c']^2 + eps): the
// "Residual + RMSNorm" box before the MoE FFN in the single-layer figure of
// the Deep Dive (§3.3); the variance is computed in fp32 and then rsqrt and
// the weight are applied, as the Transformers Dots1 article describes
// Dots1RMSNorm.
//
// One wavefront per row.  Lanes read 16-byte chunks (8 bf16 or 4 fp32) at
// stride 64 chunks, so each load instruction covers 1 KB of the row.  The
// sum of squares runs in fp32 in a fixed order (per lane in chunk order,
// then a fixed xor-shuffle tree), so the result is deterministic.  Rows up
// to 8192 bf16 (4096 fp32) stay in registers for the output pass; each
// output is rounded once.  HBM-bound: reads T*H and writes T*H elements.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRowsPerBlock = 4;

template <int AK>
__device__ __forceinline__ void unpack_chunk(const uint4 u, float (&v)[8]) {
  if constexpr (AK == K_BF16) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_to_f32(static_cast<uint16_t>(w[j] & 0xFFFF));
      v[2 * j + 1] = bf16_to_f32(static_cast<uint16_t>(w[j] >> 16));
    }
  } else {
    v[0] = __uint_as_float(u.x);
    v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z);
    v[3] = __uint_as_float(u.w);
  }
}

// Rows of up to 64 * RC chunks stay in registers between the sum of squares
// and the output (one HBM read of h); longer rows are read twice.
template <int AK, int RC>
__global__ __launch_bounds__(64 * kRowsPerBlock) void rmsnorm_kernel(const void* __restrict__ h,
                                                                     const void* __restrict__ gamma,
                                                                     float eps,
                                                                     void* __restrict__ out, int T,
                                                                     int H) {
  constexpr int PER = (AK == K_BF16) ? 8 : 4;  // elements per 16-byte chunk
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave
  const int chunks = H / PER;
  const long long row = static_cast<long long>(t) * chunks;
  const bool resident = chunks <= 64 * RC;

  uint4 raw[RC];
  float ss = 0.f;
  auto sumsq = [&](const uint4 u) {
    float x[8];
    unpack_chunk<AK>(u, x);
#pragma unroll
    for (int j = 0; j < PER; ++j) ss = fmaf(x[j], x[j], ss);
  };
  const uint4* hv = reinterpret_cast<const uint4*>(h) + row;
  if (resident) {
#pragma unroll
    for (int i = 0; i < RC; ++i) {
      const int q = lane + 64 * i;
      raw[i] = q < chunks ? hv[q] : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < RC; ++i)
      if (lane + 64 * i < chunks) sumsq(raw[i]);
  } else {
    for (int q = lane; q < chunks; q += 64) sumsq(hv[q]);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  const float r = 1.0f / sqrtf(ss / static_cast<float>(H) + eps);

  auto store = [&](int q, const uint4 u) {
    float x[8], g[8];
    unpack_chunk<AK>(u, x);
    unpack_chunk<AK>(reinterpret_cast<const uint4*>(gamma)[q], g);
    if constexpr (AK == K_BF16) {
      uint4 o;
      uint32_t* ow = &o.x;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ow[j] = f32_to_bf16(g[2 * j] * (x[2 * j] * r)) |
                (static_cast<uint32_t>(f32_to_bf16(g[2 * j + 1] * (x[2 * j + 1] * r))) << 16);
      reinterpret_cast<uint4*>(out)[row + q] = o;
    } else {
      reinterpret_cast<float4*>(out)[row + q] =
          float4{g[0] * (x[0] * r), g[1] * (x[1] * r), g[2] * (x[2] * r), g[3] * (x[3] * r)};
    }
  };
  if (resident) {
#pragma unroll
    for (int i = 0; i < RC; ++i) {
      const int q = lane + 64 * i;
      if (q < chunks) store(q, raw[i]);
    }
  } else {
    for (int q = lane; q < chunks; q += 64) store(q, hv[q]);
  }
}

}  // namespace

hipError_t launch_rmsnorm(int act_kind, const void* h, const void* gamma, float eps, void* out,
                          int T, int H, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const int grid = (T + kRowsPerBlock - 1) / kRowsPerBlock;
  if (act_kind == K_BF16)
    hipLaunchKernelGGL((rmsnorm_kernel<K_BF16, 16>), dim3(grid), dim3(64 * kRowsPerBlock), 0, st,
                       h, gamma, eps, out, T, H);
  else
    hipLaunchKernelGGL((rmsnorm_kernel<K_F32, 16>), dim3(grid), dim3(64 * kRowsPerBlock), 0, st,
                       h, gamma, eps, out, T, H);
  return hipGetLastError();
}

}  // namespace moe
