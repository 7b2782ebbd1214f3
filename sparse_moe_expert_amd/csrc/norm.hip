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
// then a fixed xor-shuffle tree), so the result is deterministic; the second
// pass re-reads the row (an L2 hit) and rounds each output once.  HBM-bound:
// reads T*H and writes T*H elements.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRowsPerBlock = 4;

template <int AK>
__device__ __forceinline__ void load_chunk(const void* base, long long i, float (&v)[8]) {
  if constexpr (AK == K_BF16) {
    const uint4 u = reinterpret_cast<const uint4*>(base)[i];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_to_f32(static_cast<uint16_t>(w[j] & 0xFFFF));
      v[2 * j + 1] = bf16_to_f32(static_cast<uint16_t>(w[j] >> 16));
    }
  } else {
    const float4 f = reinterpret_cast<const float4*>(base)[i];
    v[0] = f.x;
    v[1] = f.y;
    v[2] = f.z;
    v[3] = f.w;
  }
}

template <int AK>
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

  float ss = 0.f;
  for (int q = lane; q < chunks; q += 64) {
    float v[8];
    load_chunk<AK>(h, row + q, v);
#pragma unroll
    for (int j = 0; j < PER; ++j) ss = fmaf(v[j], v[j], ss);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  const float r = 1.0f / sqrtf(ss / static_cast<float>(H) + eps);

  for (int q = lane; q < chunks; q += 64) {
    float v[8], g[8];
    load_chunk<AK>(h, row + q, v);
    load_chunk<AK>(gamma, q, g);
    if constexpr (AK == K_BF16) {
      uint4 o;
      uint32_t* ow = &o.x;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ow[j] = f32_to_bf16(g[2 * j] * (v[2 * j] * r)) |
                (static_cast<uint32_t>(f32_to_bf16(g[2 * j + 1] * (v[2 * j + 1] * r))) << 16);
      reinterpret_cast<uint4*>(out)[row + q] = o;
    } else {
      reinterpret_cast<float4*>(out)[row + q] =
          float4{g[0] * (v[0] * r), g[1] * (v[1] * r), g[2] * (v[2] * r), g[3] * (v[3] * r)};
    }
  }
}

}  // namespace

hipError_t launch_rmsnorm(int act_kind, const void* h, const void* gamma, float eps, void* out,
                          int T, int H, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const int grid = (T + kRowsPerBlock - 1) / kRowsPerBlock;
  if (act_kind == K_BF16)
    hipLaunchKernelGGL(rmsnorm_kernel<K_BF16>, dim3(grid), dim3(64 * kRowsPerBlock), 0, st, h,
                       gamma, eps, out, T, H);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<K_F32>, dim3(grid), dim3(64 * kRowsPerBlock), 0, st, h,
                       gamma, eps, out, T, H);
  return hipGetLastError();
}

}  // namespace moe
