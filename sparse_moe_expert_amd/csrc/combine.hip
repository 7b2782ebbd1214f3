// Combine and FP8 activation quantisation (gfx950).
//
// Combine: out[t] = Σ_s y_shared[s, t] + Σ_j w[t, j] * y_sorted[inv[t*k + j]],
// the weighted sum of the k expert outputs plus the always-on shared expert
// (Deep Dive §3.1 forward; §3.3 figure "Weighted sum" then "Shared Expert
// (always) … add").  A workgroup gathers the k fp32 rows of one token (at
// small T, a quarter or half of its columns) in slot order; fp32
// accumulation in a fixed order, one rounding to the output type at the
// store, no atomics.  In a block forward the residual stream is added
// first (§3.3 figure, "Residual + Output").
//
// Quantisation: per row and 128 channels, scale = amax / 448 (fp32, 1 for an
// all-zero block) and code = e4m3(v / scale), round to nearest even -- the
// FP8 format of "dots3-note 架构深度解析" (mlqm.cn, «核心架构参数一览»:
// BF16、FP8) at per-token-per-128-channel granularity.
#include "combine_device.h"

namespace moe {
namespace {

template <int OK, bool YF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y,
                                                      const void* __restrict__ ysh,
                                                      const int32_t* __restrict__ yexp,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ inv,
                                                      const void* __restrict__ residual,
                                                      void* __restrict__ out, int T, int H, int k,
                                                      int S) {
  __shared__ float ws[kMaxTopK];
  __shared__ long long rs[kMaxTopK];
  // block (t, part): a 1/gridDim.y share of token t's columns
  const int per = (H / static_cast<int>(gridDim.y) + 7) & ~7;
  const int c0 = static_cast<int>(blockIdx.y) * per;
  const int c1 = min(H, c0 + per);
  combine_token<OK, YF16>(y, ysh, w, inv, residual, out, T, H, k, S, blockIdx.x, ws, rs, c0, c1,
                          yexp);
}

// 16 lanes per 128-channel block, 8 channels per lane.
__global__ __launch_bounds__(256) void quant_rows_fp8_kernel(const uint16_t* __restrict__ x,
                                                             int rows, int cols,
                                                             uint8_t* __restrict__ q,
                                                             float* __restrict__ scales) {
  const long long gid = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int nblk = cols / kQBlock;
  const long long blk = gid >> 4;
  const int sub = static_cast<int>(gid & 15);
  const bool on = blk < static_cast<long long>(rows) * nblk;
  float v[8];
  float amax = 0.f;
  const long long base = on ? (blk / nblk) * cols + (blk % nblk) * kQBlock + sub * 8 : 0;
  if (on) {
    const uint4 u = *reinterpret_cast<const uint4*>(x + base);
    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(static_cast<uint16_t>(w4[i]));
      v[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(w4[i] >> 16));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = row16_fmax(amax);
  if (!on) return;
  const float scale = (amax == 0.f) ? 1.0f : amax / 448.0f;
  uint2 codes;
  codes.x = f32x4_to_e4m3(v[0] / scale, v[1] / scale, v[2] / scale, v[3] / scale);
  codes.y = f32x4_to_e4m3(v[4] / scale, v[5] / scale, v[6] / scale, v[7] / scale);
  *reinterpret_cast<uint2*>(q + base) = codes;
  if (sub == 0) scales[blk] = scale;
}

}  // namespace

hipError_t launch_combine(int act_kind, const void* y, const void* ysh, const int32_t* yexp,
                          const float* w, const int32_t* inv, const void* residual, void* out,
                          int T, int H, int k, int S, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  // Small batches: split each token's columns over up to 4 blocks (at least
  // 1024 columns each) so that the launch has ~1024 blocks.  Measured at
  // T=256: 16.7 us with one block per token, 13.3 us split in 4.
  int parts = 1;
  while (parts < 4 && static_cast<long long>(T) * parts < 1024 && H / (2 * parts) >= 1024) parts *= 2;
  const dim3 g(T, parts);
  if (act_kind == K_BF16) {
    if (yexp)
      hipLaunchKernelGGL((combine_kernel<K_BF16, true>), g, dim3(256), 0, st, y, ysh, yexp, w, inv,
                         residual, out, T, H, k, S);
    else
      hipLaunchKernelGGL((combine_kernel<K_BF16, false>), g, dim3(256), 0, st, y, ysh, yexp, w,
                         inv, residual, out, T, H, k, S);
  } else {
    if (yexp) return hipErrorInvalidValue;  // fp32 layers keep fp32 y
    hipLaunchKernelGGL((combine_kernel<K_F32, false>), g, dim3(256), 0, st, y, ysh, yexp, w, inv,
                       residual, out, T, H, k, S);
  }
  return hipGetLastError();
}

hipError_t launch_quant_rows_fp8(const uint16_t* x_bf16, int rows, int cols, uint8_t* q,
                                 float* scales, hipStream_t st) {
  const long long threads = static_cast<long long>(rows) * (cols / kQBlock) * 16;
  if (threads <= 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_fp8_kernel, dim3(static_cast<unsigned>((threads + 255) / 256)),
                     dim3(256), 0, st, x_bf16, rows, cols, q, scales);
  return hipGetLastError();
}

}  // namespace moe
