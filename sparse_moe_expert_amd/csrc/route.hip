// Router selection: sigmoid scores, bias-for-selection top-k, renormalised
// weights -- one wavefront per token (gfx950).
//
// Scores are sigmoid of the router logits and the choice uses score + bias
// (noaux_tc), while the weights renormalise the unbiased scores of the k
// chosen experts (norm_topk_prob): "dots3-note 架构深度解析" (mlqm.cn),
// «稀疏激活Top-8 路由»; top-k then renormalisation as in the Dots3MoELayer
// forward of the Deep Dive §3.1; routed_scaling_factor from the Transformers
// Dots1 article's «MoE 路由与专家相关字段» table.
//
// Each lane holds E/64 keys (expert e = slot * 64 + lane), as the
// order-preserving 32-bit integer image of the fp32 key.  A round takes each
// lane's best key, the wave maximum by DPP steps inside each 16-lane row and
// four readlanes, then ballots slot by slot for the lowest expert index
// holding it, so equal keys go to the lower index.  k rounds pick the experts
// in slot order; one more round reads the (k+1)-th key for the near-tie
// count.
//
// Group-limited routing (n_group, topk_group of the same Dots1 field table,
// which maps them to DeepSeek-V3's router): each group's score is the sum of
// its two largest keys (the table gives no formula; this is DeepSeek-V3's
// rule).  Lane g computes group g's score from the wave's keys staged in
// LDS, a max over packed (group score, complemented group index) keys picks
// topk_group groups, and the keys of the experts outside them drop out
// before the top-k rounds.
#include "route_device.h"

namespace moe {
namespace {

constexpr int kWaves = 4;  // waves (tokens) per block

template <int KPER>
__global__ __launch_bounds__(64 * kWaves) void router_topk_kernel(const float* __restrict__ logits,
                                                          int splits,
                                                          const float* __restrict__ bias, int T,
                                                          int E, int k, int n_group, int topk_group,
                                                          int norm, float rsf,
                                                          int32_t* __restrict__ idx_out,
                                                          float* __restrict__ w_out,
                                                          int32_t* __restrict__ ties) {
  __shared__ float cbuf[kWaves][kMaxExperts];  // group-limited routing only
  const int t = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave leaves together
  router_topk_token<KPER>(logits, splits, bias, T, E, k, n_group, topk_group, norm, rsf, idx_out,
                          w_out, ties, t, threadIdx.x & 63, cbuf[threadIdx.x >> 6]);
}

__global__ void zero_i32_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

hipError_t launch_router_topk(const float* logits, int splits, const float* bias, int T, int E,
                              int k, int n_group, int topk_group, int norm, float rsf, int32_t* idx,
                              float* w, int32_t* ties, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (E < 1 || E > kMaxExperts) return hipErrorInvalidValue;
  const int grid = (T + kWaves - 1) / kWaves;
  const int sp = splits < 1 ? 1 : splits, ng = n_group > 1 ? n_group : 1;
  switch (router_keys_per_lane(E)) {
    case 1:
      hipLaunchKernelGGL(router_topk_kernel<1>, dim3(grid), dim3(64 * kWaves), 0, st, logits, sp,
                         bias, T, E, k, ng, topk_group, norm, rsf, idx, w, ties);
      break;
    case 2:
      hipLaunchKernelGGL(router_topk_kernel<2>, dim3(grid), dim3(64 * kWaves), 0, st, logits, sp,
                         bias, T, E, k, ng, topk_group, norm, rsf, idx, w, ties);
      break;
    case 4:
      hipLaunchKernelGGL(router_topk_kernel<4>, dim3(grid), dim3(64 * kWaves), 0, st, logits, sp,
                         bias, T, E, k, ng, topk_group, norm, rsf, idx, w, ties);
      break;
    default:
      hipLaunchKernelGGL(router_topk_kernel<8>, dim3(grid), dim3(64 * kWaves), 0, st, logits, sp,
                         bias, T, E, k, ng, topk_group, norm, rsf, idx, w, ties);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace moe
