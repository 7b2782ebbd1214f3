// Router selection on one token (one wavefront): sigmoid scores, optional
// group limit, bias-for-selection top-k, renormalised weights.  Shared by the
// router kernel (route.hip) and the single-launch layer (fused.hip); the
// method and its sources are described in route.hip.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kPer = kMaxExperts / 64;

__device__ __forceinline__ float sigmoidf_acc(float l) { return 1.0f / (1.0f + expf(-l)); }

// One wavefront selects the experts of token t.  cw: this wave's LDS row of
// kMaxExperts floats (group-limited routing stages the keys there).
__device__ __forceinline__ void router_topk_token(const float* __restrict__ logits, int splits,
                                                  const float* __restrict__ bias, int T, int E,
                                                  int k, int n_group, int topk_group, int norm,
                                                  float rsf, int32_t* __restrict__ idx_out,
                                                  float* __restrict__ w_out,
                                                  int32_t* __restrict__ ties, int t, int lane,
                                                  float* cw) {
  const float* lrow = logits + static_cast<long long>(t) * E;
  const long long split_stride = static_cast<long long>(T) * E;
  float score[kPer];
  uint64_t key[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = i * 64 + lane;
    if (e < E) {
      // split-K partial sums, added in split order (deterministic)
      float l = lrow[e];
      for (int sp = 1; sp < splits; ++sp) l += lrow[sp * split_stride + e];
      score[i] = sigmoidf_acc(l);
      const float c = score[i] + bias[e];
      key[i] = (static_cast<uint64_t>(f32_order_key(c)) << 32) | static_cast<uint32_t>(~e);
      if (n_group > 1) cw[e] = c;
    } else {
      score[i] = 0.f;
      key[i] = 0;  // below every real key
    }
  }

  // Group limit: group g holds experts [g*G, (g+1)*G); its score is the sum
  // of its two largest keys.  The topk_group best groups (lower index first
  // among equal scores) stay; the keys of every other expert drop to 0.
  int allowed = E;
  float gap_grp = INFINITY;
  if (n_group > 1) {
    // the wave's own LDS row: make the stores visible to the other lanes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int G = E / n_group;
    uint64_t gkey = 0;
    if (lane < n_group) {
      float t1 = -INFINITY, t2 = -INFINITY;
      for (int j = 0; j < G; ++j) {
        const float v = cw[lane * G + j];
        if (v > t1) {
          t2 = t1;
          t1 = v;
        } else if (v > t2) {
          t2 = v;
        }
      }
      const float gs = (G > 1) ? t1 + t2 : t1;
      gkey = (static_cast<uint64_t>(f32_order_key(gs)) << 32) | static_cast<uint32_t>(~lane);
    }
    uint64_t chosen = 0;
    float last = 0.f;
    const int grounds = topk_group < n_group ? topk_group + 1 : topk_group;
    for (int r = 0; r < grounds; ++r) {
      uint64_t best = gkey;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const uint64_t o = shfl_xor_u64(best, m);
        best = o > best ? o : best;
      }
      const int g = static_cast<int>(~static_cast<uint32_t>(best));
      const float sc = f32_from_order_key(static_cast<uint32_t>(best >> 32));
      if (r < topk_group) {
        chosen |= 1ull << g;
        if (lane == g) gkey = 0;
        last = sc;
      } else {
        gap_grp = last - sc;
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = i * 64 + lane;
      if (e < E && !((chosen >> (e / G)) & 1ull)) key[i] = 0;
    }
    allowed = topk_group * G;
  }

  int chosen_e[kMaxTopK];
  float chosen_s[kMaxTopK];
  float prev_c = 0.f, min_gap = INFINITY, gap_sel = INFINITY;
  const int rounds = (k < allowed) ? k + 1 : k;
#pragma unroll
  for (int j = 0; j <= kMaxTopK; ++j) {
    if (j >= rounds) continue;
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) best = key[i] > best ? key[i] : best;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const uint64_t o = shfl_xor_u64(best, m);
      best = o > best ? o : best;
    }
    const int e = static_cast<int>(~static_cast<uint32_t>(best));
    const float c = f32_from_order_key(static_cast<uint32_t>(best >> 32));
    if (j < k) {
      // the owner lane retires the key and broadcasts the unbiased score
      float s_own = 0.f;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if (lane == (e & 63) && i == (e >> 6)) {
          s_own = score[i];
          key[i] = 0;
        }
      }
      const float s = __shfl(s_own, e & 63, 64);
      if (j < kMaxTopK) {
        chosen_e[j] = e;
        chosen_s[j] = s;
      }
      if (j > 0) min_gap = fminf(min_gap, prev_c - c);
    } else {
      gap_sel = prev_c - c;
    }
    prev_c = c;
  }

  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (j < k) sum += chosen_s[j];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k && lane == j) {
      const float w = norm ? (chosen_s[j] / sum) * rsf : chosen_s[j] * rsf;
      idx_out[static_cast<long long>(t) * k + j] = chosen_e[j];
      w_out[static_cast<long long>(t) * k + j] = w;
    }
  }
  if (ties && lane == 0) {
    if (gap_sel <= kTieEps || gap_grp <= kTieEps) atomicAdd(&ties[0], 1);
    if (min_gap <= kTieEps) atomicAdd(&ties[1], 1);
  }
}

}  // namespace moe
