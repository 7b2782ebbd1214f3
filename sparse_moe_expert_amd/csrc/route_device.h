// Router selection on one token (one wavefront): sigmoid scores, optional
// group limit, bias-for-selection top-k, renormalised weights.  Shared by the
// router kernel (route.hip) and the single-launch layer (fused.hip); the
// method and its sources are described in route.hip.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ float sigmoidf_acc(float l) { return 1.0f / (1.0f + expf(-l)); }

// Wave-wide maximum of a 32-bit value, returned to every lane (scalar):
// DPP steps inside each row of 16 lanes (quad xor 1, quad xor 2, half-row
// mirror, row mirror), then the four row maxima read out and compared.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x141, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x140, 0xF, 0xF, false)));
  const uint32_t r0 = __builtin_amdgcn_readlane(static_cast<int>(v), 0);
  const uint32_t r1 = __builtin_amdgcn_readlane(static_cast<int>(v), 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(static_cast<int>(v), 32);
  const uint32_t r3 = __builtin_amdgcn_readlane(static_cast<int>(v), 48);
  return max(max(r0, r1), max(r2, r3));
}

// Keys per lane for E experts (expert e = i * 64 + lane): 1, 2, 4 or 8.
__host__ __device__ inline int router_keys_per_lane(int E) {
  return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : 8;
}

// One wavefront selects the experts of token t.  cw: this wave's LDS row of
// kMaxExperts floats (group-limited routing stages the keys there).  KPER *
// 64 >= E.  A selection key is the order-preserving 32-bit image of c (0 =
// no key: taken, outside the allowed groups, or past E); among equal keys
// the lower expert index wins, as in the oracle's ordering.
template <int KPER>
__device__ __forceinline__ void router_topk_token(const float* __restrict__ logits, int splits,
                                                  const float* __restrict__ bias, int T, int E,
                                                  int k, int n_group, int topk_group, int norm,
                                                  float rsf, int32_t* __restrict__ idx_out,
                                                  float* __restrict__ w_out,
                                                  int32_t* __restrict__ ties, int t, int lane,
                                                  float* cw) {
  const float* lrow = logits + static_cast<long long>(t) * E;
  const long long split_stride = static_cast<long long>(T) * E;
  float score[KPER];
  uint32_t key[KPER];
  // split-K partial sums, added in split order (deterministic); the loads of
  // up to 8 splits are issued before their adds
  float l[KPER];
#pragma unroll
  for (int i = 0; i < KPER; ++i) l[i] = (i * 64 + lane < E) ? lrow[i * 64 + lane] : 0.f;
  for (int sp = 1; sp < splits; sp += 8) {
    float part[KPER][8];
#pragma unroll
    for (int i = 0; i < KPER; ++i)
#pragma unroll
      for (int q = 0; q < 8; ++q)
        part[i][q] = (sp + q < splits && i * 64 + lane < E)
                         ? lrow[(sp + q) * split_stride + i * 64 + lane]
                         : 0.f;
#pragma unroll
    for (int i = 0; i < KPER; ++i)
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (sp + q < splits) l[i] += part[i][q];
  }
#pragma unroll
  for (int i = 0; i < KPER; ++i) {
    const int e = i * 64 + lane;
    if (e < E) {
      score[i] = sigmoidf_acc(l[i]);
      const float c = score[i] + bias[e];
      key[i] = f32_order_key(c);
      if (n_group > 1) cw[e] = c;
    } else {
      score[i] = 0.f;
      key[i] = 0;
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
    for (int i = 0; i < KPER; ++i) {
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
    // this lane's best key (its lowest expert among equal keys), then the
    // wave's best key
    uint32_t kb = 0;
    int ib = 0;
    float sb = 0.f;
#pragma unroll
    for (int i = 0; i < KPER; ++i)
      if (key[i] > kb) {
        kb = key[i];
        ib = i;
        sb = score[i];
      }
    const uint32_t m = wave_max_u32(kb);
    // the lowest expert index holding it: lowest slot i, then lowest lane
    int wl = 0, wi = 0;
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const uint64_t hit = __ballot(kb == m && ib == i);
      if (hit) {
        wl = static_cast<int>(__builtin_ctzll(hit));
        wi = i;
        break;
      }
    }
    const int e = wi * 64 + wl;
    const float c = f32_from_order_key(m);
    if (j < k) {
      // the owner lane retires the key; the unbiased score is read from it
#pragma unroll
      for (int i = 0; i < KPER; ++i)
        if (lane == wl && i == wi) key[i] = 0;
      const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sb), wl));
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
