// One tile of the weight-streaming decode GEMM, shared by its kernel
// (gemm_decode.hip) and the single-launch layer (fused.hip); the method is
// described in gemm_decode.hip.
#pragma once

#include "gemm_sched.h"

namespace moe {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 16-byte weight load.  STREAM (expert weights): each touched expert's
// matrix is read exactly once per launch, so the load is marked
// non-temporal and the weight stream does not displace the cached token rows
// (measured at T=256: gate/up 1.360 -> 1.258 ms, down 0.745 -> 0.670 ms).  The
// router weight is read by every token tile and stays a cached load.
typedef int w16_vec_t __attribute__((ext_vector_type(4)));
template <bool STREAM>
__device__ __forceinline__ uint4 load_weights16(const char* ptr) {
  if constexpr (STREAM)
    return __builtin_bit_cast(
        uint4, __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) w16_vec_t*>(
                   reinterpret_cast<uintptr_t>(ptr))));
  else
    return *reinterpret_cast<const uint4*>(ptr);
}

template <int MT, int NT, int NA>
struct Regs {
  uint4 a[NA][MT][4];  // NA = 2: A and its bf16 residue A_lo
  uint4 b[NT][4];
};

// One 4-wave tile (block index b, see find_tile_at) of the decode GEMM.
// LO (projection only): A is a two-term bf16 split, A + A_lo (p.A_lo), and
// both terms multiply the same weight fragments.  STREAM: the weights are
// expert weights, read once per launch (non-temporal loads).
template <int MT, bool DUAL, int NT, bool LO = false, bool STREAM = true>
__device__ __forceinline__ void decode_tile(const GemmLaunch& p, int b) {
  static_assert(!(DUAL && LO), "the two-term A is the down projection's input");
  constexpr int NA = LO ? 2 : 1;
  // NT 16-row weight tiles per wave: gate/up holds NT/2 gate tiles and the
  // NT/2 matching up tiles
  constexpr int BM = 16 * MT;
  constexpr int WC = DUAL ? 8 * NT : 16 * NT;  // output columns per wave
  constexpr int BN = 4 * WC;                   // per block (4 waves)
  TileJob job;
  if (!find_tile_at<BM, BN, DUAL>(p, job, b)) return;

  const int lane = threadIdx.x & 63;
  const int wave = (threadIdx.x >> 6) & 3;
  const int lrow = lane & 15;
  const int lgrp = lane >> 4;
  const int K = p.K;
  const int N = p.N;
  // split K (fp32 projection only): block row y takes K-blocks
  // [y * nkb, (y + 1) * nkb) and writes C + y * c_split_stride
  int nkb = K / 128, kb0 = 0;
  long long c_off = 0;
  if (!DUAL && p.k_splits > 1) {
    nkb /= p.k_splits;
    kb0 = static_cast<int>(blockIdx.y) * nkb;
    c_off = static_cast<long long>(blockIdx.y) * p.c_split_stride;
  }
  const long long rowb_a = p.lda * 2;
  const long long rowb_b = static_cast<long long>(K) * 2;

  // this wave's weight rows
  const int wn0 = job.n0 + wave * WC;
  const char* bptr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int wr;
    if constexpr (DUAL) {
      // tiles [0, NT/2) gate rows, [NT/2, NT) the matching up rows
      const int n = min(wn0 + (t % (NT / 2)) * 16 + lrow, N - 1);
      wr = (t < NT / 2) ? n : N + n;
    } else {
      wr = min(wn0 + t * 16 + lrow, N - 1);
    }
    bptr[t] = job.W + w_tile_row_off(p.w_tiled, wr, rowb_b) + w_tile_k_off(p.w_tiled, lgrp * 16);
  }
  const char* aptr[NA][MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int r = min(m * 16 + lrow, job.rows_here - 1);
    const int src = gemm_a_source_row(p, job.row_begin + job.m0 + r);
    aptr[0][m] = static_cast<const char*>(p.A) + src * rowb_a + lgrp * 16;
    if constexpr (LO) aptr[NA - 1][m] = static_cast<const char*>(p.A_lo) + src * rowb_a + lgrp * 16;
  }

  // a 128-wide K-block of bf16 is 256 bytes: four 64-byte tile columns of the
  // tiled layout, load s reading column s (16 rows x 64 bytes, 1 KB contiguous)
  const int s_stride_b = static_cast<int>(w_tile_k_off(p.w_tiled, 64));
  auto load = [&](Regs<MT, NT, NA>& R, int kb) {
    const int off = (kb0 + kb) * 256;
    const int off_b = static_cast<int>(w_tile_k_off(p.w_tiled, (kb0 + kb) * 256));
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        R.b[t][s] = load_weights16<STREAM>(bptr[t] + off_b + s * s_stride_b);
#pragma unroll
    for (int q = 0; q < NA; ++q)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          R.a[q][m][s] = *reinterpret_cast<const uint4*>(aptr[q][m] + off + s * 64);
  };

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[m][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Regs<MT, NT, NA>& R) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int q = 0; q < NA; ++q)
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int t = 0; t < NT; ++t)
            acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, R.a[q][m][s]), __builtin_bit_cast(bf16x8, R.b[t][s]),
                acc[m][t], 0, 0, 0);
  };

  Regs<MT, NT, NA> r0, r1;
  load(r0, 0);
  int kb = 0;
  for (; kb + 2 <= nkb; kb += 2) {
    load(r1, kb + 1);
    compute(r0);
    if (kb + 2 < nkb) load(r0, kb + 2);
    compute(r1);
  }
  if (kb < nkb) compute(r0);

  // 16x16 accumulator layout: lane l, element i -> token row 4*(l/16) + i,
  // weight row l%16 of the tile.
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = m * 16 + lgrp * 4 + i;
      if (r >= job.rows_here) continue;
      const long long row = job.row_begin + job.m0 + r;
      if constexpr (DUAL) {
#pragma unroll
        for (int j = 0; j < NT / 2; ++j) {
          const int n = wn0 + j * 16 + lrow;
          if (n < N) {
            const float g = acc[m][j][i];
            const float u = acc[m][j + NT / 2][i];
            const float h = silu_mul(g, u);
            const uint16_t hi = f32_to_bf16(h);
            reinterpret_cast<uint16_t*>(gemm_out_row<2>(p, row))[n] = hi;
            if (p.C_lo)
              reinterpret_cast<uint16_t*>(static_cast<char*>(p.C_lo) + row * p.ldc * 2)[n] =
                  f32_to_bf16(h - bf16_to_f32(hi));
          }
        }
      } else {
        float* dst = reinterpret_cast<float*>(gemm_out_row<4>(p, row)) + c_off;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int n = wn0 + t * 16 + lrow;
          if (n < N) dst[n] = acc[m][t][i];
        }
      }
    }
}

}  // namespace moe
