// Weight-streaming grouped GEMM for the decode regime (a handful of token
// rows per expert), bf16 operands, fp32 accumulation (gfx950).
//
// Same computation as the other grouped GEMM kernels -- gate/up + SwiGLU
// (gmm1 -> swiglu of the Deep Dive §8.2 figure; packed gate_up per the
// Transformers Dots1 article «并行策略字段») or a plain projection -- shaped for
// the HBM roofline: every weight byte of every touched expert is read once,
// and the rows per expert (about 8 at T=256, top-8 of 256) are too few for
// any on-chip reuse of the weights to matter.
//
//  * One wave owns NT 16-row weight tiles for 16*MT token rows over the whole
//    K: 8*NT h-columns (NT/2 gate tiles + the NT/2 matching up tiles) or
//    16*NT output columns.  A workgroup is 4 such waves side by side in N.
//    NT = 4 is used (measured at T=256: 2% faster than NT = 2).
//  * Weights go straight from HBM into registers, no LDS, no barriers: per
//    128-wide K-block a lane makes 4 x 16-byte loads of one weight row, and
//    the next K-block's loads are issued before the current block's MFMAs.
//    Load s of lane group g (= lane / 16) reads chunk 4s + g of the block:
//    one load instruction covers 64 contiguous bytes of each of 16 rows, and
//    step s of the MFMA sees K in its natural order.
//  * The expert's token rows (A) come from L2: all waves of the expert read
//    the same few rows.
//  * v_mfma_f32_16x16x32_bf16: rows = tokens (lane%16), columns = weight rows.
#include "gemm_sched.h"

namespace moe {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int MT, int NT>
struct Regs {
  uint4 a[MT][4];
  uint4 b[NT][4];
};

template <int MT, bool DUAL, int NT>
__global__ __launch_bounds__(256) void gemm_decode_kernel(GemmLaunch p) {
  // NT 16-row weight tiles per wave: gate/up holds NT/2 gate tiles and the
  // NT/2 matching up tiles
  constexpr int BM = 16 * MT;
  constexpr int WC = DUAL ? 8 * NT : 16 * NT;  // output columns per wave
  constexpr int BN = 4 * WC;                   // per block (4 waves)
  TileJob job;
  if (!find_tile<BM, BN, DUAL>(p, job)) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lrow = lane & 15;
  const int lgrp = lane >> 4;
  const int K = p.K;
  const int N = p.N;
  const int nkb = K / 128;
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
    bptr[t] = job.W + wr * rowb_b + lgrp * 16;
  }
  const char* aptr[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int r = min(m * 16 + lrow, job.rows_here - 1);
    const int src = gemm_a_source_row(p, job.row_begin + job.m0 + r);
    aptr[m] = static_cast<const char*>(p.A) + src * rowb_a + lgrp * 16;
  }

  auto load = [&](Regs<MT, NT>& R, int kb) {
    const int off = kb * 256;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s) R.b[t][s] = *reinterpret_cast<const uint4*>(bptr[t] + off + s * 64);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int s = 0; s < 4; ++s) R.a[m][s] = *reinterpret_cast<const uint4*>(aptr[m] + off + s * 64);
  };

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[m][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Regs<MT, NT>& R) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, R.a[m][s]), __builtin_bit_cast(bf16x8, R.b[t][s]),
              acc[m][t], 0, 0, 0);
  };

  Regs<MT, NT> r0, r1;
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
            reinterpret_cast<uint16_t*>(gemm_out_row<2>(p, row))[n] =
                f32_to_bf16(g / (1.0f + expf(-g)) * u);
          }
        }
      } else {
        float* dst = reinterpret_cast<float*>(gemm_out_row<4>(p, row));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int n = wn0 + t * 16 + lrow;
          if (n < N) dst[n] = acc[m][t][i];
        }
      }
    }
}

template <int MT, bool DUAL, int NT>
hipError_t launch_decode(const GemmLaunch& g, hipStream_t st) {
  constexpr int BM = 16 * MT;
  constexpr int BN = 4 * (DUAL ? 8 * NT : 16 * NT);
  const int ntn = (g.N + BN - 1) / BN;
  const long long ub_m =
      g.single_group_rows > 0 ? (g.single_group_rows + BM - 1) / BM : g.grid_mtiles_upper;
  const long long total = ub_m * ntn;
  if (total <= 0) return hipSuccess;
  const long long grid = ((total + 7) / 8) * 8;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_decode_kernel<MT, DUAL, NT>), dim3(static_cast<unsigned>(grid)),
                     dim3(256), 0, st, g);
  return hipGetLastError();
}

// Tile shapes: gate/up bn = 64 (NT 2) or 128 (NT 4) h columns; projection
// bn = 128 (NT 2) or 256 (NT 4) output columns; bm = 16 or 32 rows.
template <int MT>
hipError_t launch_mt(TileShape ts, bool dual, const GemmLaunch& g, hipStream_t st) {
  if (dual) return ts.bn == 64 ? launch_decode<MT, true, 2>(g, st) : launch_decode<MT, true, 4>(g, st);
  return ts.bn == 128 ? launch_decode<MT, false, 2>(g, st) : launch_decode<MT, false, 4>(g, st);
}

}  // namespace

bool gemm_decode_supported(int a_kind, int out_kind, TileShape ts, bool dual) {
  if (a_kind != K_BF16 || (ts.bm != 16 && ts.bm != 32)) return false;
  if (dual) return out_kind == K_BF16 && (ts.bn == 64 || ts.bn == 128);
  return out_kind == K_F32 && (ts.bn == 128 || ts.bn == 256);
}

hipError_t launch_gemm_decode(TileShape ts, bool dual, const GemmLaunch& g, hipStream_t st) {
  return ts.bm == 16 ? launch_mt<1>(ts, dual, g, st) : launch_mt<2>(ts, dual, g, st);
}

}  // namespace moe
