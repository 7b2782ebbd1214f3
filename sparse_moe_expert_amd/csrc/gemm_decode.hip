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
//  * Expert weights are read with non-temporal loads: every byte is used
//    once per launch, and the stream of them (8 GB for gate/up at T=256)
//    would otherwise displace the token rows that every block re-reads.
//    Measured at T=256: gate/up 1.360 -> 1.258 ms (6.4 TB/s), down 0.745 ->
//    0.670 ms.  The router weight (one implicit group) is re-read by every
//    token tile and keeps cached loads.
//  * The expert's token rows (A) come from L2: all waves of the expert read
//    the same few rows.
//  * v_mfma_f32_16x16x32_bf16: rows = tokens (lane%16), columns = weight rows.
//  * h as two bf16 terms: the gate/up epilogue stores hi = bf16(h) and
//    lo = bf16(h - hi); the projection multiplies both by the same weight
//    registers (twice the MFMAs and the L2-resident token loads, no extra
//    weight bytes), so h enters the down GEMM with ~16 significant bits.
#include "gemm_decode_device.h"

namespace moe {
namespace {

template <int MT, bool DUAL, int NT, bool LO, bool STREAM>
__global__ __launch_bounds__(256) void gemm_decode_kernel(GemmLaunch p) {
  decode_tile<MT, DUAL, NT, LO, STREAM>(p, blockIdx.x);
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
  // split K: projection only, whole K-blocks per split
  const int splits = g.k_splits > 1 ? g.k_splits : 1;
  if (splits > 1 && (DUAL || (g.K / 128) % splits != 0)) return hipErrorInvalidValue;
  const dim3 gd(static_cast<unsigned>(grid), static_cast<unsigned>(splits));
  // expert weights stream (non-temporal); the router's single weight matrix
  // (single_group_rows > 0) is shared by all token tiles and stays cached
  const bool stream = g.single_group_rows == 0;
  if (!DUAL && g.A_lo)
    hipLaunchKernelGGL((gemm_decode_kernel<MT, DUAL, NT, !DUAL, true>), gd, dim3(256), 0, st, g);
  else if (stream)
    hipLaunchKernelGGL((gemm_decode_kernel<MT, DUAL, NT, false, true>), gd, dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_decode_kernel<MT, DUAL, NT, false, false>), gd, dim3(256), 0, st, g);
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
