// Weight-streaming grouped FP8 GEMM for mid-size batches (about 100 to 200
// token rows per expert), e4m3 operands with fp32 block scales, fp32
// accumulation (gfx950).
//
// Same computation as the other FP8 grouped GEMMs -- gate/up + SwiGLU with h
// re-quantised per token and 128 columns, or the plain projection -- with a
// tiling chosen for the HBM roofline of that regime: below the fp8 ridge
// point (~625 flop/byte) the weights are the cost, so
//
//  * a tile holds up to 192 token rows, all the rows of an expert at these
//    batch sizes, so each expert's weights stream from HBM once (with
//    128-row tiles an expert just over 128 rows read its weights twice);
//  * each of the 8 waves owns 32 weight rows (two 16-row MFMA tiles) over
//    the whole K, loaded straight from memory into registers as the A
//    operand of v_mfma_scale_f32_16x16x128_f8f6f4, two steps ahead (64 KB
//    of weights in flight per CU; three steps ahead measured no faster).  The MFMA takes any order of K as long as
//    both operands use the same one: lane l holds 16-byte chunks l / 16 and
//    4 + l / 16 of the 128-byte step of row l % 16, so each of the two load
//    instructions reads 64 whole bytes of 16 rows (one contiguous kilobyte of
//    MOE_LAYOUT_TILED) instead of every other 16 bytes of 32 rows;
//  * the token rows (shared by all waves) stream global -> LDS by DMA into a
//    ring of three 24 KB slots, rows 128 bytes wide with 16-byte chunks
//    XOR-swizzled by row so fragment reads do not conflict;
//  * one K step is one 128-wide scale block, so each MFMA's partial product
//    is scaled once, by the token's row scale times the weight block scale
//    (DeepSeek-V3 Technical Report, FP8 training section), and added to the
//    fp32 accumulators;
//  * token scales for the whole K and the weight block scales of the tile are
//    staged in LDS before the main loop;
//  * gate/up: a block's 256 weight rows are 128 gate rows and the matching
//    128 up rows, so its 128 h columns are exactly one quantisation block of
//    h: SiLU(g) * u, then per token amax / 448 and e4m3 codes, on chip.
#include <utility>

#include "gemm_sched.h"

namespace moe {
namespace {

constexpr int BM = 192;                     // token rows per block
constexpr int WAVES = 8;
constexpr int THREADS = WAVES * 64;
constexpr int BROWS = WAVES * 32;           // weight rows per block
constexpr int STEP = 128;                   // K bytes per step (one scale block)
constexpr int D = 2;                        // steps loaded ahead
constexpr int S = D + 1;                    // ring slots (weights and tokens)
constexpr int A_SLOT = BM * STEP;           // 24 KB of token rows per step
constexpr int A_DMA = A_SLOT / 16 / THREADS;  // 16-byte DMA chunks per thread per step: 3
constexpr int W_LOADS = 4;                  // 16-byte weight loads per thread per step
constexpr int MAX_KB = 64;                  // K <= 8192
constexpr int kXcdChunk = 32;               // tiles per XCD chunk: one block per CU, 32 CUs per XCD
constexpr int SA_OFF = S * A_SLOT;          // token scales [kb][row] fp32
constexpr int SB_OFF = SA_OFF + MAX_KB * BM * 4;  // weight block scales [2][kb] fp32
constexpr int LDC = 128 + 4;                // fp32 epilogue tile row stride
constexpr int SMEM = SB_OFF + 2 * MAX_KB * 4;
static_assert(BM * LDC * 4 <= SMEM, "epilogue tile inside the operand buffers");
static_assert(A_SLOT % (16 * THREADS) == 0, "whole DMA chunks per thread");

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 128-byte LDS rows: chunk c of row r at c ^ ((r >> 1) & 7), so the 16 rows
// a fragment read touches at one logical chunk hit 16 distinct bank groups.
__device__ __forceinline__ int swz_key(int r) { return (r >> 1) & 7; }

template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// This thread's DMA of the step has landed (vmcnt), its LDS reads are done
// (lgkmcnt 0); then the workgroup barrier, without a memory fence that would
// drain the loads still in flight.
template <int N>
__device__ __forceinline__ void step_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

__device__ __forceinline__ i32x4_t gload16(const char* p) {
  return *reinterpret_cast<const __attribute__((address_space(1))) i32x4_t*>(
      reinterpret_cast<uintptr_t>(p));
}

// MT: 16-row token tiles computed (4, 8 or 12; the ragged rows past the
// tile's last row in the last of them are computed and never stored).  Only
// those MT * 16 rows are brought in: AD = MT / 4 DMA chunks per thread and
// step (a tile of 65-128 rows moves 16 KB of token rows per step, not 24).
template <bool DUAL, int MT>
__device__ __forceinline__ void tile_body(const GemmLaunch& p, const TileJob& job, char* smem) {
  static_assert(MT % 4 == 0 && MT / 4 <= A_DMA, "64-row groups of the 192-row tile");
  constexpr int AD = MT / 4;          // 16-byte DMA chunks per thread per step
  constexpr int OPS = AD + W_LOADS;   // vector memory ops per thread per step
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = p.N;
  const int K = p.K;
  const int nk = K / STEP;
  const long long rowb_b = K;  // e4m3 weight row bytes

  // ---- token rows: DMA chunk j of the thread fills tile row
  // (j * WAVES + wave) * 8 + lane / 8 at physical chunk lane % 8 (rows past
  // the tile's last row repeat it: every thread issues the same number of
  // loads per step, which the step's vmcnt wait counts on)
  const char* a_src[AD];
#pragma unroll
  for (int j = 0; j < AD; ++j) {
    const int r = (j * WAVES + wave) * 8 + (lane >> 3);
    const int lchunk = (lane & 7) ^ swz_key(r);
    const int src = gemm_a_source_row(p, job.row_begin + job.m0 + min(r, job.rows_here - 1));
    a_src[j] = static_cast<const char*>(p.A) + static_cast<long long>(src) * p.lda + lchunk * 16;
  }
  // ---- weight rows of this wave: tile 0 and tile 1
  const char* w_src[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    int row;
    if constexpr (DUAL) {  // tile 0: gate rows, tile 1: the matching up rows
      const int n = min(job.n0 + wave * 16 + (lane & 15), N - 1);
      row = t == 0 ? n : N + n;
    } else {
      row = min(job.n0 + wave * 32 + t * 16 + (lane & 15), N - 1);
    }
    w_src[t] = job.W + w_tile_row_off(p.w_tiled, row, rowb_b) + w_tile_k_off(p.w_tiled, 16 * (lane >> 4));
  }
  // the block's two weight row blocks (DUAL: gate, up; projection: rows
  // [n0, n0 + 128) and [n0 + 128, n0 + 256)) stage their scales in LDS
  float* sa_tab = reinterpret_cast<float*>(smem + SA_OFF);
  float* sb_tab = reinterpret_cast<float*>(smem + SB_OFF);
  const int kblocks = K / kQBlock;
  float sb_val = 0.f;
  int sb_slot = -1;
  if (tid < 2 * nk) {
    const int q = tid / nk, kb = tid - q * nk;
    const int rb = DUAL ? ((q == 0 ? 0 : N) + min(job.n0, N - 1)) / kQBlock
                        : min(job.n0 + q * 128, N - 1) / kQBlock;
    sb_val = job.WS[static_cast<long long>(rb) * kblocks + kb];
    sb_slot = q * MAX_KB + kb;
  }
  // token scales sa_tab[kb * BM + r] of the tile's MT * 16 rows by 4-byte
  // DMA, 64 rows of one K block per instruction; every wave issues the same
  // number (the last repeated)
  {
    const int per_kb = AD;
    const int total = per_kb * nk;
    const int n_iss = (total + WAVES - 1) / WAVES;
    for (int i = 0; i < n_iss; ++i) {
      const int idx = min(i * WAVES + wave, total - 1);
      const int kb = idx / per_kb;
      const int r = (idx - kb * per_kb) * 64 + lane;
      const int src = gemm_a_source_row(p, job.row_begin + job.m0 + min(r, job.rows_here - 1));
      __builtin_amdgcn_global_load_lds(p.a_scale + static_cast<long long>(src) * kblocks + kb,
                                       (lds_ptr_t)(sa_tab + kb * BM + (idx - kb * per_kb) * 64),
                                       4, 0, 0);
    }
  }

  i32x4_t wr[S][2][2];  // weight ring: slot, tile, 16-byte half
  auto issue = [&](auto rc, int kt) __attribute__((always_inline)) {
    constexpr int R = decltype(rc)::value;  // ring slot of step kt
    const int ks = min(kt, nk - 1);         // past the end: repeat the last step
    const long long wo = w_tile_k_off(p.w_tiled, static_cast<long long>(ks) * STEP);
    const long long wo2 = w_tile_k_off(p.w_tiled, static_cast<long long>(ks) * STEP + 64);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      wr[R][t][0] = gload16(w_src[t] + wo);   // chunk l / 16
      wr[R][t][1] = gload16(w_src[t] + wo2);  // chunk 4 + l / 16
    }
    char* base = smem + R * A_SLOT;
#pragma unroll
    for (int j = 0; j < AD; ++j)
      __builtin_amdgcn_global_load_lds(a_src[j] + ks * STEP,
                                       (lds_ptr_t)(base + (j * WAVES + wave) * 1024), 16, 0, 0);
  };

  f32x4 acc[2][MT];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[t][m] = f32x4{0.f, 0.f, 0.f, 0.f};

  // token fragment of tile m: row m*16 + lane%16, logical chunks l/16 and
  // 4 + l/16 (the weights' K order)
  const int r16 = lane & 15;
  const int c0 = lane >> 4;
  const int key = swz_key(r16);  // rows 16 apart share the key
  const int x_off0 = r16 * STEP + ((c0 ^ key) << 4);
  const int x_off1 = r16 * STEP + (((c0 + 4) ^ key) << 4);

  auto compute = [&](auto rc, int kt) __attribute__((always_inline)) {
    constexpr int R = decltype(rc)::value;
    const char* As = smem + R * A_SLOT;
    // weight block scale of each tile: DUAL, tile 0 gate and tile 1 up rows;
    // projection, both tiles in the block's first or second 128 rows
    const float sb0 = sb_tab[(DUAL ? 0 : (wave >> 2)) * MAX_KB + kt];
    const float sb1 = sb_tab[(DUAL ? 1 : (wave >> 2)) * MAX_KB + kt];
    const float* sa = sa_tab + kt * BM + r16;
    const i32x8_t w0 = __builtin_shufflevector(wr[R][0][0], wr[R][0][1], 0, 1, 2, 3, 4, 5, 6, 7);
    const i32x8_t w1 = __builtin_shufflevector(wr[R][1][0], wr[R][1][1], 0, 1, 2, 3, 4, 5, 6, 7);
    // token fragments read two tiles ahead of their MFMAs
    auto frag = [&](int m) __attribute__((always_inline)) {
      const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(As + m * 16 * STEP + x_off0);
      const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(As + m * 16 * STEP + x_off1);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    i32x8_t xf[3];
    float sv[4];  // four: tile m + 2's scale is read before tile m - 1's is used
    xf[0] = frag(0);
    sv[0] = sa[0];
    xf[1] = frag(1);
    sv[1] = sa[16];
    // the partial products of tile m are scaled into acc after the MFMAs of
    // tile m + 1 are issued, so no wave waits on its own MFMA result
    f32x4 pp[2][2];
#pragma unroll
    for (int m = 0; m <= MT; ++m) {
      if (m + 2 < MT) {
        xf[(m + 2) % 3] = frag(m + 2);
        sv[(m + 2) % 4] = sa[(m + 2) * 16];
      }
      if (m < MT) {
        // cbsz = blgp = 0: both operands e4m3; E8M0 scales 127 = 2^0
        pp[m & 1][0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            w0, xf[m % 3], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
        pp[m & 1][1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            w1, xf[m % 3], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
      }
      if (m > 0) {
        const float sp = sv[(m - 1) % 4];
        acc[0][m - 1] += pp[(m - 1) & 1][0] * (sp * sb0);
        acc[1][m - 1] += pp[(m - 1) & 1][1] * (sp * sb1);
      }
      // DS reads of tile m + 2, the two MFMAs of tile m, the scaling of tile m - 1
      if (m + 2 < MT) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // DS read
      if (m < MT) __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);      // MFMA
      if (m > 0) __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);      // VALU
    }
  };

  // prologue: steps 0 .. D-1 (each: weights then tokens)
  [&]<int... Rs>(std::integer_sequence<int, Rs...>) __attribute__((always_inline)) {
    (issue(std::integral_constant<int, Rs>{}, Rs), ...);
  }(std::make_integer_sequence<int, D>{});
  if (sb_slot >= 0) sb_tab[sb_slot] = sb_val;

  // step kt: wait for this thread's step-kt DMA (the D - 1 later steps' ops
  // may stay in flight), barrier, issue step kt + D into the slot step kt - 1
  // used, compute step kt
  auto iter = [&](auto rc, int kt) __attribute__((always_inline)) {
    constexpr int R = decltype(rc)::value;
    step_barrier<OPS * (D - 1)>();
    issue(std::integral_constant<int, (R + D) % S>{}, kt + D);
    compute(rc, kt);
  };
  // the ring slots are compile-time: S iterations per loop trip
  int kt = 0;
  auto run = [&](auto... rs) __attribute__((always_inline)) {
    for (; kt + S <= nk; kt += S) (iter(rs, kt + decltype(rs)::value), ...);
    ((kt + decltype(rs)::value < nk ? iter(rs, kt + decltype(rs)::value) : void()), ...);
  };
  [&]<int... Rs>(std::integer_sequence<int, Rs...>) __attribute__((always_inline)) {
    run(std::integral_constant<int, Rs>{}...);
  }(std::make_integer_sequence<int, S>{});

  // ------------------------------------------------------------ epilogue
  wait_vmem<0>();   // the repeated last steps' DMA has landed too
  __syncthreads();  // every wave is done with the operand buffers
  float* Cs = reinterpret_cast<float*>(smem);
  const int lgrp = lane >> 4;
  // 16x16 accumulator layout: lane l, element i -> weight row 4 (l / 16) + i of
  // the tile, token l % 16 of the token tile
  if constexpr (DUAL) {
    // h = SiLU(g) * u into Cs[token][h column], h column = 16 wave + 4 (l/16) + i
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Cs[(m * 16 + r16) * LDC + wave * 16 + lgrp * 4 + i] = silu_mul(acc[0][m][i], acc[1][m][i]);
    __syncthreads();
    // per token: scale = amax / 448 over the 128 columns, codes = e4m3(h / scale);
    // 16 lanes per row, 8 columns each
    for (int q = tid; q < MT * 16 * 16; q += THREADS) {
      const int r = q >> 4;
      const int c8 = (q & 15) * 8;
      const float* src = Cs + r * LDC + c8;
      float v[8];
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[i] = src[i];
        amax = fmaxf(amax, fabsf(v[i]));
      }
      amax = row16_fmax(amax);
      const float scale = (amax == 0.f) ? 1.0f : amax / 448.0f;
      const int n = job.n0 + c8;
      if (r < job.rows_here && n < N) {
        const long long row = job.row_begin + job.m0 + r;
        uint2 codes;
        codes.x = f32x4_to_e4m3(v[0] / scale, v[1] / scale, v[2] / scale, v[3] / scale);
        codes.y = f32x4_to_e4m3(v[4] / scale, v[5] / scale, v[6] / scale, v[7] / scale);
        *reinterpret_cast<uint2*>(gemm_out_row<1>(p, row) + n) = codes;
        if ((q & 15) == 0) p.c_scale[row * (N / kQBlock) + job.n0 / kQBlock] = scale;
      }
    }
  } else {
    // fp32 y in two passes of 128 columns (waves 0-3, then 4-7) through
    // Cs[token][column], stored as 512-byte row segments
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if ((wave >> 2) == half) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              Cs[(m * 16 + r16) * LDC + (wave & 3) * 32 + t * 16 + lgrp * 4 + i] = acc[t][m][i];
      }
      __syncthreads();
      for (int q = tid; q < MT * 16 * 32; q += THREADS) {
        const int r = q >> 5;
        const int c4 = (q & 31) * 4;
        const int n = job.n0 + half * 128 + c4;
        if (r < job.rows_here && n < N) {
          const float* src = Cs + r * LDC + c4;
          float* dst = reinterpret_cast<float*>(gemm_out_row<4>(p, job.row_begin + job.m0 + r));
          if (n + 4 <= N) {
            // y is read once, by the combine
            __builtin_nontemporal_store(f32x4{src[0], src[1], src[2], src[3]},
                                        reinterpret_cast<f32x4*>(dst + n));
          } else {
            for (int i = 0; n + i < N; ++i) dst[n + i] = src[i];
          }
        }
      }
      __syncthreads();
    }
  }
}

template <bool DUAL>
__global__ __launch_bounds__(THREADS, 1) void gemm_fp8s_kernel(GemmLaunch p) {
  constexpr int BN = DUAL ? 128 : 256;  // output columns per block
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  TileJob job;
  if (!find_tile<BM, BN, DUAL, kXcdChunk>(p, job)) return;
  const int mt = (job.rows_here + 63) / 64 * 4;  // token tiles, a multiple of 4
  if (mt <= 4) tile_body<DUAL, 4>(p, job, smem);
  else if (mt <= 8) tile_body<DUAL, 8>(p, job, smem);
  else tile_body<DUAL, 12>(p, job, smem);
}

template <bool DUAL>
hipError_t launch_fp8s(const GemmLaunch& g, hipStream_t st) {
  constexpr int BN = DUAL ? 128 : 256;
  if (g.K % STEP != 0 || g.K / STEP > MAX_KB || g.k_splits > 1 || !g.a_scale) return hipErrorInvalidValue;
  if (DUAL && (g.N % kQBlock != 0 || !g.c_scale)) return hipErrorInvalidValue;
  const int ntn = (g.N + BN - 1) / BN;
  const long long ub_m =
      g.single_group_rows > 0 ? (g.single_group_rows + BM - 1) / BM : g.grid_mtiles_upper;
  const long long total = ub_m * ntn;
  if (total <= 0) return hipSuccess;
  const long long c8 = 8LL * xcd_chunk<kXcdChunk>(total);
  const long long grid = ((total + c8 - 1) / c8) * c8;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_fp8s_kernel<DUAL>), dim3(static_cast<unsigned>(grid)), dim3(THREADS), 0,
                     st, g);
  return hipGetLastError();
}

}  // namespace

bool gemm_fp8s_supported(int a_kind, int out_kind, TileShape ts, bool dual) {
  if (a_kind != K_FP8 || ts.bm != BM) return false;
  if (dual) return out_kind == K_FP8 && ts.bn == 128;
  return out_kind == K_F32 && ts.bn == 256;
}

hipError_t launch_gemm_fp8s(bool dual, const GemmLaunch& g, hipStream_t st) {
  return dual ? launch_fp8s<true>(g, st) : launch_fp8s<false>(g, st);
}

}  // namespace moe
