// Large-tile grouped GEMM for the prefill regime (hundreds of rows per
// expert), bf16 or fp8-e4m3 operands, fp32 accumulation (gfx950).
//
// Same computation as the generic kernel in gemm.hip -- gate/up + SwiGLU
// (gmm1 -> swiglu of the Deep Dive §8.2 figure, SwiGLU with packed gate_up
// per the Transformers Dots1 article «并行策略字段») or a plain projection --
// with a tiling chosen for the MFMA roofline:
//
//  * A workgroup of 16 waves (4 per SIMD) owns 128 rows x 512 weight rows.
//    Sixteen waves per CU are what it takes to keep enough loads in flight:
//    measured on MI355X, streaming throughput per CU grows with the number of
//    issuing waves (about 27 GB/s with 4, 50 with 8, 78 with 16), not with
//    how deep one wave's queue is.
//  * bf16: each wave owns 64 rows x 64 weight rows (2 x 2 tiles of
//    v_mfma_f32_32x32x16_bf16, 64 fp32 accumulators per lane).
//  * fp8: each wave owns 32 rows x 128 weight rows (2 x 8 tiles of
//    v_mfma_scale_f32_16x16x128_f8f6f4, weight rows as the MFMA rows), one
//    instruction per 128-wide scale block, so the per-block scales (row scale
//    of the activations times block scale of the weights, DeepSeek-V3
//    Technical Report, FP8 training section) multiply each partial product
//    once before it is added to the fp32 accumulators.  The gate/up variant
//    quantizes h per token and 128 columns in its epilogue.
//  * For the gate/up GEMM each group of 64 weight rows is 32 gate rows and the
//    32 matching up rows, so SiLU(g) * u is formed on chip.
//  * Tiles of A (gathered token rows) and W stream global -> LDS with
//    global_load_lds_dwordx4 (no register staging), double buffered in
//    128-byte K-slices (64 bf16 or 128 e4m3 per row; 80 KB per stage, two
//    fill the 160 KB LDS).  One wait and one fence-free barrier per slice.
//    16-byte chunks XOR-swizzled by row so the 16 lanes of each LDS read
//    phase hit 16 distinct bank groups.
//  * 128 rows per tile keeps the ragged last tile of each expert (about 512
//    rows each at T=16384) to ~12% padding.
#include "gemm_sched.h"

namespace moe {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128;
constexpr int BROWS = 512;               // weight rows per block
// K-slices are 128 bytes per row: 64 bf16 or 128 e4m3 elements.
constexpr int NS = 2;                    // K-slices resident in LDS
constexpr int WAVES = 16;                // 4 per SIMD
constexpr int THREADS = WAVES * 64;
constexpr int A_BYTES = BM * 128;
constexpr int B_BYTES = BROWS * 128;
constexpr int STAGE = A_BYTES + B_BYTES; // 80 KB; two stages fill the 160 KB LDS
constexpr int A_DMA = A_BYTES / 1024 / WAVES;  // 8-row DMA groups per wave: 1
constexpr int B_DMA = B_BYTES / 1024 / WAVES;  // 4
constexpr int DMA_PER_STAGE = A_DMA + B_DMA;

// LDS is 64 banks x 4 bytes and serves a 128-bit read 16 lanes at a time.
// With 128-byte rows, 16 consecutive rows read at the same logical chunk land
// on 16 distinct 16-byte bank groups when chunk c of row r is stored at
// c ^ ((r >> 1) & 7).
__device__ __forceinline__ int swz_key(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ swz_key(r)) << 4); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One 16-byte chunk per lane, global -> LDS.  The LDS destination of lane i
// is wave_base + 16 * i (wave_base must be wave-uniform).
__device__ __forceinline__ void dma16(const void* g, char* wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)(wave_base), 16, 0, 0);
}

// s_waitcnt vmcnt(n) with the other counters unconstrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads(), which
// would drain every outstanding DMA (vmcnt(0)).  The ordering the pipeline
// needs is explicit: each wave waits for its own slice-kt DMA (wait_vmem)
// before the barrier, and its slice kt-1 LDS reads have been consumed by
// issued MFMAs before it gets there.  The empty asm statements keep the
// compiler from moving LDS accesses across.
__device__ __forceinline__ void barrier_no_fence() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(4))) float* const_f32_ptr;

// PARTN (gate/up only): N is not a multiple of the 256-column tile, so the
// waves of the last n-tile whose columns lie past N skip their work.
template <int AK, int OK, bool DUAL, bool PARTN>
__global__ __launch_bounds__(THREADS, 1) void gemm_big_kernel(GemmLaunch p) {
  constexpr int BN = DUAL ? 256 : 512;  // output columns per block
  constexpr int ESZ = (AK == K_FP8) ? 1 : 2;
  constexpr int KE = 128 / ESZ;         // K elements per 128-byte slice
  __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE];

  TileJob job;
  if (!find_tile<BM, BN, DUAL>(p, job)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index is uniform across the wave: keep it (and what derives from it) scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = p.K;
  int nk = K / KE;
  // split K (projection with fp32 output): this block's K-slices [kt0, kt0 + nk)
  // go to C + blockIdx.y * c_split_stride
  int kt0 = 0;
  if (p.k_splits > 1) {
    nk /= p.k_splits;
    kt0 = blockIdx.y * nk;
    if constexpr (OK == K_F32) {
      p.C = static_cast<float*>(p.C) + blockIdx.y * p.c_split_stride;
      p.C2 = static_cast<float*>(p.C2) + blockIdx.y * p.c_split_stride;
    }
  }
  const int N = p.N;
  const long long rowb_a = p.lda * ESZ;
  const long long rowb_b = static_cast<long long>(K) * ESZ;

  // DMA group g (8 rows x 128 bytes = 1 KB) fills tile rows g*8 + lane/8 at
  // physical chunk lane%8, which holds logical chunk (lane%8) ^ key(row).
  // Groups g = i*WAVES + wave.
  const int rsub = lane >> 3;
  const char* a_src[A_DMA];
#pragma unroll
  for (int i = 0; i < A_DMA; ++i) {
    const int r = (i * WAVES + wave) * 8 + rsub;
    const int lchunk = (lane & 7) ^ swz_key(r);
    const int rr = min(r, job.rows_here - 1);
    const int src = gemm_a_source_row(p, job.row_begin + job.m0 + rr);
    a_src[i] = static_cast<const char*>(p.A) + src * rowb_a + lchunk * 16;
  }
  uint32_t b_off[B_DMA];
  // projection: 8-row weight groups wholly past the last output column are
  // not loaded (their rows would be clamped duplicates no stored output uses)
  bool b_act[B_DMA];
#pragma unroll
  for (int i = 0; i < B_DMA; ++i) b_act[i] = job.n0 + (i * WAVES + wave) * 8 < N;
#pragma unroll
  for (int i = 0; i < B_DMA; ++i) {
    const int r = (i * WAVES + wave) * 8 + rsub;
    const int lchunk = (lane & 7) ^ swz_key(r);
    int wr;
    if constexpr (DUAL) {
      // tile rows [q*64, q*64+64): 32 gate rows then the 32 matching up rows
      const int q = r >> 6, rr = r & 63;
      const int n = min(job.n0 + q * 32 + (rr & 31), N - 1);
      wr = (rr < 32) ? n : N + n;
    } else {
      wr = min(job.n0 + r, N - 1);
    }
    b_off[i] = static_cast<uint32_t>(w_tile_row_off(p.w_tiled, wr, rowb_b) +
                                     w_tile_k_off(p.w_tiled, lchunk * 16));
  }

  // wave (wm, wn): rows [wm*64, +64) x B-tile rows [wn*64, +64)
  const int wm = wave >> 3;
  const int wn = wave & 7;
  const int lrow = lane & 31;
  const int lhalf = lane >> 5;

  // FP8 waves form a 4 x 4 grid instead: wave (wm8, wn8) owns tokens
  // [wm8*32, +32) x B-tile rows [wn8*128, +128), as 2 x 8 tiles of
  // v_mfma_scale_f32_16x16x128_f8f6f4 with the weight rows as the output
  // rows.  Each K-slice is one 128-wide scale block, and a lane's 4
  // accumulators of a tile share one token (its column) and one 128-row
  // weight block, so each partial product takes a single scale product per
  // lane: row scale of A times block scale of W.
  const int wm8 = wave >> 2;
  const int wn8 = wave & 3;
  const int r16 = lane & 15;
  int sa_off[2] = {0, 0};
  float sa_next[2] = {0.f, 0.f};
  const int kblocks = K / kQBlock;
  if constexpr (AK == K_FP8) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int r = min(wm8 * 32 + tt * 16 + r16, job.rows_here - 1);
      sa_off[tt] = gemm_a_source_row(p, job.row_begin + job.m0 + r) * kblocks;
    }
  }

  // FP8 weight block scales of the wave's 128 B-tile rows.  Gate/up: h
  // columns [n0 + wn8*64, +64), all in one 128-block, [0] its gate block and
  // [1] its up block.  Projection: output rows [n0 + wn8*128, +128), one block.
  const float* sb_src[2] = {nullptr, nullptr};
  if constexpr (AK == K_FP8) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      int wr0;
      if constexpr (DUAL) wr0 = (q == 0 ? 0 : N) + min(job.n0 + wn8 * 64, N - 1);
      else wr0 = min(job.n0 + wn8 * 128, N - 1);
      sb_src[q] = job.WS + static_cast<long long>(wr0 / kQBlock) * kblocks;
    }
  }
  // Weight block scales, loaded with the slice's DMA.  Wave-uniform: scalar loads
  // through the constant address space (the scales are read-only here), which
  // keeps them off the vector memory counter that the slice pipeline waits on.
  float sb_next[2] = {0.f, 0.f};
  auto load_sb = [&](int kt) {
    sb_next[0] = ((const_f32_ptr)(sb_src[0]))[kt];
    sb_next[1] = ((const_f32_ptr)(sb_src[1]))[kt];
  };
  auto issue = [&](int kt) {
    char* base = smem + (kt % NS) * STAGE;
    const int koff = (kt0 + kt) * 128;
    // K-slices start on a 64-byte tile column, so slice and chunk offsets add
    const int koff_b = static_cast<int>(w_tile_k_off(p.w_tiled, koff));
#pragma unroll
    for (int i = 0; i < A_DMA; ++i)
      if ((i * WAVES + wave) * 8 < job.rows_here)  // rows past the tile's end are never read
        dma16(a_src[i] + koff, base + (i * WAVES + wave) * 1024);
#pragma unroll
    for (int i = 0; i < B_DMA; ++i)
      if (DUAL || b_act[i]) dma16(job.W + b_off[i] + koff_b, base + A_BYTES + (i * WAVES + wave) * 1024);
    if constexpr (AK == K_FP8) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) sa_next[tt] = p.a_scale[sa_off[tt] + kt0 + kt];
      load_sb(kt0 + kt);
    }
  };

  // FP8 LDS read offsets of this lane: A-tile row wm8*32 + r16 and B-tile row
  // wn8*128 + r16 (+16 per tile), logical chunks c0 and c0+1.  Rows 16 apart
  // share the swizzle key.
  int x_off0 = 0, x_off1 = 0, w_off0 = 0, w_off1 = 0;
  if constexpr (AK == K_FP8) {
    const int c0 = 2 * (lane >> 4);
    const int key = swz_key(r16);
    x_off0 = (wm8 * 32 + r16) * 128 + ((c0 ^ key) << 4);
    x_off1 = (wm8 * 32 + r16) * 128 + (((c0 + 1) ^ key) << 4);
    w_off0 = (wn8 * 128 + r16) * 128 + ((c0 ^ key) << 4);
    w_off1 = (wn8 * 128 + r16) * 128 + (((c0 + 1) ^ key) << 4);
  }
  f32x16 acc[2][2];   // bf16: 2 x 2 tiles of 32x32
  f32x4 acc8[8][2];   // fp8: 8 weight tiles x 2 token tiles of 16x16
  if constexpr (AK == K_FP8) {
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc8[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};
  }

  // whether this wave's row sub-tiles hold rows of the tile and (projection:
  // the router's 256 experts fill half a 512-column tile) whether its weight
  // rows give columns below N; work outside is never stored.  Wave-uniform.
  // Gate/up tiles are tested for columns only when N = I is not a multiple
  // of the tile width (PARTN); a wave's 64 weight rows give h columns
  // [n0 + wn*32, +32) (bf16) or its 128 rows [n0 + wn8*64, +64) (fp8).
  const bool n_act = DUAL ? (!PARTN || job.n0 + wn * 32 < N) : job.n0 + wn * 64 < N;
  const bool m_act[2] = {n_act && wm * 64 < job.rows_here, n_act && wm * 64 + 32 < job.rows_here};
  const bool n_act8 = DUAL ? (!PARTN || job.n0 + wn8 * 64 < N) : job.n0 + wn8 * 128 < N;
  const bool t_act[1] = {n_act8 && wm8 * 32 < job.rows_here};

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue(s);

  for (int kt = 0; kt < nk; ++kt) {
    // slice kt has landed for this thread once only the slices issued after
    // it (at most NS-2 of them) are outstanding
    if constexpr (NS > 2) {
      if (kt + NS - 2 < nk) wait_vmem<(NS - 2) * DMA_PER_STAGE>();
      else wait_vmem<0>();
    } else {
      wait_vmem<0>();
    }
    barrier_no_fence();  // everyone's slice kt landed; slice kt-1's buffer is free
    const float sa_cur[2] = {sa_next[0], sa_next[1]};
    const float sb_cur[2] = {sb_next[0], sb_next[1]};
    if (kt + NS - 1 < nk) issue(kt + NS - 1);
    const char* As = smem + (kt % NS) * STAGE;
    const char* Bs = As + A_BYTES;
    if constexpr (AK == K_FP8) {
      // Lane l holds 32 bytes of row l%16: logical chunks 2*(l/16) and
      // 2*(l/16)+1 of the slice, the same K order for both operands.
      const float sbg = sb_cur[0];
      const float sbu = DUAL ? sb_cur[1] : sbg;
      const float sg[2] = {sa_cur[0] * sbg, sa_cur[1] * sbg};
      const float su[2] = {sa_cur[0] * sbu, sa_cur[1] * sbu};
      // A wave whose 32 tokens all lie past the tile's last row (the ragged
      // tail of an expert) skips the slice: its outputs are never stored.
      if (!t_act[0]) continue;
      i32x8_t xf[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(As + x_off0 + tt * 2048);
        const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(As + x_off1 + tt * 2048);
        xf[tt] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int tw = 0; tw < 8; ++tw) {
        const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(Bs + w_off0 + tw * 2048);
        const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(Bs + w_off1 + tw * 2048);
        const i32x8_t wf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        // gate/up: tiles with (tw & 2) set are up rows
        const bool up = DUAL && (tw & 2);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          // cbsz = blgp = 0: both operands e4m3; E8M0 scales 127 = 2^0
          const f32x4 t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wf, xf[tt], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
          acc8[tw][tt] += t * (up ? su[tt] : sg[tt]);
        }
      }
      continue;
    }
    // 32-row sub-tiles wholly past the tile's last row (the ragged tail of
    // an expert) are skipped: their outputs are never stored
    if (!m_act[0]) continue;
#pragma unroll
    for (int s = 0; s < KE / 16; ++s) {
      const int ch = s * 2 + lhalf;
      bf16x8 a[2], b[2];
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
        if (m_act[tm]) a[tm] = *reinterpret_cast<const bf16x8*>(As + swz(wm * 64 + tm * 32 + lrow, ch));
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
        b[tn] = *reinterpret_cast<const bf16x8*>(Bs + swz(wn * 64 + tn * 32 + lrow, ch));
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
        if (m_act[tm]) {
#pragma unroll
          for (int tn = 0; tn < 2; ++tn)
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[tm], b[tn], acc[tm][tn], 0, 0, 0);
        }
    }
  }

  // ------------------------------------------------------------ epilogue
  // 32x32 accumulator layout: lane l, element i -> row 8*(i/4) + 4*(l/32) + i%4,
  // column l%32 of the 32x32 tile (bf16: rows = tokens, columns = weight rows).
  if constexpr (AK == K_FP8) {
    __syncthreads();  // all waves are done with the operand buffers
    constexpr int LDC = 256 + 4;
    float* Cs = reinterpret_cast<float*>(smem);
    if constexpr (DUAL) {
      // h = SiLU(g) * u into Cs[token][h column], then per token and 128
      // columns: scale = amax / 448, code = e4m3(h / scale)
      // 16x16 layout (weight rows as rows): lane l, element i -> weight row
      // 4*(l/16) + i of the tile, token l%16 of the tile.  B-tile rows
      // [q*64, +64) are 32 gate rows then the 32 matching up rows, so gate
      // tile tw (tw & 2 clear) pairs with up tile tw + 2, h column
      // q*32 + (tw & 1)*16 + row, q = 2*wn8 + tw/4.
#pragma unroll
      for (int tw = 0; tw < 8; ++tw) {
        if (tw & 2) continue;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tok = wm8 * 32 + tt * 16 + r16;
            const int c = (2 * wn8 + (tw >> 2)) * 32 + (tw & 1) * 16 + 4 * (lane >> 4) + i;
            const float g = acc8[tw][tt][i];
            const float u = acc8[tw + 2][tt][i];
            Cs[tok * LDC + c] = silu_mul(g, u);
          }
      }
      __syncthreads();
      static_assert(OK == K_FP8, "FP8 gate/up output is e4m3 + scales");
      for (int q = tid; q < BM * 32; q += THREADS) {
        const int r = q >> 5;
        const int c8 = (q & 31) * 8;  // 16 lanes per 128-column block
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
          if ((q & 15) == 0) p.c_scale[row * (N / kQBlock) + n / kQBlock] = scale;
        }
      }
    } else {
      static_assert(OK == K_F32, "FP8 projection output is fp32");
      // two passes of 256 output columns through Cs[token][column]
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if ((wn8 >> 1) == half) {
#pragma unroll
          for (int tw = 0; tw < 8; ++tw)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int tok = wm8 * 32 + tt * 16 + r16;
                const int c = (wn8 & 1) * 128 + tw * 16 + 4 * (lane >> 4) + i;
                Cs[tok * LDC + c] = acc8[tw][tt][i];
              }
        }
        __syncthreads();
        for (int q = tid; q < BM * 64; q += THREADS) {
          const int r = q >> 6;
          const int c4 = (q & 63) * 4;
          const int n = job.n0 + half * 256 + c4;
          if (r < job.rows_here && n < N) {
            const float* src = Cs + r * LDC + c4;
            float* dst = reinterpret_cast<float*>(gemm_out_row<4>(p, job.row_begin + job.m0 + r));
            if (n + 4 <= N) {
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
  } else if constexpr (DUAL) {
    __syncthreads();  // all waves are done with the operand buffers
    constexpr int LDC = 256 + 4;
    float* Cs = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = wm * 64 + tm * 32 + 8 * (i >> 2) + 4 * lhalf + (i & 3);
        const int c = wn * 32 + lrow;
        const float g = acc[tm][0][i];
        const float u = acc[tm][1][i];
        Cs[r * LDC + c] = silu_mul(g, u);
      }
    __syncthreads();
    static_assert(OK == K_BF16, "gate/up output is bf16 here");
    for (int q = tid; q < BM * 32; q += THREADS) {
      const int r = q >> 5;
      const int c8 = (q & 31) * 8;
      const int n = job.n0 + c8;
      if (r >= job.rows_here || n >= N) continue;
      const float* src = Cs + r * LDC + c8;
      char* dst = gemm_out_row<2>(p, job.row_begin + job.m0 + r);
      if (n + 8 <= N) {
        uint4 o;
        o.x = f32_to_bf16(src[0]) | (static_cast<uint32_t>(f32_to_bf16(src[1])) << 16);
        o.y = f32_to_bf16(src[2]) | (static_cast<uint32_t>(f32_to_bf16(src[3])) << 16);
        o.z = f32_to_bf16(src[4]) | (static_cast<uint32_t>(f32_to_bf16(src[5])) << 16);
        o.w = f32_to_bf16(src[6]) | (static_cast<uint32_t>(f32_to_bf16(src[7])) << 16);
        *reinterpret_cast<uint4*>(dst + static_cast<long long>(n) * 2) = o;
      } else {
        for (int i = 0; n + i < N; ++i)
          reinterpret_cast<uint16_t*>(dst)[n + i] = f32_to_bf16(src[i]);
      }
    }
  } else {
    static_assert(OK == K_F32, "projection output is fp32 here");
    // Staged through LDS in two passes of 256 columns, so that each lane
    // stores 16 bytes and a wave stores one contiguous 1 KB row segment (the
    // accumulator layout would give 4-byte stores, 4x the store instructions).
    __syncthreads();  // all waves are done with the operand buffers
    constexpr int LDC = 256 + 4;
    float* Cs = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if ((wn >> 2) == half) {
#pragma unroll
        for (int tm = 0; tm < 2; ++tm)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = wm * 64 + tm * 32 + 8 * (i >> 2) + 4 * lhalf + (i & 3);
#pragma unroll
            for (int tn = 0; tn < 2; ++tn) Cs[r * LDC + (wn & 3) * 64 + tn * 32 + lrow] = acc[tm][tn][i];
          }
      }
      __syncthreads();
      for (int q = tid; q < BM * 64; q += THREADS) {
        const int r = q >> 6;
        const int c4 = (q & 63) * 4;
        const int n = job.n0 + half * 256 + c4;
        if (r < job.rows_here && n < N) {
          const float* src = Cs + r * LDC + c4;
          float* dst = reinterpret_cast<float*>(gemm_out_row<4>(p, job.row_begin + job.m0 + r));
          if (n + 4 <= N) {
            // y is read once, by the combine: nontemporal stores keep it from
            // evicting the weight tiles the other m-tiles still read from L2
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

template <int AK, int OK, bool DUAL>
hipError_t launch_big(const GemmLaunch& g, hipStream_t st) {
  constexpr int BN = DUAL ? 256 : 512;
  const int ntn = (g.N + BN - 1) / BN;
  const long long ub_m =
      g.single_group_rows > 0 ? (g.single_group_rows + BM - 1) / BM : g.grid_mtiles_upper;
  const long long total = ub_m * ntn;
  if (total <= 0) return hipSuccess;
  const long long grid = ((total + 7) / 8) * 8;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const unsigned splits = g.k_splits > 1 ? static_cast<unsigned>(g.k_splits) : 1u;
  if (DUAL && g.N % BN != 0)
    hipLaunchKernelGGL((gemm_big_kernel<AK, OK, DUAL, true>),
                       dim3(static_cast<unsigned>(grid), splits), dim3(THREADS), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_big_kernel<AK, OK, DUAL, false>),
                       dim3(static_cast<unsigned>(grid), splits), dim3(THREADS), 0, st, g);
  return hipGetLastError();
}

}  // namespace

bool gemm_big_supported(int a_kind, int out_kind, TileShape ts, bool dual) {
  if (ts.bm != BM) return false;
  if (a_kind == K_BF16) {
    if (dual) return out_kind == K_BF16 && ts.bn == 256;
    return out_kind == K_F32 && ts.bn == 512;
  }
  if (a_kind == K_FP8) {
    if (dual) return out_kind == K_FP8 && ts.bn == 256;
    return out_kind == K_F32 && ts.bn == 512;
  }
  return false;
}

hipError_t launch_gemm_big(int a_kind, int out_kind, bool dual, const GemmLaunch& g,
                           hipStream_t st) {
  if (a_kind == K_BF16) {
    if (dual && out_kind == K_BF16) return launch_big<K_BF16, K_BF16, true>(g, st);
    if (!dual && out_kind == K_F32) return launch_big<K_BF16, K_F32, false>(g, st);
  } else if (a_kind == K_FP8) {
    if (dual && out_kind == K_FP8) return launch_big<K_FP8, K_FP8, true>(g, st);
    if (!dual && out_kind == K_F32) return launch_big<K_FP8, K_F32, false>(g, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
