// Large-tile grouped bf16 GEMM for the prefill regime (hundreds of rows per
// expert), fp32 accumulation (gfx950).
//
// Same computation as the other grouped GEMM kernels -- gate/up + SwiGLU
// (gmm1 -> swiglu of the Deep Dive §8.2 figure, SwiGLU with packed gate_up
// per the Transformers Dots1 article «并行策略字段») or a plain projection --
// with a schedule built for the MFMA roofline:
//
//  * A workgroup owns 128 rows x 512 weight rows; its waves form a WM x WN
//    grid, each wave a (128/WM) x (512/WN) tile of v_mfma_f32_32x32x16_bf16.
//  * For gate/up, a wave's weight rows are half gate rows and the matching
//    up rows, so SiLU(g) * u is formed on chip.
//  * Operands stream global -> LDS with global_load_lds_dwordx4 (no register
//    staging) in 64-byte K-slices (32 bf16 per row): 8 KB of token rows plus
//    32 KB of weight rows per slice, in a ring of 4 slices (160 KB, the whole
//    LDS), so three slices are in flight while one is multiplied.
//  * Measured (T=16384 gate/up, 4 waves of 128 x 128): the MFMA and LDS-read
//    side alone runs at ~2.07 PFLOP/s, and removing the MFMAs does not change
//    the time: the operand DMA bounds it, and its rate grows with the number
//    of waves that issue it, not with how many loads one wave keeps in
//    flight.  Hence the wave grid is a parameter (the register file bounds
//    it: 8 waves hold 128 accumulators each, 16 waves 64).
//  * The 40 one-KB DMA groups of a slice (16 rows x 64 bytes each) are dealt
//    round-robin to the waves; rows past the end of a tile re-load its last
//    row, and past the last K-slice the ring re-loads that slice into buffers
//    no longer read, so each wave waits for one constant count of loads.
//  * Schedule inside a slice: after the slice barrier each wave multiplies the
//    previous slice's K-step-1 fragments (already in registers) while the DMA
//    of the slice three ahead and this slice's K-step-0 reads are slotted
//    between its MFMAs; then multiplies the K-step-0 fragments with the
//    K-step-1 reads slotted in.  No MFMA waits on a read issued just before.
//  * LDS rows are 64 bytes; chunk c of row r is stored at c ^ ((r >> 2) & 3),
//    so the 16 lanes of each ds_read_b128 phase (16 consecutive rows, one
//    chunk) hit 16 distinct 16-byte bank groups.
//  * 32-row sub-tiles wholly past an expert's last row skip their MFMAs (the
//    ragged last tile of each expert); weight rows past N skip theirs too.
#include "gemm_sched.h"

namespace moe {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int BM = 128;                     // rows per block
constexpr int BROWS = 512;                  // weight rows per block
constexpr int SLICE_B = 64;                 // bytes per row per K-slice
constexpr int KE = SLICE_B / 2;             // bf16 elements per K-slice
constexpr int NS = 4;                       // slices in the LDS ring
constexpr int A_BYTES = BM * SLICE_B;       // 8 KB
constexpr int B_BYTES = BROWS * SLICE_B;    // 32 KB
constexpr int STAGE = A_BYTES + B_BYTES;    // 40 KB
constexpr int A_GROUPS = BM / 16;           // 1 KB DMA groups of a slice: 8 of A
constexpr int GROUPS = STAGE / 1024;        // and 32 of B
// Wave grid: waves along the rows x along the weight rows.  Measured on the
// T=16384 gate/up GEMM: 1 x 4 (128 x 128 per wave) 6.2 ms, 1 x 8 (128 x 64)
// 5.6 ms, 2 x 8 (64 x 64) 5.6 ms, 2 x 4 (64 x 128) 5.7 ms, before the 1 KB
// weight tiles; with them 1 x 8 4.87 ms and 2 x 8 4.94 ms.
constexpr int WM = 1;
constexpr int WN = 8;
constexpr int WAVES = WM * WN;
constexpr int THREADS = WAVES * 64;
constexpr int TM = BM / WM;                 // rows per wave
constexpr int TN = BROWS / WN;              // weight rows per wave
constexpr int MSUB = TM / 32;               // 32-row MFMA sub-tiles per wave
constexpr int NSUB = TN / 32;
constexpr int JMAX = (GROUPS + WAVES - 1) / WAVES;  // DMA groups per wave (at most)
static_assert(MSUB >= 1 && NSUB >= 2 && NSUB % 2 == 0, "wave tile");

__device__ __forceinline__ int swz_key(int r) { return (r >> 2) & 3; }
// byte offset of logical 16-byte chunk c (0..3) of row r inside a tile
__device__ __forceinline__ int swz(int r, int c) { return r * SLICE_B + ((c ^ swz_key(r)) << 4); }

// One 16-byte chunk per lane, global -> LDS at wave_base + 16 * lane.
__device__ __forceinline__ void dma16(const void* g, char* wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)(wave_base), 16, 0, 0);
}

// s_waitcnt vmcnt(n), other counters unconstrained (gfx9 encoding: vmcnt
// bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt lgkmcnt(0), other counters unconstrained.
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads(), which would
// drain every outstanding DMA.  The ordering the ring needs is explicit:
// each wave waits for its own DMA of the slice (wait_vmem) and for its LDS
// reads of the previous slice (wait_lgkm0) before the barrier.
__device__ __forceinline__ void barrier_no_fence() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

struct Frags {
  bf16x8 a[MSUB];
  bf16x8 b[NSUB];
};

// The main loop and epilogue of one tile for a wave that computes MS of its
// MSUB 32-row sub-tiles (the rest lie past the tile's end, or all of them
// when its weight rows lie past N).  Every wave runs the same DMA and
// barrier sequence; cnt = its DMA groups per slice (JMAX or JMAX - 1).
template <bool DUAL, int MS>
__device__ __forceinline__ void tile_body(GemmLaunch& p, const TileJob& job, char* smem, int nk,
                                          int kt0, const char* const* src, const bool* is_a,
                                          int cnt) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int N = p.N;
  // DMA of slice kt into ring buffer kt % NS.  Past the last slice the ring
  // keeps loading (the last slice again, into buffers nothing reads any
  // more), so that every iteration waits for the same count of loads.
  auto issue = [&](int kt) {
    char* base = smem + (kt % NS) * STAGE;
    const int koff = (kt0 + min(kt, nk - 1)) * SLICE_B;
    // a 64-byte K-slice is exactly one tile column of the tiled layout
    const int koff_b = static_cast<int>(w_tile_k_off(p.w_tiled, koff));
#pragma unroll
    for (int j = 0; j < JMAX; ++j)
      if (j < cnt) dma16(src[j] + (is_a[j] ? koff : koff_b), base + (j * WAVES + wave) * 1024);
  };
  auto wait_slice = [&]() {  // slice kt landed: NS - 2 later slices may be in flight
    if (cnt == JMAX) wait_vmem<(NS - 2) * JMAX>();
    else wait_vmem<(NS - 2) * (JMAX - 1)>();
  };

  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  f32x16 acc[MSUB][NSUB];
#pragma unroll
  for (int a = 0; a < MSUB; ++a)
#pragma unroll
    for (int b = 0; b < NSUB; ++b) acc[a][b] = f32x16{};

  auto read = [&](Frags& f, const char* st, int step) {
    const char* As = st;
    const char* Bs = st + A_BYTES;
    const int ch = step * 2 + lhalf;
#pragma unroll
    for (int m = 0; m < MS; ++m)
      f.a[m] = *reinterpret_cast<const bf16x8*>(As + swz(wm * TM + m * 32 + lrow, ch));
    if constexpr (MS > 0) {
#pragma unroll
      for (int n = 0; n < NSUB; ++n)
        f.b[n] = *reinterpret_cast<const bf16x8*>(Bs + swz(wn * TN + n * 32 + lrow, ch));
    }
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int m = 0; m < MS; ++m)
#pragma unroll
      for (int n = 0; n < NSUB; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[m], f.b[n], acc[m][n], 0, 0, 0);
  };
  // Instruction order inside a slice (groups of the scheduler barrier):
  //  1. the previous slice's K-step-1 MFMAs (their fragments are already in
  //     registers), with the DMA of the slice three ahead and then this
  //     slice's K-step-0 reads slotted in, two after each MFMA;
  //  2. this slice's K-step-0 MFMAs, with its K-step-1 reads slotted in one
  //     after each MFMA from the first on.
  // With an LDS DMA of the wave in flight the compiler can only wait for all
  // LDS reads at once (lgkmcnt(0)), so the K-step-1 reads come after the
  // wait that precedes the first K-step-0 MFMA, or that wait would stall on
  // them.
  constexpr int NREAD = MS > 0 ? MS + NSUB : 0;
  constexpr int NMFMA = MS * NSUB;
  auto order = [&]() {
    if constexpr (MS > 0) {
#pragma unroll
      for (int i = 0; i < NMFMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int q = 2 * i + t;
          if (q < JMAX) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM (DMA)
          else if (q - JMAX < NREAD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        }
      }
#pragma unroll
      for (int q = 2 * NMFMA; q < JMAX + NREAD; ++q) {  // what did not fit between them
        if (q < JMAX) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < NMFMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < NREAD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int i = NMFMA; i < NREAD; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  // slices 0 .. NS-2 in flight before the loop
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s);

  Frags f0, f1;
  wait_slice();
  barrier_no_fence();
  issue(NS - 1);
  read(f0, smem, 0);
  read(f1, smem, 1);
  mma(f0);
  for (int kt = 1; kt < nk; ++kt) {
    wait_slice();
    wait_lgkm0();        // this wave's reads of slice kt-1 are in registers
    barrier_no_fence();  // every wave's slice kt landed; slice kt-1's buffer is free
    issue(kt + NS - 1);
    const char* st = smem + (kt % NS) * STAGE;
    read(f0, st, 0);
    mma(f1);  // K-step 1 of slice kt-1
    read(f1, st, 1);
    mma(f0);
    order();
  }
  mma(f1);

  // ------------------------------------------------------------ epilogue
  // 32x32 accumulator layout: lane l, element i -> row 8*(i/4) + 4*(l/32) + i%4,
  // column l%32 of the 32x32 tile (rows = tokens, columns = weight rows).
  __syncthreads();  // all waves are done with the operand ring
  constexpr int LDC = 256 + 4;
  float* Cs = reinterpret_cast<float*>(smem);
  if constexpr (DUAL) {
    // h = SiLU(g) * u into Cs[row][h column]; wave (wm, wn) owns rows
    // [wm*TM, +TM) and h columns [wn*TN/2, +TN/2): n-subtiles j < NSUB/2 are
    // gate columns, j + NSUB/2 the matching up columns
#pragma unroll
    for (int m = 0; m < MS; ++m)
#pragma unroll
      for (int j = 0; j < NSUB / 2; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = wm * TM + m * 32 + 8 * (i >> 2) + 4 * lhalf + (i & 3);
          const int c = wn * (TN / 2) + j * 32 + lrow;
          Cs[r * LDC + c] = silu_mul(acc[m][j][i], acc[m][j + NSUB / 2][i]);
        }
    __syncthreads();
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
    // fp32 output staged through LDS in two passes of 256 columns, so that
    // each lane stores 16 bytes and a wave one contiguous 1 KB row segment
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if ((wn * TN) / 256 == half) {
#pragma unroll
        for (int m = 0; m < MS; ++m)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = wm * TM + m * 32 + 8 * (i >> 2) + 4 * lhalf + (i & 3);
#pragma unroll
            for (int n = 0; n < NSUB; ++n)
              Cs[r * LDC + (wn * TN) % 256 + n * 32 + lrow] = acc[m][n][i];
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
            // evicting the weight slices the other m-tiles still read from L2
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

template <bool DUAL, bool PARTN>
__global__ __launch_bounds__(THREADS, 1) void gemm_prefill_kernel(GemmLaunch p) {
  constexpr int BN = DUAL ? 256 : 512;  // output columns per block
  __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE];

  TileJob job;
  if (!find_tile<BM, BN, DUAL>(p, job)) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int K = p.K;
  int nk = K / KE;
  int kt0 = 0;
  if (p.k_splits > 1) {  // split K (fp32 projection): slices [kt0, kt0 + nk)
    nk /= p.k_splits;
    kt0 = blockIdx.y * nk;
    p.C = static_cast<float*>(p.C) + blockIdx.y * p.c_split_stride;
    p.C2 = static_cast<float*>(p.C2) + blockIdx.y * p.c_split_stride;
  }
  const int N = p.N;
  const long long rowb_a = p.lda * 2;
  const long long rowb_b = static_cast<long long>(K) * 2;

  // DMA group g (16 rows x 64 bytes = 1 KB; groups [0, 8) token rows, [8, 40)
  // weight rows): lane i fills tile row g*16 + i/4 at physical chunk i%4,
  // which holds logical chunk (i%4) ^ key(row); the key of row g*16 + i/4 is
  // (i/16) & 3.  Wave w takes groups g = j*WAVES + w.
  const int rsub = lane >> 2;
  const int lchunk = (lane & 3) ^ ((lane >> 4) & 3);
  const char* src[JMAX];
  bool is_a[JMAX];
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < JMAX; ++j) {
    const int g = j * WAVES + wave;
    cnt += g < GROUPS;
    is_a[j] = g < A_GROUPS;
    if (g < A_GROUPS) {
      const int r = g * 16 + rsub;
      const int srow = gemm_a_source_row(p, job.row_begin + job.m0 + min(r, job.rows_here - 1));
      src[j] = static_cast<const char*>(p.A) + srow * rowb_a + lchunk * 16;
    } else {
      const int r = (min(g, GROUPS - 1) - A_GROUPS) * 16 + rsub;
      int wr;
      if constexpr (DUAL) {
        // weight rows [q*TN, q*TN + TN): TN/2 gate rows, then the matching up rows
        const int q = r / TN, rr = r % TN;
        const int n = min(job.n0 + q * (TN / 2) + rr % (TN / 2), N - 1);
        wr = (rr < TN / 2) ? n : N + n;
      } else {
        wr = min(job.n0 + r, N - 1);
      }
      src[j] = job.W + w_tile_row_off(p.w_tiled, wr, rowb_b) + lchunk * 16;
    }
  }
  // 32-row sub-tiles past the tile's last row, and (projection, or gate/up
  // when N is not a multiple of 256) weight rows past N, are not computed:
  // their outputs are never stored.  Wave-uniform.
  const bool n_act = DUAL ? (!PARTN || job.n0 + wn * (TN / 2) < N) : job.n0 + wn * TN < N;
  const int m_subs = n_act ? max(0, min(MSUB, (job.rows_here - wm * TM + 31) >> 5)) : 0;
  switch (m_subs) {
    case 4: if constexpr (MSUB >= 4) tile_body<DUAL, 4>(p, job, smem, nk, kt0, src, is_a, cnt); break;
    case 3: if constexpr (MSUB >= 3) tile_body<DUAL, 3>(p, job, smem, nk, kt0, src, is_a, cnt); break;
    case 2: if constexpr (MSUB >= 2) tile_body<DUAL, 2>(p, job, smem, nk, kt0, src, is_a, cnt); break;
    case 1: if constexpr (MSUB >= 1) tile_body<DUAL, 1>(p, job, smem, nk, kt0, src, is_a, cnt); break;
    default: tile_body<DUAL, 0>(p, job, smem, nk, kt0, src, is_a, cnt); break;
  }
}

template <bool DUAL>
hipError_t launch_prefill(const GemmLaunch& g, hipStream_t st) {
  constexpr int BN = DUAL ? 256 : 512;
  if (g.K % KE != 0) return hipErrorInvalidValue;
  const int splits = g.k_splits > 1 ? g.k_splits : 1;
  if ((g.K / KE) % splits != 0) return hipErrorInvalidValue;
  const int ntn = (g.N + BN - 1) / BN;
  const long long ub_m =
      g.single_group_rows > 0 ? (g.single_group_rows + BM - 1) / BM : g.grid_mtiles_upper;
  const long long total = ub_m * ntn;
  if (total <= 0) return hipSuccess;
  const long long grid = ((total + 7) / 8) * 8;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 gd(static_cast<unsigned>(grid), static_cast<unsigned>(splits));
  if (DUAL && g.N % BN != 0)
    hipLaunchKernelGGL((gemm_prefill_kernel<DUAL, true>), gd, dim3(THREADS), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_prefill_kernel<DUAL, false>), gd, dim3(THREADS), 0, st, g);
  return hipGetLastError();
}

}  // namespace

bool gemm_prefill_supported(int a_kind, int out_kind, TileShape ts, bool dual) {
  if (a_kind != K_BF16 || ts.bm != BM) return false;
  if (dual) return out_kind == K_BF16 && ts.bn == 256;
  return out_kind == K_F32 && ts.bn == 512;
}

hipError_t launch_gemm_prefill(bool dual, const GemmLaunch& g, hipStream_t st) {
  return dual ? launch_prefill<true>(g, st) : launch_prefill<false>(g, st);
}

}  // namespace moe
