// Large-tile grouped GEMM for the prefill regime (hundreds of rows per
// expert), bf16 operands, fp32 accumulation (gfx950).
//
// Same computation as the generic kernel in gemm.hip -- gate/up + SwiGLU
// (gmm1 -> swiglu of the Deep Dive §8.2 figure, SwiGLU with packed gate_up
// per the Transformers Dots1 article «并行策略字段») or a plain projection --
// with a tiling chosen for the MFMA roofline:
//
//  * A workgroup of 16 waves (4 per SIMD) owns 128 rows x 512 weight rows;
//    each wave owns 64 rows x 64 weight rows (2 x 2 tiles of
//    v_mfma_f32_32x32x16_bf16, 64 fp32 accumulators per lane).  Sixteen waves
//    per CU are what it takes to keep enough loads in flight: measured on
//    MI355X, streaming throughput per CU grows with the number of issuing
//    waves (about 27 GB/s with 4, 50 with 8, 78 with 16), not with how deep
//    one wave's queue is.
//  * For the gate/up GEMM a wave's 64 weight rows are 32 gate rows and the 32
//    matching up rows, so SiLU(g) * u is formed in registers.
//  * Tiles of A (gathered token rows) and W stream global -> LDS with
//    global_load_lds_dwordx4 (no register staging), double buffered in
//    64-wide K-slices (80 KB each; two fill the 160 KB LDS).  One wait and one
//    fence-free barrier per slice.  16-byte chunks XOR-swizzled by row so the
//    16 lanes of each LDS read phase hit 16 distinct bank groups.
//  * 128 rows per tile keeps the ragged last tile of each expert (about 512
//    rows each at T=16384) to ~12% padding.
#include "gemm_sched.h"

namespace moe {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128;
constexpr int BROWS = 512;               // weight rows per block
constexpr int KS = 64;                   // bf16 elements per K-slice (128 bytes per row)
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

template <int OK, bool DUAL>
__global__ __launch_bounds__(THREADS, 1) void gemm_big_kernel(GemmLaunch p) {
  constexpr int BN = DUAL ? 256 : 512;  // output columns per block
  __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE];

  TileJob job;
  if (!find_tile<BM, BN, DUAL>(p, job)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int K = p.K;
  const int nk = K / KS;
  const int N = p.N;
  const long long rowb_a = p.lda * 2;
  const long long rowb_b = static_cast<long long>(K) * 2;

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
    b_off[i] = static_cast<uint32_t>(wr * rowb_b + lchunk * 16);
  }

  auto issue = [&](int kt) {
    char* base = smem + (kt % NS) * STAGE;
    const int koff = kt * (KS * 2);
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) dma16(a_src[i] + koff, base + (i * WAVES + wave) * 1024);
#pragma unroll
    for (int i = 0; i < B_DMA; ++i)
      dma16(job.W + b_off[i] + koff, base + A_BYTES + (i * WAVES + wave) * 1024);
  };

  // wave (wm, wn): rows [wm*64, +64) x B-tile rows [wn*64, +64)
  const int wm = wave >> 3;
  const int wn = wave & 7;
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue(s);

  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
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
    if (kt + NS - 1 < nk) issue(kt + NS - 1);
    const char* As = smem + (kt % NS) * STAGE;
    const char* Bs = As + A_BYTES;
#pragma unroll
    for (int s = 0; s < KS / 16; ++s) {
      const int ch = s * 2 + lhalf;
      bf16x8 a[2], b[2];
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
        a[tm] = *reinterpret_cast<const bf16x8*>(As + swz(wm * 64 + tm * 32 + lrow, ch));
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
        b[tn] = *reinterpret_cast<const bf16x8*>(Bs + swz(wn * 64 + tn * 32 + lrow, ch));
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[tm], b[tn], acc[tm][tn], 0, 0, 0);
    }
  }

  // ------------------------------------------------------------ epilogue
  // 32x32 accumulator layout: lane l, element i -> row 8*(i/4) + 4*(l/32) + i%4,
  // column l%32 of the 32x32 tile.
  if constexpr (DUAL) {
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
        Cs[r * LDC + c] = g / (1.0f + expf(-g)) * u;
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
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = wm * 64 + tm * 32 + 8 * (i >> 2) + 4 * lhalf + (i & 3);
        if (r >= job.rows_here) continue;
        float* dst = reinterpret_cast<float*>(gemm_out_row<4>(p, job.row_begin + job.m0 + r));
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) {
          const int n = job.n0 + wn * 64 + tn * 32 + lrow;
          if (n < N) dst[n] = acc[tm][tn][i];
        }
      }
  }
}

template <int OK, bool DUAL>
hipError_t launch_big(const GemmLaunch& g, hipStream_t st) {
  constexpr int BN = DUAL ? 256 : 512;
  const int ntn = (g.N + BN - 1) / BN;
  const long long ub_m =
      g.single_group_rows > 0 ? (g.single_group_rows + BM - 1) / BM : g.grid_mtiles_upper;
  const long long total = ub_m * ntn;
  if (total <= 0) return hipSuccess;
  const long long grid = ((total + 7) / 8) * 8;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_big_kernel<OK, DUAL>), dim3(static_cast<unsigned>(grid)), dim3(THREADS),
                     0, st, g);
  return hipGetLastError();
}

}  // namespace

bool gemm_big_supported(int a_kind, int out_kind, TileShape ts, bool dual) {
  if (a_kind != K_BF16 || ts.bm != BM) return false;
  if (dual) return out_kind == K_BF16 && ts.bn == 256;
  return out_kind == K_F32 && ts.bn == 512;
}

hipError_t launch_gemm_big(int out_kind, bool dual, const GemmLaunch& g, hipStream_t st) {
  if (dual && out_kind == K_BF16) return launch_big<K_BF16, true>(g, st);
  if (!dual && out_kind == K_F32) return launch_big<K_F32, false>(g, st);
  return hipErrorInvalidValue;
}

}  // namespace moe
