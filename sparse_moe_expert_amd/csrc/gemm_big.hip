// Large-tile grouped GEMM for the prefill regime (hundreds of rows per
// expert), bf16 operands, fp32 accumulation (gfx950).
//
// Same computation as the generic kernel in gemm.hip -- gate/up + SwiGLU
// (gmm1 -> swiglu of the Deep Dive §8.2 figure, SwiGLU with packed gate_up
// per the Transformers Dots1 article «并行策略字段») or a plain projection --
// with a tiling chosen for the MFMA roofline:
//
//  * A workgroup (4 waves) owns 128 rows x 512 weight rows.  Each wave owns
//    all 128 rows x 128 weight rows: 4 x 4 tiles of v_mfma_f32_32x32x16_bf16,
//    256 fp32 accumulators per lane.  A 128 x 128 wave tile reads 512 bytes of
//    LDS per k per wave, about half of the LDS bandwidth at the MFMA peak.
//  * For the gate/up GEMM a wave's 128 weight rows are 64 gate rows and the 64
//    matching up rows, so SiLU(g) * u is formed in registers.
//  * Tiles of A (gathered token rows) and W stream global -> LDS with
//    global_load_lds_dwordx4 (no register staging), double buffered: the DMA
//    of K-slice kt+1 overlaps the MFMAs of slice kt; one wait + barrier per
//    slice.  128-byte rows, 16-byte chunks XOR-swizzled by row so that the
//    8 lanes of each LDS access phase hit 8 distinct bank groups.
//  * 128 rows per tile keeps the ragged last tile of each expert (about 512
//    rows each at T=16384) to ~12% padding.
#include "gemm_sched.h"

namespace moe {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128;
constexpr int BROWS = 512;               // weight rows per block
constexpr int A_BYTES = BM * 128;        // one 64-element bf16 K-slice per row
constexpr int B_BYTES = BROWS * 128;
constexpr int STAGE = A_BYTES + B_BYTES; // 80 KB; two stages fill the 160 KB LDS

__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One 16-byte chunk per lane, global -> LDS.  The LDS destination of lane i
// is wave_base + 16 * i (wave_base must be wave-uniform).
__device__ __forceinline__ void dma16(const void* g, char* wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)(wave_base), 16, 0, 0);
}

// s_waitcnt vmcnt(0), other counters unconstrained (gfx9 encoding).
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int OK, bool DUAL>
__global__ __launch_bounds__(256, 1) void gemm_big_kernel(GemmLaunch p) {
  constexpr int BN = DUAL ? 256 : 512;  // output columns per block
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  TileJob job;
  if (!find_tile<BM, BN, DUAL>(p, job)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int K = p.K;
  const int nk = K / 64;
  const int N = p.N;
  const long long rowb_a = p.lda * 2;
  const long long rowb_b = static_cast<long long>(K) * 2;

  // DMA instruction i of this wave fills tile rows (i*4 + wave)*8 + lane/8,
  // physical chunk lane%8, which holds logical chunk (lane%8) ^ (row%8).
  const int rsub = lane >> 3;
  const int lchunk = (lane & 7) ^ rsub;
  const char* a_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (i * 4 + wave) * 8 + rsub;
    const int rr = min(r, job.rows_here - 1);
    const int src = gemm_a_source_row(p, job.row_begin + job.m0 + rr);
    a_src[i] = static_cast<const char*>(p.A) + src * rowb_a + lchunk * 16;
  }
  uint32_t b_off[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = (i * 4 + wave) * 8 + rsub;
    int wr;
    if constexpr (DUAL) {
      const int q = r >> 7, rr = r & 127;
      const int n = min(job.n0 + q * 64 + (rr & 63), N - 1);
      wr = (rr < 64) ? n : N + n;
    } else {
      wr = min(job.n0 + r, N - 1);
    }
    b_off[i] = static_cast<uint32_t>(wr * rowb_b + lchunk * 16);
  }

  auto issue = [&](int kt, int buf) {
    char* base = smem + buf * STAGE;
    const int koff = kt * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(a_src[i] + koff, base + (i * 4 + wave) * 1024);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      dma16(job.W + b_off[i] + koff, base + A_BYTES + (i * 4 + wave) * 1024);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

  issue(0, 0);
  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmem_all();   // this thread's DMA for slice kt has landed
    __syncthreads();   // ... everyone's has; and slice kt-1's buffer is free
    if (kt + 1 < nk) issue(kt + 1, (kt + 1) & 1);
    const char* As = smem + (kt & 1) * STAGE;
    const char* Bs = As + A_BYTES;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = s * 2 + lhalf;
      bf16x8 a[4], b[4];
#pragma unroll
      for (int tm = 0; tm < 4; ++tm)
        a[tm] = *reinterpret_cast<const bf16x8*>(As + swz(tm * 32 + lrow, ch));
#pragma unroll
      for (int tn = 0; tn < 4; ++tn)
        b[tn] = *reinterpret_cast<const bf16x8*>(Bs + swz(wave * 128 + tn * 32 + lrow, ch));
#pragma unroll
      for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
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
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = tm * 32 + 8 * (i >> 2) + 4 * lhalf + (i & 3);
          const int c = wave * 64 + tn * 32 + lrow;
          const float g = acc[tm][tn][i];
          const float u = acc[tm][tn + 2][i];
          Cs[r * LDC + c] = g / (1.0f + expf(-g)) * u;
        }
    __syncthreads();
    static_assert(OK == K_BF16, "gate/up output is bf16 here");
    for (int q = tid; q < BM * 32; q += 256) {
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
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = tm * 32 + 8 * (i >> 2) + 4 * lhalf + (i & 3);
        if (r >= job.rows_here) continue;
        float* dst = reinterpret_cast<float*>(gemm_out_row<4>(p, job.row_begin + job.m0 + r));
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
          const int n = job.n0 + wave * 128 + tn * 32 + lrow;
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
  hipLaunchKernelGGL((gemm_big_kernel<OK, DUAL>), dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     st, g);
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
