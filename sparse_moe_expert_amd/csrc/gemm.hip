// Grouped MFMA GEMM for the expert FFNs and the router logits (gfx950).
//
// One launch runs every expert ("group") of one projection:
//   gate/up (dual):  h[p, n] = SiLU(Σ_k A[p,k] Wg[n,k]) * (Σ_k A[p,k] Wu[n,k])
//   down / router:   C[p, n] = Σ_k A[p,k] W[n,k]
// where W is the group's nn.Linear weight [N, K] (row n = output feature), so
// each output column reads one contiguous weight row: exactly the K-major
// operand layout the MFMA B operand wants, no repacking.  The SwiGLU form and
// the packed gate/up weight (gate rows first) follow the Transformers Dots1
// article («并行策略字段»: gate_up_proj packed, down_proj; hidden_act silu)
// and the gmm1 -> swiglu -> gmm2 chain of the Deep Dive §8.2 figure.
//
// Tiling: a workgroup of 4 waves computes a BM x BN output tile of one group,
// staging 128-byte K-slices of A and B through LDS (double buffered, XOR
// swizzled 16-byte chunks).  MFMA per operand kind:
//   bf16: v_mfma_f32_16x16x32_bf16          (K 32 per instruction)
//   fp32: v_mfma_f32_16x16x4_f32            (K 4)
//   fp8 : v_mfma_scale_f32_16x16x128_f8f6f4 (K 128, e4m3, unit E8M0 scales)
// FP8 keeps one fp32 accumulator per output and adds each 128-K partial
// product times (row scale of A) * (block scale of W), since the K-slice of a
// stage is exactly one 128-wide scale block.
//
// Schedule: m-tiles of all groups are numbered group by group on the device
// (GroupDesc::tile_begin_*); a block finds its group by binary search.  Block
// ids are remapped so each XCD (blocks are dealt round-robin to the 8 XCDs)
// owns one contiguous run of tiles: the n-tiles of one m-tile, and the m-tiles
// of one expert, then share that XCD's L2.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

template <int AK> struct OpTr;
template <> struct OpTr<K_BF16> {
  static constexpr int ESZ = 2, KSTAGE = 64, KSTEPS = 2, CPL = 1;
};
template <> struct OpTr<K_F32> {
  static constexpr int ESZ = 4, KSTAGE = 32, KSTEPS = 2, CPL = 1;
};
template <> struct OpTr<K_FP8> {
  static constexpr int ESZ = 1, KSTAGE = 128, KSTEPS = 1, CPL = 2;
};

template <int AK>
__device__ __forceinline__ f32x4 mma(const uint4* a, const uint4* b, f32x4 c);

template <>
__device__ __forceinline__ f32x4 mma<K_BF16>(const uint4* a, const uint4* b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                                 __builtin_bit_cast(bf16x8, b[0]), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mma<K_F32>(const uint4* a, const uint4* b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[0].x), __uint_as_float(b[0].x), c,
                                           0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[0].y), __uint_as_float(b[0].y), c,
                                           0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[0].z), __uint_as_float(b[0].z), c,
                                           0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[0].w), __uint_as_float(b[0].w), c,
                                           0, 0, 0);
  return c;
}
template <>
__device__ __forceinline__ f32x4 mma<K_FP8>(const uint4* a, const uint4* b, f32x4 c) {
  i32x8 av = {(int)a[0].x, (int)a[0].y, (int)a[0].z, (int)a[0].w,
              (int)a[1].x, (int)a[1].y, (int)a[1].z, (int)a[1].w};
  i32x8 bv = {(int)b[0].x, (int)b[0].y, (int)b[0].z, (int)b[0].w,
              (int)b[1].x, (int)b[1].y, (int)b[1].z, (int)b[1].w};
  // cbsz = blgp = 0: both operands e4m3; E8M0 scale 127 = 2^0.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, 127, 0, 127);
}

// Byte offset of 16-byte chunk `c` (0..7) of row `r` inside a 128-byte-row tile.
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

__device__ __forceinline__ int a_source_row(const GemmLaunch& p, int row) {
  if (!p.perm) return row;
  if (row < p.R) return p.perm[row] / p.k;
  return (row - p.R) % p.T;
}

template <int OK>
__device__ __forceinline__ char* out_row_ptr(const GemmLaunch& p, long long row) {
  constexpr int OSZ = (OK == K_F32) ? 4 : (OK == K_BF16 ? 2 : 1);
  if (row < p.c_split) return static_cast<char*>(p.C) + row * p.ldc * OSZ;
  return static_cast<char*>(p.C2) + (row - p.c_split) * p.ldc * OSZ;
}

// LO: the A operand is a two-term bf16 split (A + A_lo, the down projection of
// a split h); the A tile then holds BM rows of A followed by BM rows of A_lo.
template <int AK, int OK, int BM, int BN, bool DUAL, bool LO>
struct Cfg {
  using Tr = OpTr<AK>;
  static constexpr int WAVES_M = (BM >= 64) ? 2 : 1;
  static constexpr int WAVES_N = 4 / WAVES_M;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int NB = DUAL ? 2 : 1;
  static constexpr int NA = LO ? 2 : 1;
  static constexpr int BROWS = BN * NB;
  static constexpr int A_BYTES = NA * BM * 128, B_BYTES = BROWS * 128;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_CHUNKS = NA * BM * 8, B_CHUNKS = BROWS * 8;
  static constexpr int A_LOADS = (A_CHUNKS + 255) / 256, B_LOADS = B_CHUNKS / 256;
  static constexpr int LDC = BN + 4;  // fp32 epilogue tile row stride
  static constexpr int EPI_BYTES = BM * LDC * 4;
  static constexpr int SCALE_BYTES = (AK == K_FP8) ? 2 * BM * 4 : 0;
  static constexpr int MAIN_BYTES = 2 * STAGE + SCALE_BYTES;
  static constexpr int SMEM = MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES;
  static_assert(TM >= 1 && TN >= 1, "tile too small for 4 waves");
  static_assert(B_CHUNKS % 256 == 0, "B tile must be a multiple of 32 rows");
  static_assert(128 % BN == 0 || BN % 128 == 0, "BN must tile 128-wide scale blocks");
};

template <int AK, int OK, int BM, int BN, bool DUAL, bool LO>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemmLaunch p) {
  static_assert(!LO || (AK == K_BF16 && OK == K_F32 && !DUAL), "two-term A: bf16 projection");
  using C = Cfg<AK, OK, BM, BN, DUAL, LO>;
  using Tr = typename C::Tr;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // ------------------------------------------------------------ schedule
  const int ntn = (p.N + BN - 1) / BN;
  int total_m;
  if (p.single_group_rows > 0) {
    total_m = (p.single_group_rows + BM - 1) / BM;
  } else {
    total_m = *p.total_mtiles;
  }
  const int total = total_m * ntn;
  const int per_xcd = (total + 7) >> 3;
  const int slot = blockIdx.x >> 3;
  if (slot >= per_xcd) return;
  const int w_id = (blockIdx.x & 7) * per_xcd + slot;
  if (w_id >= total) return;
  const int mt = w_id / ntn;
  const int nt = w_id - mt * ntn;

  int row_begin, rows, tile_begin;
  const char* W;
  const float* WS;
  if (p.single_group_rows > 0) {
    row_begin = 0;
    rows = p.single_group_rows;
    tile_begin = 0;
    W = static_cast<const char*>(p.b_single);
    WS = nullptr;
  } else {
    int lo = 0;
    if (p.mtile_group) {
      lo = p.mtile_group[mt];
    } else {
      int hi = p.num_groups - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        const int tb = DUAL ? p.groups[mid].tile_begin_gu : p.groups[mid].tile_begin_dn;
        if (tb <= mt) lo = mid; else hi = mid - 1;
      }
    }
    const GroupDesc gd = p.groups[lo];
    row_begin = gd.row_begin;
    rows = gd.rows;
    tile_begin = DUAL ? gd.tile_begin_gu : gd.tile_begin_dn;
    W = static_cast<const char*>(DUAL ? gd.w_gu : gd.w_dn);
    WS = DUAL ? gd.s_gu : gd.s_dn;
  }
  const int m0 = (mt - tile_begin) * BM;
  const int rows_here = min(BM, rows - m0);
  const int n0 = nt * BN;
  const int K = p.K;
  // split K: this block's K-stages [kt_begin, kt_end), output at its own offset
  int kt_begin = 0, kt_end = K / Tr::KSTAGE;
  if (p.k_splits > 1) {
    const int per = kt_end / p.k_splits;
    kt_begin = blockIdx.y * per;
    kt_end = kt_begin + per;
    if constexpr (OK == K_F32) {
      p.C = static_cast<float*>(p.C) + blockIdx.y * p.c_split_stride;
      p.C2 = static_cast<float*>(p.C2) + blockIdx.y * p.c_split_stride;
    }
  }
  const long long row_bytes_a = p.lda * Tr::ESZ;
  const long long row_bytes_b = static_cast<long long>(K) * Tr::ESZ;

  // ------------------------------------------------- per-thread load setup
  const char* a_src[C::A_LOADS];
  int a_lds[C::A_LOADS];
  bool a_on[C::A_LOADS];
#pragma unroll
  for (int i = 0; i < C::A_LOADS; ++i) {
    const int q = i * 256 + tid;
    a_on[i] = q < C::A_CHUNKS;
    const int r = a_on[i] ? (q >> 3) : 0;
    const int c = q & 7;
    const bool lo = LO && r >= BM;  // rows [BM, 2BM) of the tile: A_lo
    const int rr = min(lo ? r - BM : r, rows_here - 1);
    const int src = a_source_row(p, row_begin + m0 + rr);
    a_src[i] = static_cast<const char*>(lo ? p.A_lo : p.A) + src * row_bytes_a + c * 16;
    a_lds[i] = swz(r, c);
  }
  const char* b_src[C::B_LOADS];
  int b_lds[C::B_LOADS];
#pragma unroll
  for (int i = 0; i < C::B_LOADS; ++i) {
    const int q = i * 256 + tid;
    const int r = q >> 3;  // 0 .. BROWS-1
    const int c = q & 7;
    const int sb = r / BN;
    const int n = min(n0 + (r - sb * BN), p.N - 1);
    b_src[i] = W + w_tile_row_off(p.w_tiled, sb * p.N + n, row_bytes_b) + w_tile_k_off(p.w_tiled, c * 16);
    b_lds[i] = C::A_BYTES + swz(r, c);
  }
  // FP8: row scales of A (one per row and 128-K block) and the W block scales
  const float* a_scale_src = nullptr;
  if constexpr (AK == K_FP8) {
    if (tid < BM) {
      const int rr = min(tid, rows_here - 1);
      const int src = a_source_row(p, row_begin + m0 + rr);
      a_scale_src = p.a_scale + static_cast<long long>(src) * (K / kQBlock);
    }
  }
  float* s_scale = reinterpret_cast<float*>(smem + 2 * C::STAGE);

  uint4 ra[C::A_LOADS], rb[C::B_LOADS];
  float ras = 0.f;
  auto gload = [&](int kt) {
    const int koff = kt * 128;
    // K-stages start on a 64-byte tile column, so stage and chunk offsets add
    const long long koff_b = w_tile_k_off(p.w_tiled, koff);
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i)
      if (a_on[i]) ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + koff);
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i) rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + koff_b);
    if constexpr (AK == K_FP8) {
      if (tid < BM) ras = a_scale_src[kt];
    }
  };
  auto lstore = [&](int stage) {
    char* base = smem + stage * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i)
      if (a_on[i]) *reinterpret_cast<uint4*>(base + a_lds[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i) *reinterpret_cast<uint4*>(base + b_lds[i]) = rb[i];
    if constexpr (AK == K_FP8) {
      if (tid < BM) s_scale[stage * BM + tid] = ras;
    }
  };

  // ------------------------------------------------------------ main loop
  const int wm0 = (wave / C::WAVES_N) * C::WM;
  const int wn0 = (wave % C::WAVES_N) * C::WN;
  f32x4 acc[C::NB][C::TM][C::TN];
#pragma unroll
  for (int sb = 0; sb < C::NB; ++sb)
#pragma unroll
    for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn) acc[sb][tm][tn] = f32x4{0.f, 0.f, 0.f, 0.f};

  // FP8 block scale of W for this tile: gate block and up block
  const int kblocks = K / kQBlock;
  const float* ws_gate = nullptr;
  const float* ws_up = nullptr;
  if constexpr (AK == K_FP8) {
    ws_gate = WS + static_cast<long long>(n0 / kQBlock) * kblocks;
    ws_up = WS + static_cast<long long>((p.N + n0) / kQBlock) * kblocks;
  }

  gload(kt_begin);
  lstore(0);
  __syncthreads();

  const int lrow = lane & 15;
  const int lgrp = lane >> 4;
  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int cur = (kt - kt_begin) & 1;
    if (kt + 1 < kt_end) gload(kt + 1);
    const char* As = smem + cur * C::STAGE;
    const char* Bs = As + C::A_BYTES;
    float bscale[C::NB];
    f32x4 ascale[C::TM];
    if constexpr (AK == K_FP8) {
      bscale[0] = ws_gate[kt];
      if constexpr (DUAL) bscale[1] = ws_up[kt];
#pragma unroll
      for (int tm = 0; tm < C::TM; ++tm) {
        const float* sc = s_scale + cur * BM + wm0 + tm * 16 + lgrp * 4;
        ascale[tm] = f32x4{sc[0], sc[1], sc[2], sc[3]};
      }
    }
#pragma unroll
    for (int s = 0; s < Tr::KSTEPS; ++s) {
      uint4 af[C::TM][Tr::CPL];
      uint4 af_lo[C::TM];
      uint4 bf[C::NB][C::TN][Tr::CPL];
#pragma unroll
      for (int tm = 0; tm < C::TM; ++tm) {
        const int r = wm0 + tm * 16 + lrow;
#pragma unroll
        for (int c = 0; c < Tr::CPL; ++c) {
          const int ch = (Tr::CPL == 1) ? (s * 4 + lgrp) : (2 * lgrp + c);
          af[tm][c] = *reinterpret_cast<const uint4*>(As + swz(r, ch));
        }
        if constexpr (LO) af_lo[tm] = *reinterpret_cast<const uint4*>(As + swz(BM + r, s * 4 + lgrp));
      }
#pragma unroll
      for (int sb = 0; sb < C::NB; ++sb)
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn) {
          const int r = sb * BN + wn0 + tn * 16 + lrow;
#pragma unroll
          for (int c = 0; c < Tr::CPL; ++c) {
            const int ch = (Tr::CPL == 1) ? (s * 4 + lgrp) : (2 * lgrp + c);
            bf[sb][tn][c] = *reinterpret_cast<const uint4*>(Bs + swz(r, ch));
          }
        }
#pragma unroll
      for (int sb = 0; sb < C::NB; ++sb)
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < C::TN; ++tn) {
            if constexpr (AK == K_FP8) {
              const f32x4 part = mma<AK>(af[tm], bf[sb][tn], f32x4{0.f, 0.f, 0.f, 0.f});
              const f32x4 sc = ascale[tm] * bscale[sb];
              acc[sb][tm][tn] += part * sc;
            } else {
              acc[sb][tm][tn] = mma<AK>(af[tm], bf[sb][tn], acc[sb][tm][tn]);
              if constexpr (LO) acc[sb][tm][tn] = mma<AK>(&af_lo[tm], bf[sb][tn], acc[sb][tm][tn]);
            }
          }
    }
    if (kt + 1 < kt_end) lstore(cur ^ 1);
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogue
  // Stage the fp32 tile in LDS (the operand buffers are free after the final
  // barrier), then write whole rows with 16-byte stores.
  float* Cs = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm0 + tm * 16 + lgrp * 4 + i;
        const int c = wn0 + tn * 16 + lrow;
        float v = acc[0][tm][tn][i];
        if constexpr (DUAL) {
          const float g = v;
          const float u = acc[C::NB - 1][tm][tn][i];
          v = silu_mul(g, u);
        }
        Cs[r * C::LDC + c] = v;
      }
  __syncthreads();

  if constexpr (OK == K_FP8) {
    // Per row and 128 columns: scale = amax / 448, code = e4m3(v / scale).
    static_assert(BN == 128, "FP8 output needs one full 128-column block per tile");
    for (int q = tid; q < BM * 16; q += 256) {
      const int r = q >> 4;
      const int c8 = (q & 15) * 8;
      const float* src = Cs + r * C::LDC + c8;
      float v[8];
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[i] = src[i];
        amax = fmaxf(amax, fabsf(v[i]));
      }
      amax = row16_fmax(amax);
      const float scale = (amax == 0.f) ? 1.0f : amax / 448.0f;
      if (r < rows_here) {
        const long long row = row_begin + m0 + r;
        uint2 codes;
        codes.x = f32x4_to_e4m3(v[0] / scale, v[1] / scale, v[2] / scale, v[3] / scale);
        codes.y = f32x4_to_e4m3(v[4] / scale, v[5] / scale, v[6] / scale, v[7] / scale);
        *reinterpret_cast<uint2*>(out_row_ptr<OK>(p, row) + n0 + c8) = codes;
        if ((q & 15) == 0) p.c_scale[row * (p.N / kQBlock) + n0 / kQBlock] = scale;
      }
    }
  } else if constexpr (OK == K_BF16) {
    for (int q = tid; q < BM * (BN / 8); q += 256) {
      const int r = q / (BN / 8);
      const int c8 = (q % (BN / 8)) * 8;
      if (r >= rows_here) continue;
      const int n = n0 + c8;
      const float* src = Cs + r * C::LDC + c8;
      char* dst = out_row_ptr<OK>(p, row_begin + m0 + r);
      // two-term h: hi = bf16(v), lo = bf16(v - hi) into C_lo (same row)
      char* dst_lo = p.C_lo ? static_cast<char*>(p.C_lo) + (row_begin + m0 + r) * p.ldc * 2 : nullptr;
      if (n + 8 <= p.N && (p.ldc & 7) == 0) {
        uint16_t hi[8], lo[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          hi[i] = f32_to_bf16(src[i]);
          lo[i] = f32_to_bf16(src[i] - bf16_to_f32(hi[i]));
        }
        uint4 o;
        o.x = hi[0] | (static_cast<uint32_t>(hi[1]) << 16);
        o.y = hi[2] | (static_cast<uint32_t>(hi[3]) << 16);
        o.z = hi[4] | (static_cast<uint32_t>(hi[5]) << 16);
        o.w = hi[6] | (static_cast<uint32_t>(hi[7]) << 16);
        *reinterpret_cast<uint4*>(dst + static_cast<long long>(n) * 2) = o;
        if (dst_lo) {
          o.x = lo[0] | (static_cast<uint32_t>(lo[1]) << 16);
          o.y = lo[2] | (static_cast<uint32_t>(lo[3]) << 16);
          o.z = lo[4] | (static_cast<uint32_t>(lo[5]) << 16);
          o.w = lo[6] | (static_cast<uint32_t>(lo[7]) << 16);
          *reinterpret_cast<uint4*>(dst_lo + static_cast<long long>(n) * 2) = o;
        }
      } else {
        for (int i = 0; i < 8 && n + i < p.N; ++i) {
          const uint16_t hi = f32_to_bf16(src[i]);
          reinterpret_cast<uint16_t*>(dst)[n + i] = hi;
          if (dst_lo) reinterpret_cast<uint16_t*>(dst_lo)[n + i] = f32_to_bf16(src[i] - bf16_to_f32(hi));
        }
      }
    }
  } else {
    for (int q = tid; q < BM * (BN / 4); q += 256) {
      const int r = q / (BN / 4);
      const int c4 = (q % (BN / 4)) * 4;
      if (r >= rows_here) continue;
      const int n = n0 + c4;
      const float* src = Cs + r * C::LDC + c4;
      float* dst = reinterpret_cast<float*>(out_row_ptr<OK>(p, row_begin + m0 + r));
      if (n + 4 <= p.N && (p.ldc & 3) == 0) {
        *reinterpret_cast<float4*>(dst + n) = float4{src[0], src[1], src[2], src[3]};
      } else {
        for (int i = 0; i < 4 && n + i < p.N; ++i) dst[n + i] = src[i];
      }
    }
  }
}

template <int AK, int OK, int BM, int BN, bool DUAL>
hipError_t launch_t(const GemmLaunch& g, hipStream_t st) {
  constexpr bool kCanLo = AK == K_BF16 && OK == K_F32 && !DUAL;
  const int ntn = (g.N + BN - 1) / BN;
  const long long ub_m =
      g.single_group_rows > 0 ? (g.single_group_rows + BM - 1) / BM : g.grid_mtiles_upper;
  const long long total = ub_m * ntn;
  if (total <= 0) return hipSuccess;
  const long long grid = ((total + 7) / 8) * 8;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const unsigned splits = g.k_splits > 1 ? static_cast<unsigned>(g.k_splits) : 1u;
  const dim3 gd(static_cast<unsigned>(grid), splits);
  if (g.A_lo) {
    if (!kCanLo) return hipErrorInvalidValue;
    hipLaunchKernelGGL((grouped_gemm_kernel<AK, OK, BM, BN, DUAL, kCanLo>), gd, dim3(256), 0, st, g);
  } else {
    hipLaunchKernelGGL((grouped_gemm_kernel<AK, OK, BM, BN, DUAL, false>), gd, dim3(256), 0, st, g);
  }
  return hipGetLastError();
}

template <int AK, int OK, bool DUAL>
hipError_t launch_shape(TileShape ts, const GemmLaunch& g, hipStream_t st) {
  if constexpr (OK != K_FP8) {
    if (ts.bm == 16 && ts.bn == 64) return launch_t<AK, OK, 16, 64, DUAL>(g, st);
    if (ts.bm == 64 && ts.bn == 64) return launch_t<AK, OK, 64, 64, DUAL>(g, st);
  }
  if (ts.bm == 16 && ts.bn == 128) return launch_t<AK, OK, 16, 128, DUAL>(g, st);
  if (ts.bm == 64 && ts.bn == 128) return launch_t<AK, OK, 64, 128, DUAL>(g, st);
  if (ts.bm == 128 && ts.bn == 128) return launch_t<AK, OK, 128, 128, DUAL>(g, st);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(int a_kind, int out_kind, TileShape ts, const GemmLaunch& g,
                       hipStream_t st) {
  const bool dual = g.dual != 0;
  const bool split = g.k_splits > 1;  // the generic and large-tile kernels split K
  if (split && (out_kind != K_F32 || dual)) return hipErrorInvalidValue;
  if (gemm_prefill_supported(a_kind, out_kind, ts, dual)) {
    if (g.A_lo || g.C_lo) return hipErrorInvalidValue;  // one-term h only
    return launch_gemm_prefill(dual, g, st);
  }
  if (g.c_exp || g.a_exp || g.w16) return hipErrorInvalidValue;  // scaled fp16 h: large-tile kernel only
  if (gemm_fp8s_supported(a_kind, out_kind, ts, dual)) {
    if (g.A_lo || g.C_lo) return hipErrorInvalidValue;
    return launch_gemm_fp8s(dual, g, st);
  }
  if (gemm_big_supported(a_kind, out_kind, ts, dual)) {
    if (g.A_lo || g.C_lo) return hipErrorInvalidValue;  // one-term h only
    return launch_gemm_big(a_kind, out_kind, dual, g, st);
  }
  if (gemm_decode_supported(a_kind, out_kind, ts, dual) && (!split || !dual))
    return launch_gemm_decode(ts, dual, g, st);
  if (a_kind == K_F32 && out_kind == K_F32)
    return dual ? launch_shape<K_F32, K_F32, true>(ts, g, st)
                : launch_shape<K_F32, K_F32, false>(ts, g, st);
  if (a_kind == K_BF16 && out_kind == K_BF16 && dual)
    return launch_shape<K_BF16, K_BF16, true>(ts, g, st);
  if (a_kind == K_BF16 && out_kind == K_F32 && !dual)
    return launch_shape<K_BF16, K_F32, false>(ts, g, st);
  if (a_kind == K_FP8 && out_kind == K_FP8 && dual && ts.bn == 128)
    return launch_shape<K_FP8, K_FP8, true>(ts, g, st);
  if (a_kind == K_FP8 && out_kind == K_F32 && !dual)
    return launch_shape<K_FP8, K_F32, false>(ts, g, st);
  return hipErrorInvalidValue;
}

}  // namespace moe
