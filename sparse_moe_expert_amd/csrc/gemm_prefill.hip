// Large-tile grouped bf16 GEMM for the prefill regime (hundreds of rows per
// expert), fp32 accumulation (gfx950).
//
// Same computation as the other grouped GEMM kernels -- gate/up + SwiGLU
// (gmm1 -> swiglu of the Deep Dive §8.2 figure, SwiGLU with packed gate_up
// per the Transformers Dots1 article «并行策略字段») or a plain projection --
// with a schedule built for the MFMA roofline:
//
//  * A workgroup of 8 waves owns 128 token rows x 512 weight rows; wave w
//    owns all 128 rows x weight rows [64w, 64w + 64): 8 x 4 tiles of
//    v_mfma_f32_16x16x32_bf16 (128 fp32 accumulators per lane).  For
//    gate/up a wave's weight rows are 32 gate rows and the 32 matching up
//    rows, so SiLU(g) * u is formed on chip.
//  * K advances in 64-byte slices (32 bf16), one MFMA K-step each.
//  * Weight rows are private to their wave, so they go straight from memory
//    into registers: one load instruction per 16-row tile and slice fetches
//    the tile's 16 rows x 64 bytes, which in the 1 KB weight tiles of
//    MOE_LAYOUT_TILED are one contiguous kilobyte and exactly the B operand
//    of the MFMA (lane l: row l % 16, bytes 16 (l / 16) of the slice).  A
//    ring of 3 register slots keeps the loads two slices ahead.
//  * Token rows are shared by all 8 waves and staged through LDS: each wave
//    loads 16 of the 128 rows of a slice into registers three slices ahead,
//    writes them to a 3-slot LDS ring one slice ahead, and after the slice
//    barrier every wave reads its 8 A fragments.  Staging through registers
//    (not the global -> LDS DMA) keeps the LDS traffic at 72 KB per slice
//    (8 KB written, 64 KB read) instead of 136 KB, and lets the compiler wait
//    for each fragment read on its own (with an LDS DMA in flight it can only
//    wait for all of them).
//  * Measured on the T=16384 gate/up GEMM: the same MFMAs and LDS reads run
//    at ~2.07 PFLOP/s without any operand traffic; with both operands staged
//    through LDS by DMA the launch took 4.75 ms, without the LDS reads 3.27 ms.
//  * LDS rows are 64 bytes; chunk c of row r is stored at c ^ ((r >> 1) & 3).
//    Measured with the LDS bank-conflict counter on the fragment reads (16
//    consecutive rows, one chunk per 16 lanes): this key leaves no conflicts
//    (down GEMM 0%, gate/up 11%, from its epilogue), while (r >> 2) & 3,
//    r & 3, (r ^ (r >> 2)) & 3, (r >> 3) & 3 and no swizzle all conflict on
//    40-47% of the LDS cycles.
//  * 32-row sub-tiles wholly past an expert's last row skip their MFMAs (the
//    ragged last tile of each expert); waves whose weight rows lie past N
//    skip their loads and MFMAs.
#include <type_traits>

#include "gemm_sched.h"

namespace moe {
namespace {

constexpr int BM = 128;                 // token rows per block
constexpr int BROWS = 512;              // weight rows per block
constexpr int WAVES = 8;
constexpr int THREADS = WAVES * 64;
constexpr int NT = BROWS / WAVES / 16;  // 16-row weight tiles per wave: 4
constexpr int SLICE_B = 64;             // bytes per row per K-slice
constexpr int KE = SLICE_B / 2;         // bf16 elements per K-slice
constexpr int A_SLOT = BM * SLICE_B;    // 8 KB of token rows per slice
constexpr int U = 3;                    // ring slots: A staging, A in LDS, weights (U - 1 ahead)
constexpr int LDC = 256 + 4;            // fp32 epilogue tile row stride
constexpr int SMEM = BM * LDC * 4;      // epilogue tile; the A ring (24 KB) fits inside
// One block per CU: chunks of 32 consecutive tiles, one per CU of an XCD,
// are dealt round-robin to the XCDs (measured at T=16384: with contiguous
// runs per XCD, the XCD holding the shared expert's tiles ended 7% after
// the others)
constexpr int kXcdChunk = 32;

// 16-byte load through a global (address space 1) pointer: a generic pointer
// read from the group table would compile to a flat load, which the
// compiler must also count as a possible LDS access.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
template <class V>
__device__ __forceinline__ V gload(const void* ptr) {
  static_assert(sizeof(V) == 16, "16-byte loads");
  return __builtin_bit_cast(V, *reinterpret_cast<const __attribute__((address_space(1))) i32x4_t*>(
                                   reinterpret_cast<uintptr_t>(ptr)));
}

__device__ __forceinline__ int swz(int r, int c) {
  return r * SLICE_B + ((c ^ ((r >> 1) & 3)) << 4);
}

// Workgroup barrier after this wave's LDS writes of the slice completed
// (lgkmcnt(0)); no memory fence, so loads in flight stay in flight.
__device__ __forceinline__ void slice_barrier() {
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// 2^-sh as two fp16 (sh >= 0; 0 past fp16's smallest subnormal 2^-24).
__device__ __forceinline__ half2v pow2_neg_f16x2(int sh) {
  const uint32_t b = sh <= 14 ? static_cast<uint32_t>(15 - sh) << 10
                              : (sh <= 24 ? 1u << (24 - sh) : 0u);
  return __builtin_bit_cast(half2v, b | (b << 16));
}

// 8 bf16 -> 8 fp16: exact for |w| in fp16's normal range [2^-14, 65504];
// smaller magnitudes round toward zero to a multiple of 2^-24, larger ones
// saturate at 65504.
__device__ __forceinline__ half8 bf16x8_to_f16(const bf16x8& w) {
  const uint4 u = __builtin_bit_cast(uint4, w);
  const uint32_t d[4] = {u.x, u.y, u.z, u.w};
  half8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto h = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(d[i] << 16),
                                              __uint_as_float(d[i] & 0xffff0000u));
    r[2 * i] = h[0];
    r[2 * i + 1] = h[1];
  }
  return r;
}

// One tile for a wave that computes MS 16-row sub-tiles (an even number up
// to 8; 0: its weight rows lie past N, it only stages token rows).
// F16 (scaled fp16 h): the gate/up GEMM (DUAL) writes h as fp16 codes and
// block exponents (c_exp); the projection reads A that way (a_exp), brings
// each row's blocks to the row's largest exponent while staging them, runs
// fp16 MFMAs with the bf16 weights converted in registers, and scales the
// row by 2^e in its epilogue.  erow: BM ints of LDS outside smem.
// YF16 (projection of fp16 h): y leaves as fp16 codes with exponents per row
// and 256 columns (c_exp); wmax: BM x WAVES floats of LDS for the row maxima.
// W16 (projection of fp16 h): the weights are already fp16 (an fp16 copy
// made at load time by the same conversion), so no per-fragment conversion.
template <bool DUAL, int MS, bool F16, bool YF16, bool W16>
__device__ __forceinline__ void tile_body(GemmLaunch& p, const TileJob& job, char* smem, int nk,
                                          int kt0, int* erow, float* wmax) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = p.N;
  const long long rowb_a = p.lda * 2;
  const long long rowb_b = static_cast<long long>(p.K) * 2;

  // token rows this wave stages: tile rows [16 wave, +16), lane l: row
  // 16 wave + l / 4, 16-byte chunk l % 4 of the slice
  const int ar = wave * 16 + (lane >> 2);
  const int ac = lane & 3;
  const char* a_src = static_cast<const char*>(p.A) +
                      gemm_a_source_row(p, job.row_begin + job.m0 + min(ar, job.rows_here - 1)) * rowb_a +
                      ac * 16;
  const int a_dst = swz(ar, ac);
  // F16 projection: per staging row and block, the fp16 pair 2^-(e_row - e)
  // that brings the block to the row's largest exponent e_row (LDS after the
  // A ring; each slice reads its block's entry before the slice barrier)
  constexpr bool A16 = F16 && !DUAL;
  // scaled fp16 outputs (h of gate/up, y of the projection): weights as the
  // first MFMA operand, so that the accumulators hold the output transposed
  // (4 consecutive output columns of one token row per lane)
  constexpr bool TRN = (DUAL && F16) || YF16;
  static_assert(!YF16 || A16, "fp16 y comes from the projection of fp16 h");
  // bf16 token rows (PAIR, all but the fp16-h projection): one load
  // instruction covers 8 rows x 128 bytes, a pair of slices, so each
  // 128-byte line of a row is read whole by one instruction (two slices of 64
  // bytes read it half by half: gate/up 4.07 -> 3.78 ms at T=16384 in a
  // timing copy).  Lane l reads row 8 h + (l / 4) % 8 of the wave's 16 (h
  // alternates with the iteration) and chunk l % 4 of slice 2 pr + l / 32:
  // 16 consecutive lanes write 4 rows of one slot, on distinct LDS banks.
  // Four LDS slots: a pair's two slices are written while the two before
  // them may still be read.
  constexpr bool PAIR = !A16;
  constexpr int UL = PAIR ? 4 : U;  // LDS slots of token slices
  const char* ap[2] = {nullptr, nullptr};
  int ap_dst[2] = {0, 0};
  if constexpr (PAIR) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = wave * 16 + h * 8 + ((lane >> 2) & 7);
      ap[h] = static_cast<const char*>(p.A) +
              gemm_a_source_row(p, job.row_begin + job.m0 + min(r, job.rows_here - 1)) * rowb_a +
              ((lane >> 5) * 4 + (lane & 3)) * 16;
      ap_dst[h] = (lane >> 5) * A_SLOT + swz(r, lane & 3);
    }
  }
  uint32_t* mult_tab = reinterpret_cast<uint32_t*>(smem + U * A_SLOT);
  const int nb = p.exp_blocks;
  auto mult_of = [&](int kt) __attribute__((always_inline)) {
    return mult_tab[ar * nb + (kt0 + min(kt, nk - 1)) * KE / kHBlock];
  };
  // A16: the staging row's block exponents.  Up to kExpRegs blocks (K up to
  // 2048) they are loaded into registers before the first slices' loads are
  // issued and used after them, so the two memory round trips overlap (the
  // loads complete in order: waiting for the exponents leaves the slices in
  // flight); more blocks are read after the first slices' loads.
  constexpr int kExpRegs = 8;
  const int32_t* ex = nullptr;
  int exv[kExpRegs];
  if constexpr (A16) {
    ex = p.a_exp + static_cast<long long>(job.row_begin + job.m0 + min(ar, job.rows_here - 1)) * nb;
    if (nb <= kExpRegs) {
#pragma unroll
      for (int b = 0; b < kExpRegs; ++b) exv[b] = b < nb ? ex[b] : INT_MIN;
    }
  }
  auto block_shifts = [&]() __attribute__((always_inline)) {
    int e_row = INT_MIN;
    if (nb <= kExpRegs) {
#pragma unroll
      for (int b = 0; b < kExpRegs; ++b) e_row = max(e_row, exv[b]);
#pragma unroll
      for (int b = 0; b < kExpRegs; ++b)
        if (b < nb && (b & 3) == ac)
          mult_tab[ar * nb + b] = __builtin_bit_cast(uint32_t, pow2_neg_f16x2(e_row - exv[b]));
    } else {
      for (int b = 0; b < nb; ++b) e_row = max(e_row, ex[b]);
      for (int b = ac; b < nb; b += 4)
        mult_tab[ar * nb + b] = __builtin_bit_cast(uint32_t, pow2_neg_f16x2(e_row - ex[b]));
    }
    if (ac == 0) erow[ar] = e_row;
    // the shifts of a row are read by the other lanes of this wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // weight tiles of this wave: lane l reads row l % 16 of the tile, bytes
  // [16 (l / 16), +16) of the slice.  Rows past N (a partial last tile, or
  // the router's N = E below 16) read row N - 1 instead: in bounds, and the
  // columns they give are never stored.
  const char* b_src[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int row;
    if constexpr (DUAL) {  // tiles 0, 1: gate rows; 2, 3: the matching up rows
      const int n = min(job.n0 + wave * 32 + (t & 1) * 16 + (lane & 15), N - 1);
      row = t < 2 ? n : N + n;
    } else {
      row = min(job.n0 + wave * 64 + t * 16 + (lane & 15), N - 1);
    }
    b_src[t] = job.W + w_tile_row_off(p.w_tiled, row, rowb_b) + w_tile_k_off(p.w_tiled, (lane >> 4) * 16);
  }
  auto a_off = [&](int kt) __attribute__((always_inline)) { return static_cast<long long>(kt0 + min(kt, nk - 1)) * SLICE_B; };
  auto b_off = [&](int kt) __attribute__((always_inline)) { return w_tile_k_off(p.w_tiled, static_cast<long long>(kt0 + min(kt, nk - 1)) * SLICE_B); };

  uint4 a_stage[U];
  bf16x8 b_ring[U][NT];
  f32x4 acc[8][NT];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_a = [&](uint4& dst, int kt) __attribute__((always_inline)) {
    dst = gload<uint4>(a_src + a_off(kt));
  };
  auto load_b = [&](bf16x8* dst, int kt) __attribute__((always_inline)) {
    if constexpr (MS > 0) {
      const long long o = b_off(kt);
#pragma unroll
      for (int t = 0; t < NT; ++t) dst[t] = gload<bf16x8>(b_src[t] + o);
    }
  };
  // a slice of A into LDS slot `slot`; F16 projection: first multiplied by
  // its block's fp16 pair mbits (exact while the result stays normal)
  auto store_a = [&](uint4 v, int slot, uint32_t mbits) __attribute__((always_inline)) {
    if constexpr (A16) {
      const half2v mult = __builtin_bit_cast(half2v, mbits);
      v.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, v.x) * mult);
      v.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, v.y) * mult);
      v.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, v.z) * mult);
      v.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, v.w) * mult);
    }
    *reinterpret_cast<uint4*>(smem + slot * A_SLOT + a_dst) = v;
  };

  // PAIR: half h of pair pr (slices 2 pr, 2 pr + 1; pairs past the end
  // repeat the last one), and its store into the pair's two LDS slots (the
  // first of them slot0 = 2 pr % 4)
  auto load_pair = [&](uint4& dst, int pr, int h) __attribute__((always_inline)) {
    dst = gload<uint4>(ap[h] + static_cast<long long>(kt0 + min(2 * pr, nk - 2)) * SLICE_B);
  };
  auto store_pair = [&](uint4 v, int slot0, int h) __attribute__((always_inline)) {
    *reinterpret_cast<uint4*>(smem + slot0 * A_SLOT + ap_dst[h]) = v;
  };

  // Slice kt: token rows loaded at iteration kt - 3 into a_stage[kt % 3],
  // written to LDS slot kt % 3 at iteration kt - 1, read at iteration kt;
  // weights loaded at iteration kt - 2 into b_ring[kt % 3].  PAIR: iteration
  // kt loads half kt % 2 of pair (kt + 4) / 2 into a_stage[kt % 3] and stores
  // the register loaded two iterations before (half kt % 2 of pair
  // (kt + 2) / 2), so a pair is in LDS before the iteration of its first
  // slice; slice kt is read from LDS slot kt % 4.  Loads past the last slice
  // fetch the last slice again (never used), so every iteration runs the
  // same instructions.
  // prologue, in the order the iterations would have issued it
  if constexpr (PAIR) {
    uint4 t0, t1;
    load_pair(t0, 0, 0);
    load_pair(t1, 0, 1);
    load_pair(a_stage[1], 1, 0);
    load_b(b_ring[0], 0);
    load_pair(a_stage[2], 1, 1);
    load_b(b_ring[1], 1);
    store_pair(t0, 0, 0);
    store_pair(t1, 0, 1);
  } else {
    load_a(a_stage[0], 0);
#pragma unroll
    for (int j = 1; j < U; ++j) {
      load_a(a_stage[j], j);
      load_b(b_ring[j - 1], j - 1);
    }
    if constexpr (A16) block_shifts();
    store_a(a_stage[0], 0, A16 ? mult_of(0) : 0u);
  }

  auto iter = [&](auto rc, int kt) __attribute__((always_inline)) {
    constexpr int RR = decltype(rc)::value;  // kt % (PAIR ? 12 : U)
    constexpr int R = RR % U;                // register rings
    constexpr int RL = RR % UL;              // LDS slot of slice kt
    const uint32_t mb = A16 ? mult_of(kt + 1) : 0u;  // completes with the barrier's wait
    slice_barrier();                        // slice kt is in LDS for every wave
    if constexpr (PAIR) {
      store_pair(a_stage[(R + 1) % U], (((RR + 2) >> 1) * 2) % 4, RR & 1);
      load_pair(a_stage[R], (kt + 4) >> 1, RR & 1);
    } else {
      store_a(a_stage[(R + 1) % U], (R + 1) % U, mb);
      load_a(a_stage[R], kt + U);
    }
    load_b(b_ring[(R + U - 1) % U], kt + U - 1);
    if constexpr (MS > 0 && (!A16 || W16)) {
      const char* As = smem + RL * A_SLOT;
      // fragments in two halves: the second half's LDS reads run under the
      // first half's MFMAs, and the two halves share registers (fp16 h with
      // fp16 weights: the same schedule with fp16 MFMAs)
      constexpr int MH = MS / 2;
      bf16x8 af[8];
      auto mma = [&](int m, int t) __attribute__((always_inline)) {
        if constexpr (A16) {
          const half8 a = __builtin_bit_cast(half8, af[m]), w = __builtin_bit_cast(half8, b_ring[R][t]);
          acc[m][t] = TRN ? __builtin_amdgcn_mfma_f32_16x16x32_f16(w, a, acc[m][t], 0, 0, 0)
                          : __builtin_amdgcn_mfma_f32_16x16x32_f16(a, w, acc[m][t], 0, 0, 0);
        } else {
          acc[m][t] = TRN ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(b_ring[R][t], af[m], acc[m][t], 0, 0, 0)
                          : __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m], b_ring[R][t], acc[m][t], 0, 0, 0);
        }
      };
#pragma unroll
      for (int m = 0; m < MH; ++m)
        af[m] = *reinterpret_cast<const bf16x8*>(As + swz(m * 16 + (lane & 15), lane >> 4));
#pragma unroll
      for (int m = 0; m < MH; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) mma(m, t);
#pragma unroll
      for (int m = MH; m < MS; ++m)
        af[m] = *reinterpret_cast<const bf16x8*>(As + swz(m * 16 + (lane & 15), lane >> 4));
#pragma unroll
      for (int m = MH; m < MS; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) mma(m, t);
      // instruction order: the first half's fragment reads, the LDS write of
      // a later slice, the first half's MFMAs with the second half's reads
      // after the first four, then the second half's MFMAs; the five global
      // loads spread among the MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, MH, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // DS write
#pragma unroll
      for (int i = 0; i < MS * NT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if (i == MH * NT - 1) __builtin_amdgcn_sched_group_barrier(0x100, MS - MH, 0);  // DS read
        if (i % 4 == 3 && i / 4 < 1 + NT) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM
      }
    }
    if constexpr (MS > 0 && A16 && !W16) {
      // fp16 A fragments; weight tile t converted to fp16 just before its
      // MS MFMAs (weight tile major, so each conversion overlaps the MFMAs
      // of the tile before)
      const char* As = smem + R * A_SLOT;
      half8 af[8];
#pragma unroll
      for (int m = 0; m < MS; ++m)
        af[m] = *reinterpret_cast<const half8*>(As + swz(m * 16 + (lane & 15), lane >> 4));
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const half8 bf = bf16x8_to_f16(b_ring[R][t]);
#pragma unroll
        for (int m = 0; m < MS; ++m)
          acc[m][t] = TRN ? __builtin_amdgcn_mfma_f32_16x16x32_f16(bf, af[m], acc[m][t], 0, 0, 0)
                           : __builtin_amdgcn_mfma_f32_16x16x32_f16(af[m], bf, acc[m][t], 0, 0, 0);
      }
      // instruction order: fragment reads, the LDS write of the next slice,
      // then per weight tile its conversion (12 VALU) and its MS MFMAs, the
      // five global loads spread among them
      __builtin_amdgcn_sched_group_barrier(0x100, MS, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // DS write
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);  // VALU
#pragma unroll
        for (int m = 0; m < MS; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          const int i = t * MS + m;
          if (i % 4 == 3 && i / 4 < 1 + NT) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM
        }
      }
    }
  };
  int kt = 0;
  constexpr int PER = PAIR ? 12 : U;  // the rings' common period
  auto run = [&](auto... rs) __attribute__((always_inline)) {  // PER iterations, RR = 0 .. PER-1
    for (; kt + PER <= nk; kt += PER) (iter(rs, kt + decltype(rs)::value), ...);
    ((kt + decltype(rs)::value < nk ? iter(rs, kt + decltype(rs)::value) : void()), ...);
  };
  [&]<int... Rs>(std::integer_sequence<int, Rs...>) __attribute__((always_inline)) {
    run(std::integral_constant<int, Rs>{}...);
  }(std::make_integer_sequence<int, PER>{});

  // ------------------------------------------------------------ epilogue
  // 16x16 accumulator layout: lane l, element i -> row 4 (l / 16) + i (token),
  // column l % 16 (weight row) of the tile.
  __syncthreads();  // every wave is done with the A ring
  float* Cs = reinterpret_cast<float*>(smem);
  const int lrow = lane & 15;
  const int lgrp = lane >> 4;
  if constexpr (DUAL && F16) {
    // h = SiLU(g) * u from the transposed accumulators: lane l, element i ->
    // h column 32 wave + 16 t + 4 (l / 16) + i of the tile (gate tile t =
    // 0, 1, its up rows in tile t + 2), token row 16 m + l % 16.  The tile's
    // 256 columns are one exponent block: e puts the row's largest
    // |h| * 2^-e in [2^14, 2^15) (0 for a row of zeros).  Weight rows past N
    // repeat row N - 1, so their columns do not change the maximum.
    float rm[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      float v = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[m][t][i] = silu_mul(acc[m][t][i], acc[m][t + 2][i]);
          v = fmaxf(v, fabsf(acc[m][t][i]));
        }
      rm[m] = v;
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) rm[m] = fmaxf(rm[m], __shfl_xor(rm[m], 16, 64));
#pragma unroll
    for (int m = 0; m < 8; ++m) rm[m] = fmaxf(rm[m], __shfl_xor(rm[m], 32, 64));
    if (lgrp == 0) {
#pragma unroll
      for (int m = 0; m < 8; ++m) wmax[(m * 16 + lrow) * WAVES + wave] = rm[m];
    }
    __syncthreads();
    // codes into LDS, rows of 256 fp16 at a 528-byte stride (8-byte writes
    // of the 64 lanes fall on distinct banks)
    constexpr int HROW = 2 * kHBlock + 16;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int r = m * 16 + lrow;
      const f32x4 q0 = *reinterpret_cast<const f32x4*>(wmax + r * WAVES);
      const f32x4 q1 = *reinterpret_cast<const f32x4*>(wmax + r * WAVES + 4);
      const float amax = fmaxf(fmaxf(fmaxf(q0[0], q0[1]), fmaxf(q0[2], q0[3])),
                               fmaxf(fmaxf(q1[0], q1[1]), fmaxf(q1[2], q1[3])));
      const bool scaled = amax > 0.f && amax <= 3.402823466e38f;
      const int x = scaled ? __builtin_amdgcn_frexp_expf(amax) : 15;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        const h4 c = h4{static_cast<_Float16>(ldexpf(acc[m][t][0], 15 - x)),
                        static_cast<_Float16>(ldexpf(acc[m][t][1], 15 - x)),
                        static_cast<_Float16>(ldexpf(acc[m][t][2], 15 - x)),
                        static_cast<_Float16>(ldexpf(acc[m][t][3], 15 - x))};
        *reinterpret_cast<h4*>(smem + r * HROW + (wave * 32 + t * 16 + lgrp * 4) * 2) = c;
      }
      if (wave == 0 && lgrp == 0 && r < job.rows_here)
        p.c_exp[(job.row_begin + job.m0 + r) * static_cast<long long>(p.c_exp_blocks) + job.n0 / kHBlock] =
            scaled ? x - 15 : 0;
    }
    __syncthreads();
    // rows out: half a wave per row (256 columns, 512 bytes)
#pragma unroll
    for (int j = 0; j < BM / WAVES / 2; ++j) {
      const int r = wave * (BM / WAVES) + 2 * j + (lane >> 5);
      const int c8 = (lane & 31) * 8;
      const int n = job.n0 + c8;
      if (r < job.rows_here && n < N) {
        const half8 v = *reinterpret_cast<const half8*>(smem + r * HROW + c8 * 2);
        _Float16* dst = reinterpret_cast<_Float16*>(gemm_out_row<2>(p, job.row_begin + job.m0 + r));
        if (n + 8 <= N) {
          *reinterpret_cast<half8*>(dst + n) = v;
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (n + i < N) dst[n + i] = v[i];
        }
      }
    }
  } else if constexpr (DUAL) {
    // h = SiLU(g) * u into Cs[row][h column]; wave w owns h columns [32w, +32)
#pragma unroll
    for (int m = 0; m < MS; ++m)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Cs[(m * 16 + lgrp * 4 + i) * LDC + wave * 32 + t * 16 + lrow] =
              silu_mul(acc[m][t][i], acc[m][t + 2][i]);
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
  } else if constexpr (YF16) {
    // Scaled fp16 y, one exponent per row and 256 columns (waves 0-3 hold
    // block 0 of the tile, waves 4-7 block 1).  The accumulators hold y
    // transposed: lane l, element i -> output column 64 wave + 16 t +
    // 4 (l / 16) + i, token row 16 m + l % 16, scaled by 2^-erow[row].
    // The codes do not depend on erow: with amax the block's largest |acc|
    // = f 2^x (f in [1/2, 1)), code = acc * 2^(15 - x) and the block
    // exponent is x - 15 + erow (0 for a block of zeros).
    float rm[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      float v = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaxf(v, fabsf(acc[m][t][i]));
      rm[m] = v;
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) rm[m] = fmaxf(rm[m], __shfl_xor(rm[m], 16, 64));
#pragma unroll
    for (int m = 0; m < 8; ++m) rm[m] = fmaxf(rm[m], __shfl_xor(rm[m], 32, 64));
    if (lgrp == 0) {
#pragma unroll
      for (int m = 0; m < 8; ++m) wmax[(m * 16 + lrow) * WAVES + wave] = rm[m];
    }
    __syncthreads();
    // codes into LDS, rows of 512 fp16 at a 1040-byte stride (8-byte writes
    // of the 64 lanes fall on distinct banks)
    constexpr int CROW = LDC * 4;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int r = m * 16 + lrow;
      const f32x4 q = *reinterpret_cast<const f32x4*>(wmax + r * WAVES + (wave & 4));
      const float amax = fmaxf(fmaxf(q[0], q[1]), fmaxf(q[2], q[3]));
      const bool scaled = amax > 0.f && amax <= 3.402823466e38f;
      const int x = scaled ? __builtin_amdgcn_frexp_expf(amax) : 15;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        const h4 c = h4{static_cast<_Float16>(ldexpf(acc[m][t][0], 15 - x)),
                        static_cast<_Float16>(ldexpf(acc[m][t][1], 15 - x)),
                        static_cast<_Float16>(ldexpf(acc[m][t][2], 15 - x)),
                        static_cast<_Float16>(ldexpf(acc[m][t][3], 15 - x))};
        *reinterpret_cast<h4*>(smem + r * CROW + (wave * 64 + t * 16 + lgrp * 4) * 2) = c;
      }
      const int blk0 = job.n0 + (wave & 4) * 64;  // first column of this wave's block
      if ((wave & 3) == 0 && lgrp == 0 && r < job.rows_here && blk0 < N)
        p.c_exp[(job.row_begin + job.m0 + r) * static_cast<long long>(p.c_exp_blocks) + blk0 / kHBlock] =
            scaled ? x - 15 + erow[r] : 0;
    }
    __syncthreads();
    // rows out: a wave stores one row (512 columns, 1 KB) per instruction;
    // y is read once, by the combine
    static_assert(BM % WAVES == 0, "rows split evenly over the waves");
#pragma unroll
    for (int j = 0; j < BM / WAVES; ++j) {
      const int r = wave * (BM / WAVES) + j;
      if (r >= job.rows_here) break;
      const int n = job.n0 + lane * 8;
      const half8 v = *reinterpret_cast<const half8*>(smem + r * CROW + lane * 16);
      _Float16* dst = reinterpret_cast<_Float16*>(gemm_out_row<2>(p, job.row_begin + job.m0 + r));
      if (n + 8 <= N) {
        __builtin_nontemporal_store(__builtin_bit_cast(f32x4, v), reinterpret_cast<f32x4*>(dst + n));
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (n + i < N) dst[n + i] = v[i];
      }
    }
  } else {
    // fp32 output staged through LDS in two passes of 256 columns (waves 0-3,
    // then 4-7), so that each lane stores 16 bytes and a wave one contiguous
    // 1 KB row segment
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if ((wave >> 2) == half) {
#pragma unroll
        for (int m = 0; m < MS; ++m)
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              Cs[(m * 16 + lgrp * 4 + i) * LDC + (wave & 3) * 64 + t * 16 + lrow] = acc[m][t][i];
      }
      __syncthreads();
      for (int q = tid; q < BM * 64; q += THREADS) {
        const int r = q >> 6;
        const int c4 = (q & 63) * 4;
        const int n = job.n0 + half * 256 + c4;
        const float* src = Cs + r * LDC + c4;
        const int ea = A16 ? erow[r] : 0;  // A16: the row's exponent
        const f32x4 o = A16 ? f32x4{ldexpf(src[0], ea), ldexpf(src[1], ea), ldexpf(src[2], ea),
                                    ldexpf(src[3], ea)}
                            : f32x4{src[0], src[1], src[2], src[3]};
        if (r < job.rows_here && n < N) {
          float* dst = reinterpret_cast<float*>(gemm_out_row<4>(p, job.row_begin + job.m0 + r));
          if (n + 4 <= N) {
            // y is read once, by the combine: nontemporal stores keep it from
            // evicting the weight slices the other m-tiles still read from L2
            __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(dst + n));
          } else {
            for (int i = 0; n + i < N; ++i) dst[n + i] = o[i];
          }
        }
      }
      __syncthreads();
    }
  }
}

template <bool DUAL, bool PARTN, bool F16, bool YF16, bool W16 = false>
__global__ __launch_bounds__(THREADS, 1) void gemm_prefill_kernel(GemmLaunch p) {
  constexpr int BN = DUAL ? 256 : 512;  // output columns per block
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  __shared__ int erow[BM];
  // scaled fp16 outputs: row maxima per wave
  __shared__ __attribute__((aligned(16))) float wmax[(YF16 || (DUAL && F16)) ? BM * WAVES : 1];
  static_assert(U * A_SLOT + BM * kMaxHBlocks * 4 <= SMEM,
                "A ring and block shifts inside the epilogue tile");
  static_assert(!DUAL || BN == kHBlock, "one exponent per gate/up tile row");

  TileJob job;
  if (!find_tile<BM, BN, DUAL, kXcdChunk>(p, job)) return;
  if constexpr (W16)  // the group's matrix in the fp16 copy (same layout and size)
    job.W = reinterpret_cast<const char*>(reinterpret_cast<uintptr_t>(job.W) +
                                          (job.row_begin >= p.R ? p.w16_delta_sh : p.w16_delta));

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int nk = p.K / KE;
  int kt0 = 0;
  if (p.k_splits > 1) {  // split K (fp32 projection): slices [kt0, kt0 + nk)
    nk /= p.k_splits;
    kt0 = blockIdx.y * nk;
    p.C = static_cast<float*>(p.C) + blockIdx.y * p.c_split_stride;
    p.C2 = static_cast<float*>(p.C2) + blockIdx.y * p.c_split_stride;
  }
  const int N = p.N;
  // 32-row sub-tiles past the tile's last row, and (projection, or gate/up
  // when N is not a multiple of 256) weight rows past N, are not computed:
  // their outputs are never stored.  Wave-uniform.
  const bool n_act = DUAL ? (!PARTN || job.n0 + wave * 32 < N) : job.n0 + wave * 64 < N;
  const int ms = n_act ? min(4, (job.rows_here + 31) >> 5) * 2 : 0;
  switch (ms) {
    case 8: tile_body<DUAL, 8, F16, YF16, W16>(p, job, smem, nk, kt0, erow, wmax); break;
    case 6: tile_body<DUAL, 6, F16, YF16, W16>(p, job, smem, nk, kt0, erow, wmax); break;
    case 4: tile_body<DUAL, 4, F16, YF16, W16>(p, job, smem, nk, kt0, erow, wmax); break;
    case 2: tile_body<DUAL, 2, F16, YF16, W16>(p, job, smem, nk, kt0, erow, wmax); break;
    default: tile_body<DUAL, 0, F16, YF16, W16>(p, job, smem, nk, kt0, erow, wmax); break;
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
  const long long c8 = 8LL * xcd_chunk<kXcdChunk>(total);
  const long long grid = ((total + c8 - 1) / c8) * c8;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 gd(static_cast<unsigned>(grid), static_cast<unsigned>(splits));
  // scaled fp16: gate/up writes h that way (c_exp); the projection reads A
  // = h that way (a_exp) and, in the layer, writes y that way too (c_exp)
  const bool f16 = DUAL ? g.c_exp != nullptr : g.a_exp != nullptr;
  const bool yf16 = !DUAL && g.c_exp != nullptr;
  if (g.a_exp && (g.exp_blocks != (g.K + kHBlock - 1) / kHBlock || g.exp_blocks > kMaxHBlocks ||
                  g.k_splits > 1))
    return hipErrorInvalidValue;
  if (g.c_exp && g.c_exp_blocks != (g.N + kHBlock - 1) / kHBlock) return hipErrorInvalidValue;
  if (yf16 && !f16) return hipErrorInvalidValue;  // fp16 y only from fp16 h
  // bf16 token rows go in pairs of slices: an even slice count per block
  // (K a multiple of 64 elements per split; H and I are multiples of 128)
  if (!(f16 && !DUAL) && (g.K / KE / splits) % 2 != 0) return hipErrorInvalidValue;
  const bool w16 = !DUAL && g.w16;
  if ((g.w16 && DUAL) || (w16 && !f16)) return hipErrorInvalidValue;  // fp16 weights meet fp16 h only
  if constexpr (!DUAL) {
    if (w16) {
      if (yf16)
        hipLaunchKernelGGL((gemm_prefill_kernel<DUAL, false, true, true, true>), gd, dim3(THREADS), 0, st, g);
      else
        hipLaunchKernelGGL((gemm_prefill_kernel<DUAL, false, true, false, true>), gd, dim3(THREADS), 0, st, g);
      return hipGetLastError();
    }
  }
  if (DUAL && g.N % BN != 0) {
    if (f16)
      hipLaunchKernelGGL((gemm_prefill_kernel<DUAL, true, true, false>), gd, dim3(THREADS), 0, st, g);
    else
      hipLaunchKernelGGL((gemm_prefill_kernel<DUAL, true, false, false>), gd, dim3(THREADS), 0, st, g);
  } else if (yf16) {
    hipLaunchKernelGGL((gemm_prefill_kernel<DUAL, false, true, !DUAL>), gd, dim3(THREADS), 0, st, g);
  } else if (f16) {
    hipLaunchKernelGGL((gemm_prefill_kernel<DUAL, false, true, false>), gd, dim3(THREADS), 0, st, g);
  } else {
    hipLaunchKernelGGL((gemm_prefill_kernel<DUAL, false, false, false>), gd, dim3(THREADS), 0, st, g);
  }
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
