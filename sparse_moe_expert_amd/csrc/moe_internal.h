// Internal declarations shared by the host entry points and the kernel files
// of libmoe (gfx950).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "moe.h"

namespace moe {

// Element kinds of GEMM operands and outputs.
enum Kind : int { K_F32 = 0, K_BF16 = 1, K_FP8 = 2 };

constexpr int kMaxExperts = 512;
constexpr int kMaxShared = 4;
constexpr int kMaxTopK = 16;
constexpr int kQBlock = 128;          // FP8 scale granularity along K
constexpr int kDispatchChunk = 1024;  // flat (token, slot) pairs per dispatch wave
constexpr float kTieEps = 1e-6f;
constexpr int kFp8MinI = 512;         // smallest intermediate size run in FP8
constexpr int kHBlock = 256;          // h columns per exponent of the scaled fp16 h
constexpr int kMaxHBlocks = 64;       // so I <= 16384 on the large-tile bf16 path

// One GEMM group = one expert (routed e < E, shared E + s) over a contiguous
// range of rows of the sorted row space.  Rows [0, R) are the routed (token,
// slot) pairs in expert order (R = T*k); rows R + s*T + t are token t of
// shared expert s.  Built on the device from the dispatch offsets.
struct GroupDesc {
  int32_t row_begin;
  int32_t rows;
  int32_t tile_begin_gu;  // first m-tile id of this group in the gate/up GEMM
  int32_t tile_begin_dn;  // first m-tile id of this group in the down GEMM
  const void* w_gu;       // [2I, H] weights of this expert
  const float* s_gu;      // [2I/128, H/128] block scales (FP8) or null
  const void* w_dn;       // [H, I]
  const float* s_dn;      // [H/128, I/128] or null
};

// Per-GEMM tile shapes chosen on the host from the config (no device sync).
struct TileShape {
  int bm;  // rows per tile
  int bn;  // output columns per tile
};

// Byte offsets of every buffer inside the caller's workspace.
struct Layout {
  size_t logits;        // [router_splits, T, E] fp32 (split-K partial sums)
  size_t topk_idx;      // [T, k] int32
  size_t topk_w;        // [T, k] fp32
  size_t counts;        // [E] int32
  size_t offsets;       // [E + 1] int32
  size_t perm;          // [T*k] int32
  size_t inv;           // [T*k] int32
  size_t chunk_counts;  // [nchunks, E] int32
  size_t chunk_base;    // [nchunks, E] int32
  size_t groups;        // [E + S] GroupDesc
  size_t totals;        // [4] int32: m-tiles of gate/up, m-tiles of down
  size_t mtg_gu;        // [m-tile upper bound] int32: group of each gate/up m-tile
  size_t mtg_dn;        // [m-tile upper bound] int32: group of each down m-tile
  size_t xq;            // FP8: [T, H] e4m3 codes
  size_t xs;            // FP8: [T, H/128] fp32 scales
  size_t h;             // [R + S*T, I] act type, or e4m3 codes (FP8)
  size_t hlo;           // bf16 h_split: [R + S*T, I] bf16 residue h - bf16(h)
  size_t hexp;          // bf16 h_f16: [R + S*T, ceil(I / kHBlock)] int32 block exponents
  size_t yexp;          // bf16 h_f16: [R + S*T, ceil(H / kHBlock)] int32 exponents of y, y_sh
  size_t hs;            // FP8: [R + S*T, I/128] fp32 scales
  size_t y;             // [R, H] fp32  (routed expert outputs, sorted)
  size_t ysh;           // [S, T, H] fp32
  size_t xn;            // [T, H] act type: the normalised input of a block forward
  size_t fbar;          // [2] uint32: the single-launch layer's barrier counter and status
  size_t total;
  int nchunks;
  int router_splits;    // >= 1
  bool h_split;         // bf16 h kept as hi + lo (down GEMM on an HBM-bound kernel)
  bool h_f16;           // bf16 experts on the large-tile kernel: h as scaled fp16
  TileShape gu, dn, router;
};

Layout make_layout(const moe_config_t& c);

inline size_t kind_size(int kind) { return kind == K_F32 ? 4 : kind == K_BF16 ? 2 : 1; }

// Tiled weight storage: a row-major [rows, K] matrix (rows a multiple of 16,
// K * element size a multiple of 64 bytes) cut into 16-row x 64-byte tiles
// of 1 KB.  Tiles are stored row group by row group, and along K inside a
// row group.  Inside a tile the 16-byte chunks go chunk-major: chunk c (bytes
// [16 c, 16 c + 16) of the tile's 64) of tile row r sits at 256 c + 16 r.
// The MFMA operand fragment of a 16-row tile and 64-byte K step gives lane l
// row l % 16 and chunk l / 16, so one load instruction of 64 lanes x 16 bytes
// reads the whole tile with lane l at byte 16 l: 1 KB contiguous, in lane
// order.  The byte offset of (row, byte b of the row) splits into a row part
// and a K part, which the kernels add separately; for K offsets that are
// multiples of 64 the K part is additive (w_tile_k_off(a + b) =
// w_tile_k_off(a) + w_tile_k_off(b) when a % 64 == 0).
constexpr int kTileRows = 16;
constexpr int kTileBytes = 64;
__host__ __device__ inline long long w_tile_row_off(int tiled, int row, long long row_bytes) {
  return tiled ? static_cast<long long>(row >> 4) * (row_bytes * kTileRows) + (row & 15) * 16
               : static_cast<long long>(row) * row_bytes;
}
__host__ __device__ inline long long w_tile_k_off(int tiled, long long kbyte) {
  return tiled ? (kbyte >> 6) * (kTileRows * kTileBytes) + ((kbyte & 63) >> 4) * (kTileRows * 16) + (kbyte & 15)
               : kbyte;
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  All take the caller's stream.

struct GemmLaunch {
  // schedule
  const GroupDesc* groups;
  int num_groups;
  const int32_t* total_mtiles;  // device scalar: m-tiles over all groups
  int dual;                     // 1: gate/up GEMM (uses w_gu), 0: down (w_dn)
  int single_group_rows;        // >0: one implicit group of this many rows
                                // (router), weights in b_single
  const void* b_single;
  int grid_mtiles_upper;        // host upper bound of m-tiles
  const int32_t* mtile_group;   // group of each m-tile (device), or null:
                                // then a binary search over the groups
  // shapes
  int N;  // output columns (h columns for the gate/up GEMM)
  int K;  // reduction length
  // A operand
  const void* A;
  long long lda;           // elements
  const float* a_scale;    // FP8: [rows of A, K/128]
  const int32_t* perm;     // gather: A row of sorted row p < R is perm[p] / k
  int R, k, T;
  // outputs
  void* C;                 // rows [0, c_split)
  void* C2;                // rows [c_split, ...) at C2 + (row - c_split) * ldc
  long long c_split;
  long long ldc;
  float* c_scale;          // FP8 output scales [rows, N/128]
  // two-term bf16 h (gate/up writes, down reads; null = one term): the gate/up
  // output v is stored as hi = bf16(v) in C and lo = bf16(v - hi) in C_lo (same
  // row indexing, no C2 split); the down GEMM adds W * A_lo to W * A, A_lo
  // with the stride and row mapping of A
  void* C_lo;
  const void* A_lo;
  // scaled fp16 (large-tile kernel only; null = not used): an output v is
  // stored as fp16 v * 2^-e, e per row and block of kHBlock columns chosen so
  // that the block's largest |v| * 2^-e lies in [2^14, 2^15), with e in
  // c_exp [rows of the sorted row space, c_exp_blocks] (gate/up: h; down in
  // the layer: y); the down GEMM reads A = h that way through a_exp
  // [rows, exp_blocks]
  int32_t* c_exp;
  int c_exp_blocks;
  const int32_t* a_exp;
  int exp_blocks;
  // split K (generic kernel, fp32 output only): block y computes the K range
  // [y * K / k_splits, (y + 1) * K / k_splits) into C + y * c_split_stride
  int k_splits;            // 0 or 1: no split
  long long c_split_stride;  // elements
  // expert weights (groups' w_gu / w_dn) stored as 16-row x 64-byte tiles
  // (w_tile_row_off / w_tile_k_off); the router's b_single is always row-major
  int w_tiled;
  // fp16 copy of the down weights (large-tile down GEMM of scaled fp16 h
  // only; 0 = convert the bf16 fragments in registers).  The copy has w_dn's
  // layout and size, so a group's fp16 matrix lies at its bf16 address plus
  // the difference of the two bases: w16_delta for routed groups, and
  // w16_delta_sh for shared ones (rows >= R).
  int w16;
  long long w16_delta;
  long long w16_delta_sh;
};

hipError_t launch_gemm(int a_kind, int out_kind, TileShape ts, const GemmLaunch& g,
                       hipStream_t st);
// n bf16 values -> fp16, rounded toward zero (moe_convert_bf16_to_f16);
// n a multiple of 8, 16-byte aligned buffers.
hipError_t launch_convert_bf16_f16(const void* src, void* dst, long long n, hipStream_t st);
// Large-tile bf16 kernel (gemm_prefill.hip): 128 rows x 256 h-columns
// (gate/up) or 128 rows x 512 output columns (projection), bf16 operands.
bool gemm_prefill_supported(int a_kind, int out_kind, TileShape ts, bool dual);
hipError_t launch_gemm_prefill(bool dual, const GemmLaunch& g, hipStream_t st);
// Large-tile fp8 kernel (gemm_big.hip), same tile shapes.
// Weight-streaming FP8 kernel (gemm_fp8.hip): 192 token rows x 128 h-columns
// (gate/up) or 192 rows x 256 output columns (projection), e4m3 operands.
bool gemm_fp8s_supported(int a_kind, int out_kind, TileShape ts, bool dual);
hipError_t launch_gemm_fp8s(bool dual, const GemmLaunch& g, hipStream_t st);
bool gemm_big_supported(int a_kind, int out_kind, TileShape ts, bool dual);
hipError_t launch_gemm_big(int a_kind, int out_kind, bool dual, const GemmLaunch& g,
                           hipStream_t st);
// Weight-streaming bf16 kernel (gemm_decode.hip): 16 or 32 rows x 64
// h-columns (gate/up) or x 128 output columns (projection).
bool gemm_decode_supported(int a_kind, int out_kind, TileShape ts, bool dual);
hipError_t launch_gemm_decode(TileShape ts, bool dual, const GemmLaunch& g, hipStream_t st);

// logits: `splits` partial sums [splits][T][E] (added in split order).
hipError_t launch_router_topk(const float* logits, int splits, const float* bias, int T, int E,
                              int k, int n_group, int topk_group, int norm, float rsf, int32_t* idx,
                              float* w, int32_t* ties, hipStream_t st);
// Single-launch layer for the decode regime (fused.hip): one cooperative
// persistent grid runs router logits, top-k, dispatch and the tile table,
// both weight-streaming GEMMs and the combine, with grid barriers between.
struct FusedArgs {
  int T, H, E, S, k, I, n_group, topk_group, norm;
  float rsf;
  const uint16_t* x;         // [T, H] bf16
  const uint16_t* w_router;  // [E, H] bf16
  const float* bias;         // [E]
  float* logits;             // [splits, T, E]
  int splits;                // K split of the router logits (H / splits % 32 == 0)
  int32_t* idx;              // [T, k]
  float* tw;                 // [T, k]
  int32_t* ties;             // [2] or null
  int32_t* counts;           // [E]
  int32_t* offsets;          // [E + 1]
  int32_t* perm;             // [T*k]
  int32_t* inv;              // [T*k]
  GroupDesc* groups;         // [E + S]
  int32_t* totals;           // [2]: m-tiles of gate/up and down
  int32_t* mtg_gu;           // m-tile -> group tables of the two GEMMs
  int32_t* mtg_dn;
  const char* w_gu;
  const char* w_dn;
  const char* w_sh_gu;
  const char* w_sh_dn;
  TileShape tgu, tdn;        // decode tile shapes (bm 16, NT 4)
  GemmLaunch gu, dn;         // the two grouped GEMMs (tables above)
  const float* y;            // [T*k, H] fp32 (= dn.C)
  const float* ysh;          // [S, T, H] fp32 (= dn.C2)
  const void* residual;      // null or [T, H] bf16
  void* out;                 // [T, H] bf16
  uint32_t* bar;             // [2] in the workspace: barrier arrivals, status (1: a wait timed out)
  long long spin_limit;      // polls per grid barrier before a block gives up
};
bool fused_decode_supported(TileShape gu, TileShape dn);
hipError_t launch_fused_decode(const FusedArgs& a, hipStream_t st);

// RMSNorm rows of [T, H] (act kind F32 or BF16), fp32 math, one rounding.
// pack.hip: `count` row-major [rows, row_bytes] matrices -> tiled storage
hipError_t launch_pack_tiles(const void* src, void* dst, long long count, int rows,
                             long long row_bytes, hipStream_t st);
hipError_t launch_rmsnorm(int act_kind, const void* h, const void* gamma, float eps, void* out,
                          int T, int H, hipStream_t st);
hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t st);
// probe.hip: read `bytes` (multiple of 16) from src with `blocks` blocks,
// one folded word per block into sink[blocks]
hipError_t launch_stream_read(const void* src, long long bytes, uint32_t* sink, int blocks,
                              hipStream_t st);

hipError_t launch_dispatch(const int32_t* topk_idx, int T, int k, int E, int S,
                           int32_t* chunk_counts, int32_t* chunk_base, int nchunks,
                           int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                           GroupDesc* groups, int32_t* totals, int32_t* mtg_gu, int32_t* mtg_dn,
                           TileShape gu, TileShape dn,
                           const void* w_gu, const float* s_gu, const void* w_dn,
                           const float* s_dn, const void* w_sh_gu, const float* s_sh_gu,
                           const void* w_sh_dn, const float* s_sh_dn, int H, int I,
                           int expert_kind, hipStream_t st);

hipError_t launch_groups_only(const int32_t* offsets, int T, int k, int E, int S,
                              GroupDesc* groups, int32_t* totals, int32_t* mtg_gu, int32_t* mtg_dn,
                           TileShape gu, TileShape dn,
                              const void* w_gu, const float* s_gu, const void* w_dn,
                              const float* s_dn, const void* w_sh_gu, const float* s_sh_gu,
                              const void* w_sh_dn, const float* s_sh_dn, int H, int I,
                              int expert_kind, hipStream_t st);

hipError_t launch_quant_rows_fp8(const uint16_t* x_bf16, int rows, int cols, uint8_t* q,
                                 float* scales, hipStream_t st);

// residual: null, or [T, H] of the act kind, added first (block forward)
// y, ysh fp32; or, with yexp (non-null), fp16 codes scaled per row and
// kHBlock columns (exponents [T*k + S*T, ceil(H / kHBlock)], rows of the
// sorted row space)
hipError_t launch_combine(int act_kind, const void* y, const void* ysh, const int32_t* yexp,
                          const float* w, const int32_t* inv, const void* residual, void* out,
                          int T, int H, int k, int S, hipStream_t st);

}  // namespace moe
