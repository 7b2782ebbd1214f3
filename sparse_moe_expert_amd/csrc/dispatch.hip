// Dispatch: per-expert histogram, exclusive scan and stable permutation of the
// T*k (token, slot) pairs into expert-sorted order (gfx950), plus the device
// tile schedule of the grouped GEMMs.
//
// The order inside an expert is ascending flat index f = t*k + j -- the order
// in which the per-expert mask gathers tokens (x[mask]) in the Dots3MoELayer
// loop of the Deep Dive §3.1 -- so the result is a stable counting sort, the
// "dispatch" step of the §8.2 figure.  Integer only, no float, deterministic:
//   1. hist:    one wave per 1024-pair chunk counts its pairs per expert
//               (LDS atomics on integers; order-independent).
//   2. scan:    per expert, exclusive scan over chunks; then over experts.
//   3. scatter: one wave per chunk walks its pairs 64 at a time; lanes with
//               the same expert find each other with 9 ballots (bits of the
//               expert id), take rank = earlier peers, and the lowest peer
//               advances the expert's running position.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kExpertBits = 9;  // kMaxExperts = 512
static_assert((1 << kExpertBits) == kMaxExperts, "expert id bits");

__global__ __launch_bounds__(256) void dispatch_hist_kernel(const int32_t* __restrict__ idx,
                                                            int n, int E, int nchunks,
                                                            int32_t* __restrict__ chunk_counts) {
  __shared__ int32_t hist[kWavesPerBlock][kMaxExperts];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kWavesPerBlock * kMaxExperts; i += blockDim.x)
    (&hist[0][0])[i] = 0;
  __syncthreads();
  const int c = blockIdx.x * kWavesPerBlock + wave;
  if (c < nchunks) {
    const int f0 = c * kDispatchChunk;
    for (int r = 0; r < kDispatchChunk / 64; ++r) {
      const int f = f0 + r * 64 + lane;
      if (f < n) atomicAdd(&hist[wave][idx[f]], 1);
    }
  }
  __syncthreads();
  if (c < nchunks)
    for (int e = lane; e < E; e += 64) chunk_counts[static_cast<long long>(c) * E + e] = hist[wave][e];
}

// Block-wide exclusive scan of one int per thread (blockDim.x a multiple of
// 64, at most 4096; every thread calls it).  Each wave scans its 64 values
// with shuffles, one wave scans the wave totals, and each thread adds its
// wave's base: three barriers instead of two per doubling step.  Integer
// sums, so the result does not depend on the order.  sh: blockDim.x / 64
// ints of LDS, free again when the call returns.
__device__ int block_exclusive_scan(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = static_cast<int>(blockDim.x) >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < nw ? sh[lane] : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(w, off, 64);
      if (lane >= off) w += y;
    }
    if (lane < nw) sh[lane] = w;  // inclusive sums of the wave totals
  }
  __syncthreads();
  const int incl = (wave > 0 ? sh[wave - 1] : 0) + x;
  if (total) *total = sh[nw - 1];
  __syncthreads();
  return incl - v;
}

__device__ void build_groups_body(const int32_t* offsets, int T, int k, int E, int S,
                                  GroupDesc* __restrict__ groups, int32_t* __restrict__ totals,
                                  int32_t* __restrict__ mtg_gu, int32_t* __restrict__ mtg_dn,
                                  int bm_gu, int bm_dn, const char* w_gu, const float* s_gu,
                                  const char* w_dn, const float* s_dn, const char* w_sh_gu,
                                  const float* s_sh_gu, const char* w_sh_dn, const float* s_sh_dn,
                                  int H, int I, int esz, int fp8, int* sh);

// Scan over chunks and experts; then (if groups is set) the tile table from
// the offsets it just formed, in the same block: one launch less than a
// separate tile-table kernel.
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(
    const int32_t* __restrict__ chunk_counts, int nchunks, int E, int32_t* __restrict__ chunk_base,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int T, int k, int S,
    GroupDesc* __restrict__ groups, int32_t* __restrict__ totals, int32_t* __restrict__ mtg_gu,
    int32_t* __restrict__ mtg_dn, int bm_gu, int bm_dn, const char* w_gu, const float* s_gu,
    const char* w_dn, const float* s_dn, const char* w_sh_gu, const float* s_sh_gu,
    const char* w_sh_dn, const float* s_sh_dn, int H, int I, int esz, int fp8) {
  // Thread e walks expert e's column of chunk counts twice (total, then the
  // running bases).  Loads go out 16 chunks at a time so that their latencies
  // overlap instead of adding up chunk by chunk.
  constexpr int B = 16;
  __shared__ int sh[1024];
  __shared__ int32_t s_off[kMaxExperts + 1];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int c0 = 0; c0 < nchunks; c0 += B) {
      int v[B];
#pragma unroll
      for (int j = 0; j < B; ++j)
        v[j] = (c0 + j < nchunks) ? chunk_counts[static_cast<long long>(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < B; ++j) run += v[j];
    }
  }
  int total = 0;
  const int excl = block_exclusive_scan(e < E ? run : 0, sh, &total);
  if (e < E) {
    counts[e] = run;
    offsets[e] = excl;
    int acc = excl;
    for (int c0 = 0; c0 < nchunks; c0 += B) {
      int v[B];
#pragma unroll
      for (int j = 0; j < B; ++j)
        v[j] = (c0 + j < nchunks) ? chunk_counts[static_cast<long long>(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < B; ++j) {
        if (c0 + j < nchunks) chunk_base[static_cast<long long>(c0 + j) * E + e] = acc;
        acc += v[j];
      }
    }
  }
  if (e == 0) offsets[E] = total;
  if (groups) {
    if (e < E) s_off[e] = excl;
    if (e == 0) s_off[E] = total;
    __syncthreads();
    build_groups_body(s_off, T, k, E, S, groups, totals, mtg_gu, mtg_dn, bm_gu, bm_dn, w_gu, s_gu,
                      w_dn, s_dn, w_sh_gu, s_sh_gu, w_sh_dn, s_sh_dn, H, I, esz, fp8, sh);
  }
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(const int32_t* __restrict__ idx,
                                                               int n, int E, int nchunks,
                                                               const int32_t* __restrict__ chunk_base,
                                                               int32_t* __restrict__ perm,
                                                               int32_t* __restrict__ inv) {
  __shared__ int32_t run[kWavesPerBlock][kMaxExperts];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x * kWavesPerBlock + wave;
  if (c < nchunks)
    for (int e = lane; e < E; e += 64) run[wave][e] = chunk_base[static_cast<long long>(c) * E + e];
  __syncthreads();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < kDispatchChunk / 64; ++r) {
    const int f = c * kDispatchChunk + r * 64 + lane;
    const bool valid = (c < nchunks) && (f < n);
    const int e = valid ? idx[f] : 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < kExpertBits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & below);
    const int base = valid ? run[wave][e] : 0;
    __syncthreads();  // every lane has read its base before any update
    if (valid) {
      const int pos = base + rank;
      perm[pos] = f;
      inv[f] = pos;
      if (rank == 0) run[wave][e] = base + __popcll(peers);
    }
    __syncthreads();
  }
}

// Tile table of the two grouped GEMMs, by one block of 1024 threads: group g
// (routed experts, then the shared experts) gets its rows, its first m-tile
// in each GEMM, its weight (and fp8 scale) pointers, and the m-tile -> group
// lookup tables.  offsets: [E + 1] exclusive scan of the expert counts.
__device__ void build_groups_body(const int32_t* offsets, int T, int k, int E, int S,
                                  GroupDesc* __restrict__ groups, int32_t* __restrict__ totals,
                                  int32_t* __restrict__ mtg_gu, int32_t* __restrict__ mtg_dn,
                                  int bm_gu, int bm_dn, const char* w_gu, const float* s_gu,
                                  const char* w_dn, const float* s_dn, const char* w_sh_gu,
                                  const float* s_sh_gu, const char* w_sh_dn, const float* s_sh_dn,
                                  int H, int I, int esz, int fp8, int* sh) {
  const int g = threadIdx.x;
  const int G = E + S;
  const int R = T * k;
  int begin = 0, rows = 0;
  if (g < E) {
    begin = offsets[g];
    rows = offsets[g + 1] - begin;
  } else if (g < G) {
    begin = R + (g - E) * T;
    rows = T;
  }
  const int tg = (rows + bm_gu - 1) / bm_gu;
  const int td = (rows + bm_dn - 1) / bm_dn;
  int tot_g = 0, tot_d = 0;
  const int ex_g = block_exclusive_scan(tg, sh, &tot_g);
  const int ex_d = block_exclusive_scan(td, sh, &tot_d);
  if (g < G) {
    const bool shared = g >= E;
    const long long e = shared ? g - E : g;
    const long long gu_elems = 2ll * I * H, dn_elems = static_cast<long long>(H) * I;
    const long long gu_sc = fp8 ? (2ll * I / kQBlock) * (H / kQBlock) : 0;
    const long long dn_sc = fp8 ? (static_cast<long long>(H) / kQBlock) * (I / kQBlock) : 0;
    GroupDesc d;
    d.row_begin = begin;
    d.rows = rows;
    d.tile_begin_gu = ex_g;
    d.tile_begin_dn = ex_d;
    d.w_gu = (shared ? w_sh_gu : w_gu) + e * gu_elems * esz;
    d.w_dn = (shared ? w_sh_dn : w_dn) + e * dn_elems * esz;
    d.s_gu = fp8 ? (shared ? s_sh_gu : s_gu) + e * gu_sc : nullptr;
    d.s_dn = fp8 ? (shared ? s_sh_dn : s_dn) + e * dn_sc : nullptr;
    groups[g] = d;
    // m-tile -> group tables (the GEMMs look their tile's group up directly)
    for (int i = 0; i < tg; ++i) mtg_gu[ex_g + i] = g;
    for (int i = 0; i < td; ++i) mtg_dn[ex_d + i] = g;
  }
  if (g == 0) {
    totals[0] = tot_g;
    totals[1] = tot_d;
  }
}

__global__ __launch_bounds__(1024) void build_groups_kernel(
    const int32_t* __restrict__ offsets, int T, int k, int E, int S, GroupDesc* __restrict__ groups,
    int32_t* __restrict__ totals, int32_t* __restrict__ mtg_gu, int32_t* __restrict__ mtg_dn,
    int bm_gu, int bm_dn, const char* w_gu, const float* s_gu,
    const char* w_dn, const float* s_dn, const char* w_sh_gu, const float* s_sh_gu,
    const char* w_sh_dn, const float* s_sh_dn, int H, int I, int esz, int fp8) {
  __shared__ int sh[1024];
  build_groups_body(offsets, T, k, E, S, groups, totals, mtg_gu, mtg_dn, bm_gu, bm_dn, w_gu, s_gu,
                    w_dn, s_dn, w_sh_gu, s_sh_gu, w_sh_dn, s_sh_dn, H, I, esz, fp8, sh);
}

// The whole dispatch in one block of 16 waves when the pairs fit in 16 chunks
// (T*k <= 16384, the decode regime): the pairs are cut into 16 chunks of a
// multiple of 64, and wave w takes chunk w through the same three steps as
// the separate kernels -- histogram, scan over chunks then experts, stable
// scatter -- with the chunk table in LDS, then (if groups is set) the tile
// table.  Same results, bit for bit; one launch instead of four.
constexpr int kSmallChunks = 16;

__global__ __launch_bounds__(1024) void dispatch_small_kernel(
    const int32_t* __restrict__ idx, int n, int E, int nchunks, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    int T, int k, int S, GroupDesc* __restrict__ groups, int32_t* __restrict__ totals,
    int32_t* __restrict__ mtg_gu, int32_t* __restrict__ mtg_dn, int bm_gu, int bm_dn,
    const char* w_gu, const float* s_gu, const char* w_dn, const float* s_dn, const char* w_sh_gu,
    const float* s_sh_gu, const char* w_sh_dn, const float* s_sh_dn, int H, int I, int esz,
    int fp8) {
  const int cs = max(64, (n + kSmallChunks * 64 - 1) / (kSmallChunks * 64) * 64);  // pairs per chunk
  nchunks = (n + cs - 1) / cs;
  __shared__ int32_t run[kSmallChunks][kMaxExperts];  // counts, then running positions
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ int sh[1024];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kSmallChunks * kMaxExperts; i += blockDim.x) (&run[0][0])[i] = 0;
  __syncthreads();
  // 1. histogram of chunk `wave`
  if (wave < nchunks) {
    const int f0 = wave * cs;
    for (int r = 0; r < cs / 64; ++r) {
      const int f = f0 + r * 64 + lane;
      if (f < n) atomicAdd(&run[wave][idx[f]], 1);
    }
  }
  __syncthreads();
  // 2. per expert: running bases over chunks, then the exclusive scan over experts
  const int e = threadIdx.x;
  int tot_e = 0;
  if (e < E)
    for (int c = 0; c < nchunks; ++c) tot_e += run[c][e];
  int total = 0;
  const int excl = block_exclusive_scan(e < E ? tot_e : 0, sh, &total);
  if (e < E) {
    counts[e] = tot_e;
    offsets[e] = excl;
    s_off[e] = excl;
    int acc = excl;
    for (int c = 0; c < nchunks; ++c) {
      const int v = run[c][e];
      run[c][e] = acc;
      acc += v;
    }
  }
  if (e == 0) {
    offsets[E] = total;
    s_off[E] = total;
  }
  __syncthreads();
  // 3. stable scatter of chunk `wave` (as dispatch_scatter_kernel)
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < cs / 64; ++r) {
    const int f = wave * cs + r * 64 + lane;
    const bool valid = (wave < nchunks) && (f < n);
    const int ef = valid ? idx[f] : 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < kExpertBits; ++b) {
      const bool bit = (ef >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & below);
    const int base = valid ? run[wave][ef] : 0;
    __syncthreads();  // every lane has read its base before any update
    if (valid) {
      const int pos = base + rank;
      perm[pos] = f;
      inv[f] = pos;
      if (rank == 0) run[wave][ef] = base + __popcll(peers);
    }
    __syncthreads();
  }
  // 4. tile table
  if (groups)
    build_groups_body(s_off, T, k, E, S, groups, totals, mtg_gu, mtg_dn, bm_gu, bm_dn, w_gu, s_gu,
                      w_dn, s_dn, w_sh_gu, s_sh_gu, w_sh_dn, s_sh_dn, H, I, esz, fp8, sh);
}

}  // namespace

hipError_t launch_groups_only(const int32_t* offsets, int T, int k, int E, int S,
                              GroupDesc* groups, int32_t* totals, int32_t* mtg_gu,
                              int32_t* mtg_dn, TileShape gu, TileShape dn,
                              const void* w_gu, const float* s_gu, const void* w_dn,
                              const float* s_dn, const void* w_sh_gu, const float* s_sh_gu,
                              const void* w_sh_dn, const float* s_sh_dn, int H, int I,
                              int expert_kind, hipStream_t st) {
  hipLaunchKernelGGL(build_groups_kernel, dim3(1), dim3(1024), 0, st, offsets, T, k, E, S, groups,
                     totals, mtg_gu, mtg_dn, gu.bm, dn.bm, static_cast<const char*>(w_gu), s_gu,
                     static_cast<const char*>(w_dn), s_dn, static_cast<const char*>(w_sh_gu),
                     s_sh_gu, static_cast<const char*>(w_sh_dn), s_sh_dn, H, I,
                     static_cast<int>(kind_size(expert_kind)), expert_kind == K_FP8 ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_dispatch(const int32_t* topk_idx, int T, int k, int E, int S,
                           int32_t* chunk_counts, int32_t* chunk_base, int nchunks,
                           int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                           GroupDesc* groups, int32_t* totals, int32_t* mtg_gu,
                           int32_t* mtg_dn, TileShape gu, TileShape dn,
                           const void* w_gu, const float* s_gu, const void* w_dn,
                           const float* s_dn, const void* w_sh_gu, const float* s_sh_gu,
                           const void* w_sh_dn, const float* s_sh_dn, int H, int I,
                           int expert_kind, hipStream_t st) {
  const int n = T * k;
  if (nchunks <= kSmallChunks) {
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(1024), 0, st, topk_idx, n, E, nchunks,
                       counts, offsets, perm, inv, T, k, S, groups, totals, mtg_gu, mtg_dn, gu.bm,
                       dn.bm, static_cast<const char*>(w_gu), s_gu, static_cast<const char*>(w_dn),
                       s_dn, static_cast<const char*>(w_sh_gu), s_sh_gu,
                       static_cast<const char*>(w_sh_dn), s_sh_dn, H, I,
                       static_cast<int>(kind_size(expert_kind)), expert_kind == K_FP8 ? 1 : 0);
    return hipGetLastError();
  }
  const int blocks = (nchunks + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(dispatch_hist_kernel, dim3(blocks), dim3(256), 0, st, topk_idx, n, E,
                     nchunks, chunk_counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, st, chunk_counts, nchunks, E,
                     chunk_base, counts, offsets, T, k, S, groups, totals, mtg_gu, mtg_dn, gu.bm,
                     dn.bm, static_cast<const char*>(w_gu), s_gu, static_cast<const char*>(w_dn),
                     s_dn, static_cast<const char*>(w_sh_gu), s_sh_gu,
                     static_cast<const char*>(w_sh_dn), s_sh_dn, H, I,
                     static_cast<int>(kind_size(expert_kind)), expert_kind == K_FP8 ? 1 : 0);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(blocks), dim3(256), 0, st, topk_idx, n, E,
                     nchunks, chunk_base, perm, inv);
  return hipGetLastError();
}

}  // namespace moe
