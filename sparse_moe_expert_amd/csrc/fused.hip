// The whole layer in one launch, for the decode regime (gfx950).
//
// The single-launch form of the layer chain -- route -> dispatch -> gate/up +
// SwiGLU -> down -> combine, the chain that the Ascend adaptation figure of
// the Deep Dive (§8.2, FUSED_MC2) runs as one fused operator.  One
// cooperative persistent grid walks the phases with a grid barrier between
// them; every block runs every phase and meets every barrier, and each phase
// strides its work items over the grid:
//   A  router logits: 16 tokens x 16 experts x one K-split per wave, straight
//      from global memory into v_mfma_f32_16x16x32_bf16 (fp32 partial sums)
//   B  top-k per token (one wave each; adds the K-split partial sums in order)
//   C  dispatch: every block builds the expert histogram and its exclusive
//      scan in LDS from all T*k choices (a few thousand integers), counts the
//      pairs before its own slice of the flat order, and scatters that slice
//      stably (64 pairs per step, ballot peers); the GEMM tile table is
//      spread over the first blocks
//   D  gate/up + SwiGLU tiles of the weight-streaming GEMM
//   E  down tiles of the same GEMM
//   F  combine, one token per block at a time
// Phases A, B, D, E and F are the same arithmetic as the separate kernels
// (A sums K in another order than the separate router GEMM); C produces the
// same integers.  Where the layer has few tokens, the launches and the
// barriers between dependent kernels are what this removes.
//
// The grid barrier is the library's own: an arrival counter in the
// workspace, polled with s_sleep by one thread per block, and a bounded wait.
// A block that waits more than the spin limit (moe_fused_set_spin_limit)
// sets the status word next to the counter; every block that sees it stops,
// so the launch always ends, and the caller reads the status after
// synchronising (MOE_WS_BARRIER).  Polls are relaxed loads with one acquire
// fence after the wait: an acquire per poll invalidates the caches under the
// blocks still working (measured 2.71 against 2.47 ms at T=256).
//
// Measured at T=256 (dots3 decode shape, tiled weights, expert weights read
// with cached loads at the time), block 0's time from barrier to barrier:
// A 66, B 60, C 44, D 1432, E 819, F 34 us, 2.45 ms in all, against 2.15 ms
// for the separate launches (route 27, dispatch 12, gate/up 1362, down 751,
// combine 13 us).  The phases around the GEMMs take 204 us here against
// 52 us as kernels: each of the five barriers, 512 blocks arriving on one
// counter, costs tens of microseconds, more than the launch gaps they
// replace; the GEMM phases run 5% and 9% slower than the separate kernels.
// With the non-temporal expert weight loads both forms got faster, and the
// gap stayed: 2.27 ms in one launch against 1.96 ms separately.
#include <algorithm>

#include "combine_device.h"
#include "gemm_decode_device.h"
#include "route_device.h"

namespace moe {
namespace {

constexpr int kThreads = 256;  // 4 waves, the decode GEMM's tile
constexpr int kGroupsMax = kMaxExperts + kMaxShared;

// In-place exclusive scan of a[0, n) in LDS by one wavefront; returns the total.
__device__ __forceinline__ int wave_exclusive_scan(int* a, int n, int lane) {
  const int seg = (n + 63) / 64;
  const int lo = min(n, lane * seg), hi = min(n, lo + seg);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += a[i];
  int incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  int run = incl - sum;
  for (int i = lo; i < hi; ++i) {
    const int v = a[i];
    a[i] = run;
    run += v;
  }
  return __shfl(incl, 63, 64);
}

// Grid barrier number n (0, 1, ...), which every block meets once: thread 0
// publishes the block's writes of the phase (release), adds its arrival and
// polls until all gridDim.x blocks of this barrier have arrived (acquire).
// Returns false in every thread of the block when the launch must stop: this
// block polled more than spin_limit times (it then sets the status word) or
// another block did.
__device__ __forceinline__ bool grid_barrier(uint32_t* bar, long long spin_limit, unsigned n,
                                             int* s_ok) {
  __syncthreads();  // the block's writes of the phase are done
  if (threadIdx.x == 0) {
    int ok = 1;
    __threadfence();
    __hip_atomic_fetch_add(&bar[0], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned target = (n + 1) * gridDim.x;
    long long polls = 0;
    // relaxed polls (an acquire per poll would invalidate the caches each
    // time, under the blocks still working); one acquire fence after
    while (__hip_atomic_load(&bar[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (__hip_atomic_load(&bar[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
          ++polls > spin_limit) {
        __hip_atomic_store(&bar[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
    if (__hip_atomic_load(&bar[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) ok = 0;
    __atomic_thread_fence(__ATOMIC_ACQUIRE);
    __threadfence();
    *s_ok = ok;
  }
  __syncthreads();
  return *s_ok != 0;
}

__global__ __launch_bounds__(kThreads, 2) void fused_decode_kernel(FusedArgs a) {
  __shared__ int s_ok;
  unsigned nbar = 0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const long long gwave = static_cast<long long>(blockIdx.x) * 4 + wave;
  const long long nwaves = static_cast<long long>(gridDim.x) * 4;

  // ---------------------------------------------------------------- A
  if (blockIdx.x == 0 && tid == 0) {
    if (a.ties) {
      a.ties[0] = 0;
      a.ties[1] = 0;
    }
  }
  {
    const int ntt = (a.T + 15) / 16, nte = a.E / 16;
    const int KS = a.H / a.splits;
    const long long items = static_cast<long long>(ntt) * nte * a.splits;
    const int r = lane & 15, g = lane >> 4;
    for (long long it = gwave; it < items; it += nwaves) {
      const int sp = static_cast<int>(it % a.splits);
      const long long rest = it / a.splits;
      const int te = static_cast<int>(rest % nte);
      const int tm = static_cast<int>(rest / nte);
      const int t0 = tm * 16, e0 = te * 16, k0 = sp * KS;
      const uint16_t* xa = a.x + static_cast<long long>(min(t0 + r, a.T - 1)) * a.H + k0 + 8 * g;
      const uint16_t* wb = a.w_router + static_cast<long long>(e0 + r) * a.H + k0 + 8 * g;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int kk = 0; kk < KS; kk += 32) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(xa + kk);
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(wb + kk);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
      }
      // lane l, element i -> token 4*(l/16) + i, expert l%16 of the tile
      float* dst = a.logits + static_cast<long long>(sp) * a.T * a.E;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * g + i;
        if (t < a.T) dst[static_cast<long long>(t) * a.E + e0 + r] = acc[i];
      }
    }
  }
  if (!grid_barrier(a.bar, a.spin_limit, nbar++, &s_ok)) return;

  // ---------------------------------------------------------------- B
  {
    __shared__ float cbuf[4][kMaxExperts];
    const int kper = router_keys_per_lane(a.E);
    for (long long t = gwave; t < a.T; t += nwaves) {
      const int ti = static_cast<int>(t);
      if (kper == 1)
        router_topk_token<1>(a.logits, a.splits, a.bias, a.T, a.E, a.k, a.n_group, a.topk_group,
                             a.norm, a.rsf, a.idx, a.tw, a.ties, ti, lane, cbuf[wave]);
      else if (kper == 2)
        router_topk_token<2>(a.logits, a.splits, a.bias, a.T, a.E, a.k, a.n_group, a.topk_group,
                             a.norm, a.rsf, a.idx, a.tw, a.ties, ti, lane, cbuf[wave]);
      else if (kper == 4)
        router_topk_token<4>(a.logits, a.splits, a.bias, a.T, a.E, a.k, a.n_group, a.topk_group,
                             a.norm, a.rsf, a.idx, a.tw, a.ties, ti, lane, cbuf[wave]);
      else
        router_topk_token<8>(a.logits, a.splits, a.bias, a.T, a.E, a.k, a.n_group, a.topk_group,
                             a.norm, a.rsf, a.idx, a.tw, a.ties, ti, lane, cbuf[wave]);
    }
  }
  if (!grid_barrier(a.bar, a.spin_limit, nbar++, &s_ok)) return;

  // ---------------------------------------------------------------- C
  {
    __shared__ int s_cnt[kMaxExperts], s_off[kMaxExperts], s_run[kMaxExperts];
    __shared__ int s_tg[kGroupsMax], s_td[kGroupsMax];
    const int R = a.T * a.k, E = a.E, G = a.E + a.S;
    // this block's slice [f0, f1) of the flat (token, slot) order
    const int sl = ((R + static_cast<int>(gridDim.x) - 1) / static_cast<int>(gridDim.x) + 63) / 64 * 64;
    const int f0 = min(R, static_cast<int>(blockIdx.x) * sl), f1 = min(R, f0 + sl);
    for (int e = tid; e < E; e += kThreads) {
      s_cnt[e] = 0;
      s_run[e] = 0;
    }
    __syncthreads();
    // histogram of all pairs, and of the pairs before the slice
    for (int f = tid; f < R; f += kThreads) {
      const int e = a.idx[f];
      atomicAdd(&s_cnt[e], 1);
      if (f < f0) atomicAdd(&s_run[e], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += kThreads) s_off[e] = s_cnt[e];
    __syncthreads();
    if (wave == 0) wave_exclusive_scan(s_off, E, lane);
    __syncthreads();
    for (int e = tid; e < E; e += kThreads) {
      s_run[e] += s_off[e];  // first position of the slice's pairs of expert e
      if (blockIdx.x == 0) {
        a.counts[e] = s_cnt[e];
        a.offsets[e] = s_off[e];
      }
    }
    if (blockIdx.x == 0 && tid == 0) a.offsets[E] = R;
    __syncthreads();
    if (wave == 0) {
      // stable counting sort of the slice: 64 pairs per step in flat order;
      // lanes with the same expert find each other with 9 ballots (one per
      // bit of the id)
      const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      for (int fs = f0; fs < f1; fs += 64) {
        const int f = fs + lane;
        const bool valid = f < f1;
        const int e = valid ? a.idx[f] : 0;
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 9; ++b) {
          const bool bit = (e >> b) & 1;
          const uint64_t m = __ballot(bit);
          peers &= bit ? m : ~m;
        }
        const int rank = __popcll(peers & below);
        const int base = valid ? s_run[e] : 0;
        if (valid) {
          const int pos = base + rank;
          a.perm[pos] = f;
          a.inv[f] = pos;
          if (rank == 0) s_run[e] = base + __popcll(peers);
        }
      }
    }
    // tile table of the two GEMMs (groups = routed experts, then shared):
    // every block scans the groups' tile counts, the first blocks write the
    // descriptors and the m-tile -> group tables
    for (int gi = tid; gi < G; gi += kThreads) {
      const int rows = gi < E ? s_cnt[gi] : a.T;
      s_tg[gi] = (rows + a.tgu.bm - 1) / a.tgu.bm;
      s_td[gi] = (rows + a.tdn.bm - 1) / a.tdn.bm;
    }
    __syncthreads();
    if (wave == 0) {
      const int tot_g = wave_exclusive_scan(s_tg, G, lane);
      const int tot_d = wave_exclusive_scan(s_td, G, lane);
      if (blockIdx.x == 0 && lane == 0) {
        a.totals[0] = tot_g;
        a.totals[1] = tot_d;
      }
    }
    __syncthreads();
    const long long gu_elems = 2ll * a.I * a.H, dn_elems = static_cast<long long>(a.H) * a.I;
    for (long long gl = static_cast<long long>(blockIdx.x) * kThreads + tid; gl < G;
         gl += static_cast<long long>(gridDim.x) * kThreads) {
      const int gi = static_cast<int>(gl);
      const bool shared = gi >= E;
      const long long e = shared ? gi - E : gi;
      GroupDesc d;
      d.row_begin = shared ? R + (gi - E) * a.T : s_off[gi];
      d.rows = shared ? a.T : s_cnt[gi];
      d.tile_begin_gu = s_tg[gi];
      d.tile_begin_dn = s_td[gi];
      d.w_gu = (shared ? a.w_sh_gu : a.w_gu) + e * gu_elems * 2;
      d.w_dn = (shared ? a.w_sh_dn : a.w_dn) + e * dn_elems * 2;
      d.s_gu = nullptr;
      d.s_dn = nullptr;
      a.groups[gi] = d;
      for (int i = 0; i < (d.rows + a.tgu.bm - 1) / a.tgu.bm; ++i) a.mtg_gu[d.tile_begin_gu + i] = gi;
      for (int i = 0; i < (d.rows + a.tdn.bm - 1) / a.tdn.bm; ++i) a.mtg_dn[d.tile_begin_dn + i] = gi;
    }
  }
  if (!grid_barrier(a.bar, a.spin_limit, nbar++, &s_ok)) return;

  // ---------------------------------------------------------------- D, E
  // tiles strided over the grid (a multiple of 8: tile b stays on XCD b % 8)
  {
    const long long ngu = ((static_cast<long long>(a.gu.grid_mtiles_upper) *
                                ((a.gu.N + 127) / 128) + 7) / 8) * 8;
    for (long long vb = blockIdx.x; vb < ngu; vb += gridDim.x)
      decode_tile<1, true, 4>(a.gu, static_cast<int>(vb));
  }
  if (!grid_barrier(a.bar, a.spin_limit, nbar++, &s_ok)) return;
  {
    const long long ndn = ((static_cast<long long>(a.dn.grid_mtiles_upper) *
                                ((a.dn.N + 255) / 256) + 7) / 8) * 8;
    // h as two bf16 terms when the layout keeps its residue (gate/up wrote it)
    if (a.dn.A_lo) {
      for (long long vb = blockIdx.x; vb < ndn; vb += gridDim.x)
        decode_tile<1, false, 4, true>(a.dn, static_cast<int>(vb));
    } else {
      for (long long vb = blockIdx.x; vb < ndn; vb += gridDim.x)
        decode_tile<1, false, 4>(a.dn, static_cast<int>(vb));
    }
  }
  if (!grid_barrier(a.bar, a.spin_limit, nbar++, &s_ok)) return;

  // ---------------------------------------------------------------- F
  {
    __shared__ float s_w[kMaxTopK];
    __shared__ long long s_r[kMaxTopK];
    for (int t = blockIdx.x; t < a.T; t += gridDim.x) {
      combine_token<K_BF16>(a.y, a.ysh, a.tw, a.inv, a.residual, a.out, a.T, a.H, a.k, a.S, t,
                            s_w, s_r, 0, a.H);
      __syncthreads();  // s_w / s_r are rewritten for the next token
    }
  }
}

}  // namespace

bool fused_decode_supported(TileShape gu, TileShape dn) {
  // 16-row decode tiles only: the 32-row variant would raise the kernel's
  // register count (and cut its occupancy) for every phase
  return gu.bm == 16 && gu.bn == 128 && dn.bm == 16 && dn.bn == 256;
}

hipError_t launch_fused_decode(const FusedArgs& a, hipStream_t st) {
  if (a.T <= 0) return hipSuccess;
  if (!a.bar || a.spin_limit < 0) return hipErrorInvalidValue;
  int dev = 0, cus = 0, per = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fused_decode_kernel, kThreads, 0);
  if (e != hipSuccess) return e;
  // Every block must be resident at once (grid barriers).  The kernel's 248
  // VGPRs allow 2 waves per SIMD, so `per` is 2 (4-wave blocks); the cap
  // keeps it there whatever a future build's register count allows.  A
  // multiple of 8 keeps the tile -> XCD mapping of the GEMM phases.
  const int grid = (std::min(per, 2) * cus) / 8 * 8;
  if (grid < 8) return hipErrorInvalidConfiguration;
  // barrier counter and status word start at zero (a kernel, not a memset:
  // the launch may be captured into a graph)
  e = launch_zero_i32(reinterpret_cast<int32_t*>(a.bar), 2, st);
  if (e != hipSuccess) return e;
  FusedArgs args = a;
  void* params[] = {&args};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(fused_decode_kernel), dim3(grid),
                                    dim3(kThreads), params, 0, st);
}

}  // namespace moe
