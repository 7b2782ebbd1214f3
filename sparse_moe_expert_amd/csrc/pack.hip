// Expert weights rearranged into the tiled storage of moe_internal.h
// (w_tile_row_off / w_tile_k_off): 16-row x 64-byte tiles, 1 KB each,
// 16-byte chunks chunk-major inside a tile.
//
// A pure byte permutation, done once when the weights are loaded.  With it
// the 16 rows x 64 bytes that one GEMM load instruction (64 lanes x 16
// bytes) reads are one contiguous 1 KB run, lane l at byte 16 l, instead of
// 16 row pieces 2*K bytes apart: the address unit handles one contiguous
// kilobyte in lane order much faster than sixteen scattered pieces
// (measured: row-major 11.11 ms per layer at T=16384, row-major tiles 8.47,
// chunk-major tiles faster again in the gate/up GEMM).
//
// One thread moves one 16-byte chunk.  Threads walk the output in order, so
// the stores are contiguous.  Grid-stride loop over all chunks of all
// matrices.
#include "moe_internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void pack_tiles_kernel(const uint4* __restrict__ src,
                                                         uint4* __restrict__ dst,
                                                         long long total_chunks,
                                                         long long matrix_chunks,
                                                         long long row_bytes) {
  const long long tiles_per_group = row_bytes / kTileBytes;
  for (long long q = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
       q < total_chunks; q += static_cast<long long>(gridDim.x) * blockDim.x) {
    const long long m = q / matrix_chunks;
    const long long o = (q - m * matrix_chunks) * 16;  // byte offset in the tiled matrix
    const long long tile = o / (kTileRows * kTileBytes);
    const int in_tile = static_cast<int>(o - tile * (kTileRows * kTileBytes));
    const long long group = tile / tiles_per_group;
    const long long tcol = tile - group * tiles_per_group;
    const long long row = group * kTileRows + (in_tile % (kTileRows * 16)) / 16;
    const long long byte = tcol * kTileBytes + (in_tile / (kTileRows * 16)) * 16;
    dst[q] = src[(m * matrix_chunks * 16 + row * row_bytes + byte) / 16];
  }
}

// Eight bf16 values -> eight fp16 per thread: each pair of bf16 widened to
// fp32 (exact) and packed to fp16 rounded toward zero, the instruction the
// large-tile down GEMM uses on its weight fragments.
__global__ __launch_bounds__(256) void convert_bf16_f16_kernel(const uint4* __restrict__ src,
                                                               uint4* __restrict__ dst,
                                                               long long chunks) {
  for (long long q = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; q < chunks;
       q += static_cast<long long>(gridDim.x) * blockDim.x) {
    const uint4 v = src[q];
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w[i] << 16),
                                                                     __uint_as_float(w[i] & 0xffff0000u)));
    dst[q] = uint4{w[0], w[1], w[2], w[3]};
  }
}

}  // namespace

hipError_t launch_convert_bf16_f16(const void* src, void* dst, long long n, hipStream_t st) {
  const long long chunks = n / 8;
  if (chunks <= 0) return hipSuccess;
  const long long want = (chunks + 255) / 256;
  const unsigned grid = static_cast<unsigned>(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(convert_bf16_f16_kernel, dim3(grid), dim3(256), 0, st,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), chunks);
  return hipGetLastError();
}

hipError_t launch_pack_tiles(const void* src, void* dst, long long count, int rows,
                             long long row_bytes, hipStream_t st) {
  const long long matrix_chunks = static_cast<long long>(rows) * row_bytes / 16;
  const long long total = count * matrix_chunks;
  if (total <= 0) return hipSuccess;
  const long long want = (total + 255) / 256;
  const unsigned grid = static_cast<unsigned>(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(pack_tiles_kernel, dim3(grid), dim3(256), 0, st,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), total,
                     matrix_chunks, row_bytes);
  return hipGetLastError();
}

}  // namespace moe
