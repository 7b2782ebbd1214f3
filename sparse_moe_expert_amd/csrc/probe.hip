// Streaming-read kernel: the measured HBM read ceiling the benchmark sets the
// weight-streaming GEMMs against (the vendor's 8 TB/s is a peak, not what a
// read stream reaches).  Every lane reads 16-byte chunks over a grid-stride
// loop, four loads in flight, with the non-temporal hint the decode GEMMs
// give their weight stream (every byte is read once), and folds them into
// one word per block so the loads cannot be dropped.  No arithmetic of the
// layer.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                       reinterpret_cast<const __attribute__((address_space(1))) i32x4_t*>(
                                           reinterpret_cast<uintptr_t>(p))));
}

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ src,
                                                               long long chunks,
                                                               uint32_t* __restrict__ sink) {
  const long long stride = static_cast<long long>(gridDim.x) * kThreads;
  long long q = static_cast<long long>(blockIdx.x) * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; q + 3 * stride < chunks; q += 4 * stride) {
    const uint4 a = stream_load(src + q), b = stream_load(src + q + stride),
                c = stream_load(src + q + 2 * stride), d = stream_load(src + q + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; q < chunks; q += stride) {
    const uint4 a = stream_load(src + q);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), m, 64));
  __shared__ uint32_t waves[kThreads / 64];
  if ((threadIdx.x & 63) == 0) waves[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = waves[0] ^ waves[1] ^ waves[2] ^ waves[3];
}

}  // namespace

hipError_t launch_stream_read(const void* src, long long bytes, uint32_t* sink, int blocks,
                              hipStream_t st) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0, st,
                     static_cast<const uint4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace moe
