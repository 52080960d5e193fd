// tq_stream.hip -- a plain streaming read of device memory: the practical
// HBM read ceiling that decode throughput is reported against, next to the
// published peak.  Not part of the method.
//
// Every lane reads 16-byte words with non-temporal loads (as the decode reads
// each cache byte once), four in flight per iteration of a grid-stride loop,
// and folds them with XOR; each workgroup folds its lanes and XORs the result
// into one device word, so the read cannot be elided and its result is exact
// (XOR is associative and commutative: any schedule gives the same word).

#include <hip/hip_runtime.h>

#include <algorithm>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kStreamThreads = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* __restrict__ src, uint64_t n16,
                                                                     uint32_t* sink) {
  uint32_t x = 0;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kStreamThreads;
  uint64_t i = static_cast<uint64_t>(blockIdx.x) * kStreamThreads + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    x ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) x ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), w, 64));
  __shared__ uint32_t part[kStreamThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
#pragma unroll
    for (int k = 0; k < kStreamThreads / 64; ++k) y ^= part[k];
    atomicXor(sink, y);
  }
}

}  // namespace

hipError_t launch_stream_read(const void* src, uint64_t bytes, uint32_t* sink, hipStream_t stream) {
  const uint64_t n16 = bytes / 16;
  // eight workgroups per compute unit, each lane with four loads in flight
  // (measured over 2 GiB: 5.93 TB/s; four per unit 5.82, sixteen 5.68, eight
  // loads in flight per lane no better)
  const int grid = static_cast<int>(std::min<uint64_t>(2048, (n16 + kStreamThreads - 1) / kStreamThreads));
  hipLaunchKernelGGL(stream_read_kernel, dim3(std::max(grid, 1)), dim3(kStreamThreads), 0, stream,
                     static_cast<const u32x4*>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace tq
