// Streaming-read kernel of the achievable-HBM measurement (libqkvfa_bench.so).
// Each workgroup reads 16 KiB of consecutive 16-byte words per iteration
// (four non-temporal loads in flight per thread: each word is read once, and
// the non-temporal policy streams a 1 GiB read at 6.8-7.1 TB/s on MI355X against
// ~6.0-6.3 TB/s for the default policy) and folds them into a running XOR; it
// writes the XOR of its threads.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "qkvfa_bench.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, uint64_t n16,
                                                          uint32_t* __restrict__ out) {
  // a workgroup reads 4 x 256 consecutive words (16 KiB) per iteration
  const uint64_t stride = (uint64_t)gridDim.x * 1024;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (uint64_t i = (uint64_t)blockIdx.x * 1024 + threadIdx.x; i < n16; i += stride) {
    u32x4 w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t k = i + (uint64_t)u * 256;
      w[u] = k < n16 ? __builtin_nontemporal_load(src + k) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= w[u];
  }
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  __shared__ uint32_t red[256];
  red[threadIdx.x] = x;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

}  // namespace

extern "C" int qkvb_stream_read(const void* src, size_t bytes, uint32_t* out, int grid, void* stream) {
  if (!src || !out || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15) != 0 || grid < 1 ||
      grid > 65536)
    return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), (uint64_t)(bytes / 16), out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
