// Plain streaming read of a device buffer: the achievable-read marker reported
// beside the FFN kernels.  The fastest read pattern measured on MI355X (a sweep of
// grid sizes, loads in flight, grid-stride against per-workgroup slabs, normal
// against non-temporal loads, over 2 GiB): each workgroup reads one contiguous
// slab of the buffer with non-temporal 16-byte loads, eight in flight per lane
// (each wavefront instruction covering 1 KB), 8192 workgroups -- ~7.0 TB/s, where
// the same pattern with normal loads reads ~6.2 TB/s and a grid-stride pattern
// with four normal loads in flight ~5.5 TB/s.  The workgroup's XOR of everything
// it read goes to sink[workgroup] (so no load can be dropped by the compiler).
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t xor_nt(const uint4* q) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q));
  return v.x ^ v.y ^ v.z ^ v.w;
}

__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ p, size_t n16,
                                                         uint32_t* __restrict__ sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;   // 16-byte words per workgroup
  const size_t lo = static_cast<size_t>(blockIdx.x) * per;
  const size_t begin = lo < n16 ? lo : n16;
  const size_t end = begin + per < n16 ? begin + per : n16;
  size_t i = begin + threadIdx.x;
  uint32_t x = 0;
  for (; i + 7 * 256 < end; i += 8 * 256) {
    uint32_t v[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) v[d] = xor_nt(p + i + d * 256);
#pragma unroll
    for (int d = 0; d < 8; ++d) x ^= v[d];
  }
  for (; i < end; i += 256) x ^= xor_nt(p + i);
  for (int o = 32; o > 0; o >>= 1) x ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), o, 64));
  __shared__ uint32_t wave_x[4];
  if ((threadIdx.x & 63) == 0) wave_x[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = wave_x[0] ^ wave_x[1] ^ wave_x[2] ^ wave_x[3];
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  read_probe_kernel<<<kReadProbeBlocks, 256, 0, stream>>>(static_cast<const uint4*>(buf),
                                                          bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace moe
