// Plain streaming read of a device buffer: the achievable-read marker reported
// beside the FFN kernels.  Each lane reads 16 bytes per load with four loads in
// flight, grid-stride over the buffer, and the workgroup's XOR of everything it
// read goes to sink[workgroup] (so no load can be dropped by the compiler).
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t xor4(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ p, size_t n16,
                                                         uint32_t* __restrict__ sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * 256;
  size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    x ^= xor4(a) ^ xor4(b) ^ xor4(c) ^ xor4(d);
  }
  for (; i < n16; i += stride) x ^= xor4(p[i]);
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
