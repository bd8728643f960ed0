// Activations to the two-part FP8 form read by the tiled FFN's block-scaled MFMAs,
// one thread per 32-element block of a row (act_split_block).
#include "act_split.h"
#include "launch.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void act_split_kernel(const uint16_t* __restrict__ x,
                                                        int64_t n_blocks, int K,
                                                        uint8_t* __restrict__ xq,
                                                        uint8_t* __restrict__ xs) {
  const int64_t bid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (bid >= n_blocks) return;
  act_split_block(x, bid, K, xq, xs);
}

}  // namespace

hipError_t launch_act_split(const uint16_t* x, int64_t rows, int K, uint8_t* xq, uint8_t* xs,
                            hipStream_t stream) {
  const int64_t n_blocks = rows * (K / 32);
  if (n_blocks == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>((n_blocks + 255) / 256);
  act_split_kernel<<<grid, 256, 0, stream>>>(x, n_blocks, K, xq, xs);
  return hipGetLastError();
}

}  // namespace moe
