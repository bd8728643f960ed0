// Top-k routing: one wavefront per token (the selection itself is route_token in
// routing_core.h, shared with the fused front-end).  With a bit-matrix pointer the
// wavefront also writes its token's row of the bit matrix (the routing call for
// more than 64 tokens, which then needs no bit-matrix launch).
#include "launch.h"
#include "routing_core.h"

namespace moe {
namespace {

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int64_t T,
                                                    int E, int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ weights,
                                                    uint32_t* __restrict__ bm) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;   // uniform per wavefront
  int id;
  float w;
  route_token<EPL>(logits + t * E, E, k, lane, id, w);
  if (lane < k) {
    ids[t * k + lane] = id;
    weights[t * k + lane] = w;
  }
  if (bm != nullptr) {   // uniform: the token's bit-matrix row, lane w writing word w
    const int words = (E + 31) / 32;
    uint32_t word = 0;
    for (int j = 0; j < k; ++j) {
      const int e = __shfl(id, j, 64);
      if ((e >> 5) == lane) word |= 1u << (e & 31);
    }
    if (lane < words) bm[t * words + lane] = word;
  }
}

}  // namespace

hipError_t launch_route(const float* logits, int64_t T, int E, int k, int32_t* ids,
                        float* weights, hipStream_t stream, uint32_t* bm) {
  const int epl = (E + 63) / 64;
  const dim3 grid(static_cast<unsigned>((T + 3) / 4)), block(256);
  if (epl <= 1)
    route_kernel<1><<<grid, block, 0, stream>>>(logits, T, E, k, ids, weights, bm);
  else if (epl <= 2)
    route_kernel<2><<<grid, block, 0, stream>>>(logits, T, E, k, ids, weights, bm);
  else if (epl <= 4)
    route_kernel<4><<<grid, block, 0, stream>>>(logits, T, E, k, ids, weights, bm);
  else if (epl <= 8)
    route_kernel<8><<<grid, block, 0, stream>>>(logits, T, E, k, ids, weights, bm);
  else
    route_kernel<16><<<grid, block, 0, stream>>>(logits, T, E, k, ids, weights, bm);
  return hipGetLastError();
}

}  // namespace moe
