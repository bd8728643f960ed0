// Top-k routing: one wavefront per token (the selection itself is route_token in
// routing_core.h, shared with the fused front-end).  With a bit-matrix pointer the
// wavefront also writes its token's row of the bit matrix (the routing call for
// more than 64 tokens, which then needs no bit-matrix launch).
#include "act_split.h"
#include "launch.h"
#include "routing_core.h"

namespace moe {
namespace {

// Workgroups from route_blocks on convert x instead (act_split_block, one thread per
// 32-element block); they share no data with the routing workgroups.
template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int64_t T,
                                                    int E, int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ weights,
                                                    uint32_t* __restrict__ bm, int route_blocks,
                                                    const uint16_t* __restrict__ sx,
                                                    int64_t s_blocks, int sK,
                                                    uint8_t* __restrict__ sxq,
                                                    uint8_t* __restrict__ sxs) {
  if (static_cast<int>(blockIdx.x) >= route_blocks) {   // uniform per workgroup
    const int64_t bid = static_cast<int64_t>(blockIdx.x - route_blocks) * 256 + threadIdx.x;
    if (bid < s_blocks) act_split_block(sx, bid, sK, sxq, sxs);
    return;
  }
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
                        float* weights, hipStream_t stream, uint32_t* bm, const SplitArgs* split) {
  const int epl = (E + 63) / 64;
  const int route_blocks = static_cast<int>((T + 3) / 4);
  const int64_t s_blocks = split ? split->rows * (split->K / 32) : 0;
  const int split_groups = static_cast<int>((s_blocks + 255) / 256);
  const dim3 grid(static_cast<unsigned>(route_blocks + split_groups)), block(256);
  const uint16_t* sx = split ? split->x : nullptr;
  const int sK = split ? split->K : 0;
  uint8_t* sxq = split ? split->xq : nullptr;
  uint8_t* sxs = split ? split->xs : nullptr;
#define MOE_ROUTE(EPL)                                                                        \
  route_kernel<EPL><<<grid, block, 0, stream>>>(logits, T, E, k, ids, weights, bm, route_blocks, \
                                                sx, s_blocks, sK, sxq, sxs)
  if (epl <= 1)
    MOE_ROUTE(1);
  else if (epl <= 2)
    MOE_ROUTE(2);
  else if (epl <= 4)
    MOE_ROUTE(4);
  else if (epl <= 8)
    MOE_ROUTE(8);
  else
    MOE_ROUTE(16);
#undef MOE_ROUTE
  return hipGetLastError();
}

}  // namespace moe
