// Top-k routing: one wavefront per token.
//
// Selection rule (txtmix.com article, §1 and §3: top-6 of 256 experts per token,
// the "fast DeepSeek routing" step): the k largest logits, ordered by logit
// descending then expert index ascending; -0.0 ranks equal to +0.0.  Weights:
// softmax over the k chosen logits.
//
// Each lane holds EPL logits (expert e = i*64 + lane, coalesced loads) as 64-bit
// keys (order-preserving logit bits << 32 | ~e), so one unsigned max picks the
// larger logit and, on a tie, the lower index.  k rounds of a wave-wide max
// (butterfly) take the winners in order; the winner's key is retired in the lane
// that holds it.
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t order_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;   // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_bits_to_f32(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int64_t T,
                                                    int E, int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;   // uniform per wavefront
  const float* row = logits + t * E;

  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = i * 64 + lane;
    key[i] = (e < E) ? ((static_cast<uint64_t>(order_bits(row[e])) << 32) | static_cast<uint32_t>(~e))
                     : 0ull;   // below every real key
  }

  int my_id = 0;
  float my_logit = 0.f, top = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) best = key[i] > best ? key[i] : best;
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) {
      const uint64_t o = shfl_xor_u64(best, m);
      best = o > best ? o : best;
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (key[i] == best) key[i] = 0ull;
    const float l = order_bits_to_f32(static_cast<uint32_t>(best >> 32));
    if (j == 0) top = l;
    if (lane == j) {
      my_id = static_cast<int>(~static_cast<uint32_t>(best));
      my_logit = l;
    }
  }

  // softmax over the selection: fp32 exponentials, fp64 sum in j order
  const float ex = (lane < k) ? expf(my_logit - top) : 0.f;
  double sum = 0.0;
  for (int j = 0; j < k; ++j) sum += static_cast<double>(__shfl(ex, j, 64));
  if (lane < k) {
    ids[t * k + lane] = my_id;
    weights[t * k + lane] = static_cast<float>(static_cast<double>(ex) / sum);
  }
}

}  // namespace

hipError_t launch_route(const float* logits, int64_t T, int E, int k, int32_t* ids,
                        float* weights, hipStream_t stream) {
  const int epl = (E + 63) / 64;
  const dim3 grid(static_cast<unsigned>((T + 3) / 4)), block(256);
  if (epl <= 1)
    route_kernel<1><<<grid, block, 0, stream>>>(logits, T, E, k, ids, weights);
  else if (epl <= 2)
    route_kernel<2><<<grid, block, 0, stream>>>(logits, T, E, k, ids, weights);
  else if (epl <= 4)
    route_kernel<4><<<grid, block, 0, stream>>>(logits, T, E, k, ids, weights);
  else if (epl <= 8)
    route_kernel<8><<<grid, block, 0, stream>>>(logits, T, E, k, ids, weights);
  else
    route_kernel<16><<<grid, block, 0, stream>>>(logits, T, E, k, ids, weights);
  return hipGetLastError();
}

}  // namespace moe
