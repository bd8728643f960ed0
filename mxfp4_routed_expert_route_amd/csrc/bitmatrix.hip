// Token x expert routing bit matrix.
//
// A wavefront owns a logical block of floor(64/k) tokens, i.e. floor(64/k)*k
// (token, slot) entries, one per lane; with k = 6 that is 60 entries and lanes
// 60..63 are padding.  The txtmix.com article, §3, and the aihot.vn README
// translation, section "Định tuyến MXFP4", describe the failure this guards
// against: padding lanes masked only by the global bound carry entries that are
// not theirs.  Here a lane is active only if it lies inside the logical block AND
// its entry lies inside the T*k entries.  Active lanes OR their bit into the
// wavefront's rows in LDS (integer OR: order-independent), then the wavefront
// writes its rows, every word, with coalesced stores.
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;

__global__ __launch_bounds__(256) void bitmatrix_kernel(const int32_t* __restrict__ ids, int64_t T,
                                                        int E, int k, int words,
                                                        uint32_t* __restrict__ bm) {
  extern __shared__ uint32_t rows_lds[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tokens_per_wave = 64 / k;
  const int logical_block = tokens_per_wave * k;
  const int64_t tok0 = (static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave) * tokens_per_wave;
  uint32_t* rows = rows_lds + wave * tokens_per_wave * words;
  const int n_words = tokens_per_wave * words;

  for (int i = lane; i < n_words; i += 64) rows[i] = 0u;
  __syncthreads();

  const int64_t entry = tok0 * k + lane;
  const bool active = (lane < logical_block) && (entry < T * k);
  if (active) {
    const int e = ids[entry];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E))
      atomicOr(&rows[(lane / k) * words + (e >> 5)], 1u << (e & 31));
  }
  __syncthreads();

  for (int i = lane; i < n_words; i += 64) {
    const int64_t t = tok0 + i / words;
    if (t < T) bm[tok0 * words + i] = rows[i];
  }
}

}  // namespace

hipError_t launch_bitmatrix(const int32_t* ids, int64_t T, int E, int k, uint32_t* bm,
                            hipStream_t stream) {
  const int words = (E + 31) / 32;
  const int tokens_per_block = (64 / k) * kWavesPerBlock;
  const dim3 grid(static_cast<unsigned>((T + tokens_per_block - 1) / tokens_per_block)), block(256);
  const size_t lds = static_cast<size_t>(kWavesPerBlock) * (64 / k) * words * sizeof(uint32_t);
  bitmatrix_kernel<<<grid, block, lds, stream>>>(ids, T, E, k, words, bm);
  return hipGetLastError();
}

}  // namespace moe
