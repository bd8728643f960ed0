// The routing front-end in one launch for small batches: top-k routing, the
// token x expert bit matrix and the expert offsets / permutations, with exactly
// the outputs of moe_route, moe_build_bitmatrix and moe_expert_offsets.
//
// One workgroup of 16 wavefronts, for T <= 64 tokens:
//   1. wavefront w routes tokens w, w+16, w+32, w+48 (route_token);
//   2. the bit matrix is built in LDS: thread i owns entry i = t*k + j; the logical
//      block is the T*k entries, and threads past it (padding) stay inactive
//      (txtmix.com article, §3; aihot.vn README translation, "Định tuyến MXFP4");
//   3. every wavefront takes the column masks of 64 experts over the T rows
//      (lane = token); wavefront 0 scans their popcounts into counts and offsets
//      and writes each slot's row p = offsets[e] + rank of the token within e.
// With a plan buffer, wavefront 0 also writes the grouped FFN's row-tile plan
// (moe_forward_mxfp4), which saves the FFN its plan launch.  Larger batches run
// the routing kernel, which then also writes the bit matrix, and the offsets
// kernels of the separate call.
#include "config.h"
#include "launch.h"
#include "routing_core.h"

namespace moe {
namespace {

constexpr int kFrontMaxTokens = 64;

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int EPL>
__global__ __launch_bounds__(1024) void frontend_small_kernel(
    const float* __restrict__ logits, int T, int E, int k, int words, int32_t* __restrict__ ids,
    float* __restrict__ weights, uint32_t* __restrict__ bm, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ gather, int32_t* __restrict__ scatter,
    int tile_rows, int tile_bound, int32_t* __restrict__ n_tiles, RowTile* __restrict__ tiles) {
  __shared__ int ids_lds[kFrontMaxTokens * kMaxK];
  __shared__ uint32_t rows_lds[kFrontMaxTokens * (kMaxE / 32)];
  __shared__ uint64_t masks[kMaxE];
  __shared__ int off_lds[kMaxE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_waves = blockDim.x >> 6;

  // 1. routing
  for (int t = wave; t < T; t += n_waves) {
    int id;
    float w;
    route_token<EPL>(logits + static_cast<int64_t>(t) * E, E, k, lane, id, w);
    if (lane < k) {
      ids[t * k + lane] = id;
      weights[t * k + lane] = w;
      ids_lds[t * k + lane] = id;
    }
  }
  for (int i = threadIdx.x; i < T * words; i += blockDim.x) rows_lds[i] = 0u;
  __syncthreads();

  // 2. bit matrix: entries past T*k are padding lanes of the logical block
  const int n_entries = T * k;
  if (static_cast<int>(threadIdx.x) < n_entries) {
    const int e = ids_lds[threadIdx.x];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E))
      atomicOr(&rows_lds[(threadIdx.x / k) * words + (e >> 5)], 1u << (e & 31));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < T * words; i += blockDim.x) bm[i] = rows_lds[i];

  // 3. expert column masks, 64 experts per wavefront (lane = token), then counts,
  // offsets and permutations in wavefront 0
  for (int w0 = 2 * wave; w0 < words; w0 += 2 * n_waves)
    column_masks_64(rows_lds, lane, lane < T, E, words, lane, masks, w0);
  __syncthreads();
  if (wave != 0) return;
  int c[EPL];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane * EPL + i;
    c[i] = e < E ? __popcll(masks[e]) : 0;
    sum += c[i];
  }
  int incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  int run = incl - sum;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane * EPL + i;
    if (e < E) {
      counts[e] = c[i];
      offsets[e] = run;
      off_lds[e] = run;
    }
    run += c[i];
  }
  if (lane == 63) offsets[E] = incl;
  if (tiles != nullptr) {
    // the FFN's row-tile plan (same tiles and order as its plan kernel): expert e
    // cut into ceil(count / tile_rows) tiles, experts in index order
    int nt[EPL], tsum = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      nt[i] = (c[i] + tile_rows - 1) / tile_rows;
      tsum += nt[i];
    }
    int tincl = tsum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(tincl, d, 64);
      if (lane >= d) tincl += o;
    }
    int slot = tincl - tsum;
    int off = incl - sum;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      for (int t = 0; t < nt[i] && slot < tile_bound; ++t, ++slot) {
        RowTile rt;
        rt.expert = lane * EPL + i;
        rt.p_begin = off + t * tile_rows;
        rt.p_end = (t + 1) * tile_rows < c[i] ? off + (t + 1) * tile_rows : off + c[i];
        rt.multi = c[i] > tile_rows ? 1 : 0;
        tiles[slot] = rt;
      }
      off += c[i];
    }
    if (lane == 63) *n_tiles = tincl < tile_bound ? tincl : tile_bound;
  }
  wave_sync_lds();
  // one lane per (token, choice) entry: its row is the expert's offset plus the
  // earlier tokens that chose the same expert (bits below the token in its mask)
  for (int s = lane; s < n_entries; s += 64) {
    const int e = ids_lds[s];
    if (static_cast<unsigned>(e) >= static_cast<unsigned>(E)) continue;
    const int p = off_lds[e] + __popcll(masks[e] & ((1ull << (s / k)) - 1ull));
    if (p < 0 || p >= n_entries) continue;
    gather[p] = s;
    scatter[s] = p;
  }
}

}  // namespace

hipError_t launch_route_and_group(const float* logits, int64_t T, int E, int k, int32_t* ids,
                                  float* weights, uint32_t* bm, int32_t* counts, int32_t* offsets,
                                  int32_t* gather, int32_t* scatter, void* ws, hipStream_t stream,
                                  const PlanOut* plan, bool* plan_written,
                                  const SplitArgs* split, bool* split_done) {
  if (plan_written) *plan_written = false;
  if (split_done) *split_done = false;
  if (T > kFrontMaxTokens) {
    hipError_t err = launch_route(logits, T, E, k, ids, weights, stream, bm, split);
    if (err != hipSuccess) return err;
    if (split_done) *split_done = split != nullptr;
    return launch_offsets(bm, ids, T, E, k, counts, offsets, gather, scatter, ws, stream, plan,
                          plan_written);
  }
  const int words = (E + 31) / 32;
  const int epl = (E + 63) / 64;
  const int t = static_cast<int>(T);
  const int tile_rows = plan ? plan->tile_rows : 1;
  const int tile_bound = plan ? static_cast<int>(plan->tile_bound) : 0;
  int32_t* n_tiles = plan ? plan->n_tiles : nullptr;
  RowTile* tiles = plan ? static_cast<RowTile*>(plan->tiles) : nullptr;
  if (epl <= 1)
    frontend_small_kernel<1><<<1, 1024, 0, stream>>>(logits, t, E, k, words, ids, weights, bm,
                                                     counts, offsets, gather, scatter,
                                                     tile_rows, tile_bound, n_tiles, tiles);
  else if (epl <= 2)
    frontend_small_kernel<2><<<1, 1024, 0, stream>>>(logits, t, E, k, words, ids, weights, bm,
                                                     counts, offsets, gather, scatter,
                                                     tile_rows, tile_bound, n_tiles, tiles);
  else if (epl <= 4)
    frontend_small_kernel<4><<<1, 1024, 0, stream>>>(logits, t, E, k, words, ids, weights, bm,
                                                     counts, offsets, gather, scatter,
                                                     tile_rows, tile_bound, n_tiles, tiles);
  else if (epl <= 8)
    frontend_small_kernel<8><<<1, 1024, 0, stream>>>(logits, t, E, k, words, ids, weights, bm,
                                                     counts, offsets, gather, scatter,
                                                     tile_rows, tile_bound, n_tiles, tiles);
  else
    frontend_small_kernel<16><<<1, 1024, 0, stream>>>(logits, t, E, k, words, ids, weights, bm,
                                                      counts, offsets, gather, scatter,
                                                      tile_rows, tile_bound, n_tiles, tiles);
  const hipError_t err = hipGetLastError();
  if (err == hipSuccess && plan_written) *plan_written = tiles != nullptr;
  return err;
}

}  // namespace moe
