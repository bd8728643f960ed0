// Expert histogram, exclusive prefix sum, and gather / scatter permutations.
//
// Expert-major grouping of the (token, slot) rows before the expert products (the
// grouped-expert step of the deployment's README, mynewscn.com translation).
// Everything is integer work with no order-dependent atomics, so results are
// deterministic.
//
// Core step (wave_column_masks in routing_core.h): per wavefront of 64
// consecutive tokens, the 64-bit column mask of every expert; its popcount is
// the expert's count and popcount(mask & lanes-below) a token's rank among the
// expert's tokens, so an expert's rows come out in token order.
//
// Workgroups own 512 consecutive tokens (8 wavefronts).  T <= 512: one fused
// kernel does counts, offsets and permutations.  Larger T: block_counts writes
// per-workgroup expert counts, scan turns them into per-workgroup bases and
// offsets, and ranks writes the permutations.
#include "config.h"
#include "launch.h"
#include "plan.h"
#include "routing_core.h"

namespace moe {
namespace {

constexpr int kWaves = kOffsBlockTokens / 64;   // 8

// Rows of this wavefront's tokens: p = base[e] + rank of the token within e.
__device__ __forceinline__ void write_permutations(const int32_t* __restrict__ ids, int64_t t,
                                                   int64_t T, int k, int lane,
                                                   const uint64_t* __restrict__ masks,
                                                   const int32_t* __restrict__ base, int E,
                                                   int32_t* __restrict__ gather,
                                                   int32_t* __restrict__ scatter) {
  if (t >= T) return;
  const uint64_t below = (1ull << lane) - 1ull;
  const int64_t n_slots = T * k;
  int ej[kMaxK];   // the token's k expert ids, loaded together (k <= kMaxK)
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < k) ej[j] = ids[t * k + j];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j >= k) break;
    const int64_t s = t * k + j;
    const int e = ej[j];
    if (static_cast<unsigned>(e) >= static_cast<unsigned>(E)) continue;
    const int64_t p = static_cast<int64_t>(base[e]) + __popcll(masks[e] & below);
    if (p < 0 || p >= n_slots) continue;
    gather[p] = static_cast<int32_t>(s);
    scatter[s] = static_cast<int32_t>(p);
  }
}

// The FFN's row-tile plan from a workgroup whose thread t holds experts 2t and
// 2t+1 (counts c, first rows off): the same tiles, in the same expert order, as
// write_tile_plan.  Every thread calls it; wave_tot may be reused on entry only
// after a barrier.
__device__ __forceinline__ void write_tile_plan_pairs(int e0, int E, const int (&c)[2],
                                                      const int (&off)[2], int tile_rows,
                                                      int64_t tile_bound,
                                                      int32_t* __restrict__ n_tiles,
                                                      RowTile* __restrict__ tiles,
                                                      int* wave_tot) {
  int nt[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) nt[q] = e0 + q < E ? (c[q] + tile_rows - 1) / tile_rows : 0;
  int total;
  int slot0 = block_exclusive_scan(nt[0] + nt[1], wave_tot, &total);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    for (int i = 0; i < nt[q]; ++i) {
      const int64_t slot = static_cast<int64_t>(slot0) + i;
      if (slot >= tile_bound) break;
      RowTile rt;
      rt.expert = e0 + q;
      rt.p_begin = off[q] + i * tile_rows;
      rt.p_end = (i + 1) * tile_rows < c[q] ? off[q] + (i + 1) * tile_rows : off[q] + c[q];
      rt.multi = c[q] > tile_rows ? 1 : 0;
      tiles[slot] = rt;
    }
    slot0 += nt[q];
  }
  if (threadIdx.x == 0) *n_tiles = static_cast<int32_t>(total < tile_bound ? total : tile_bound);
}

// T <= 512: everything in one workgroup; with tiles != nullptr (the one-call
// layer) it also writes the FFN's row-tile plan.
__global__ __launch_bounds__(kOffsBlockTokens) void offsets_small_kernel(
    const uint32_t* __restrict__ bm, const int32_t* __restrict__ ids, int64_t T, int E, int k,
    int words, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ gather, int32_t* __restrict__ scatter, int tile_rows,
    int64_t tile_bound, int32_t* __restrict__ n_tiles, RowTile* __restrict__ tiles) {
  extern __shared__ uint64_t lds[];
  uint64_t* masks = lds;                                                   // [kWaves][E]
  int32_t* base = reinterpret_cast<int32_t*>(masks + kWaves * E);          // [kWaves][E]
  __shared__ int wave_tot[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  wave_column_masks(bm, static_cast<int64_t>(wave) * 64, T, E, words, lane, masks + wave * E);
  __syncthreads();

  // two experts per thread (E <= 1024): per-wavefront prefix, then scan over experts
  const int e0 = 2 * threadIdx.x;
  int c[2] = {0, 0};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = e0 + q;
    if (e < E) {
      int run = 0;
      for (int w = 0; w < kWaves; ++w) {
        base[w * E + e] = run;
        run += __popcll(masks[w * E + e]);
      }
      c[q] = run;
    }
  }
  int total;
  const int first = block_exclusive_scan(c[0] + c[1], wave_tot, &total);
  const int off[2] = {first, first + c[0]};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = e0 + q;
    if (e < E) {
      counts[e] = c[q];
      offsets[e] = off[q];
      for (int w = 0; w < kWaves; ++w) base[w * E + e] += off[q];
    }
  }
  if (threadIdx.x == 0) offsets[E] = total;
  __syncthreads();   // base complete; every thread has read wave_tot
  if (tiles != nullptr)   // uniform
    write_tile_plan_pairs(e0, E, c, off, tile_rows, tile_bound, n_tiles, tiles, wave_tot);
  write_permutations(ids, static_cast<int64_t>(threadIdx.x), T, k, lane, masks + wave * E,
                     base + wave * E, E, gather, scatter);
}

__global__ __launch_bounds__(kOffsBlockTokens) void block_counts_kernel(
    const uint32_t* __restrict__ bm, int64_t T, int E, int words, int32_t* __restrict__ blk) {
  extern __shared__ uint64_t masks[];   // [kWaves][E]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kOffsBlockTokens + wave * 64;
  wave_column_masks(bm, t0, T, E, words, lane, masks + wave * E);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int s = 0;
    for (int w = 0; w < kWaves; ++w) s += __popcll(masks[w * E + e]);
    blk[static_cast<int64_t>(blockIdx.x) * E + e] = s;
  }
}

// One workgroup of 1024 threads: thread e turns expert e's per-block counts into
// exclusive per-block bases (in place) and its total; a scan over e gives offsets.
// With tiles != nullptr (the one-call layer) it also writes the FFN's row-tile
// plan from the counts and offsets it holds, which saves the FFN its plan launch.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ blk, int64_t n_blocks,
                                                    int E, int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets, int tile_rows,
                                                    int64_t tile_bound, int32_t* __restrict__ n_tiles,
                                                    RowTile* __restrict__ tiles) {
  __shared__ int wave_tot[16];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    int64_t b = 0;
    for (; b + 4 <= n_blocks; b += 4) {   // four independent loads in flight
      const int c0 = blk[(b + 0) * E + e], c1 = blk[(b + 1) * E + e];
      const int c2 = blk[(b + 2) * E + e], c3 = blk[(b + 3) * E + e];
      blk[(b + 0) * E + e] = run;
      blk[(b + 1) * E + e] = run + c0;
      blk[(b + 2) * E + e] = run + c0 + c1;
      blk[(b + 3) * E + e] = run + c0 + c1 + c2;
      run += c0 + c1 + c2 + c3;
    }
    for (; b < n_blocks; ++b) {
      const int c = blk[b * E + e];
      blk[b * E + e] = run;
      run += c;
    }
    counts[e] = run;
  }
  int total;
  const int first = block_exclusive_scan(run, wave_tot, &total);
  if (e < E) offsets[e] = first;
  if (e == 0) offsets[E] = total;
  if (tiles != nullptr) {   // uniform
    __syncthreads();        // wave_tot is reused
    write_tile_plan(e, E, run, first, tile_rows, tile_bound, n_tiles, tiles, wave_tot);
  }
}

__global__ __launch_bounds__(kOffsBlockTokens) void ranks_kernel(
    const uint32_t* __restrict__ bm, const int32_t* __restrict__ ids, int64_t T, int E, int k,
    int words, const int32_t* __restrict__ blk, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ gather, int32_t* __restrict__ scatter) {
  extern __shared__ uint64_t lds[];
  uint64_t* masks = lds;                                                   // [kWaves][E]
  int32_t* base = reinterpret_cast<int32_t*>(masks + kWaves * E);          // [kWaves][E]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kOffsBlockTokens + wave * 64;
  wave_column_masks(bm, t0, T, E, words, lane, masks + wave * E);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = offsets[e] + blk[static_cast<int64_t>(blockIdx.x) * E + e];
    for (int w = 0; w < kWaves; ++w) {
      base[w * E + e] = run;
      run += __popcll(masks[w * E + e]);
    }
  }
  __syncthreads();
  write_permutations(ids, t0 + lane, T, k, lane, masks + wave * E, base + wave * E, E, gather,
                     scatter);
}

__global__ void zero_counts_kernel(int32_t* counts, int32_t* offsets, int E) {
  for (int e = threadIdx.x; e <= E; e += blockDim.x) {
    if (e < E) counts[e] = 0;
    offsets[e] = 0;
  }
}

}  // namespace

hipError_t launch_offsets(const uint32_t* bm, const int32_t* ids, int64_t T, int E, int k,
                          int32_t* counts, int32_t* offsets, int32_t* gather, int32_t* scatter,
                          void* ws, hipStream_t stream, const PlanOut* plan, bool* plan_written) {
  if (plan_written) *plan_written = false;
  if (T == 0) {
    zero_counts_kernel<<<1, 256, 0, stream>>>(counts, offsets, E);
    return hipGetLastError();
  }
  const int words = (E + 31) / 32;
  const size_t lds_masks = static_cast<size_t>(kWaves) * E * sizeof(uint64_t);
  const size_t lds_base = static_cast<size_t>(kWaves) * E * sizeof(int32_t);
  RowTile* tiles = plan ? static_cast<RowTile*>(plan->tiles) : nullptr;
  if (T <= kOffsBlockTokens) {
    offsets_small_kernel<<<1, kOffsBlockTokens, lds_masks + lds_base, stream>>>(
        bm, ids, T, E, k, words, counts, offsets, gather, scatter, plan ? plan->tile_rows : 1,
        plan ? plan->tile_bound : 0, plan ? plan->n_tiles : nullptr, tiles);
    const hipError_t err = hipGetLastError();
    if (err == hipSuccess && plan_written) *plan_written = tiles != nullptr;
    return err;
  }
  const int64_t n_blocks = (T + kOffsBlockTokens - 1) / kOffsBlockTokens;
  int32_t* blk = static_cast<int32_t*>(ws);
  const dim3 grid(static_cast<unsigned>(n_blocks)), block(kOffsBlockTokens);
  block_counts_kernel<<<grid, block, lds_masks, stream>>>(bm, T, E, words, blk);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  scan_kernel<<<1, 1024, 0, stream>>>(blk, n_blocks, E, counts, offsets,
                                      plan ? plan->tile_rows : 1, plan ? plan->tile_bound : 0,
                                      plan ? plan->n_tiles : nullptr, tiles);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (plan_written) *plan_written = tiles != nullptr;
  ranks_kernel<<<grid, block, lds_masks + lds_base, stream>>>(bm, ids, T, E, k, words, blk,
                                                              offsets, gather, scatter);
  return hipGetLastError();
}

}  // namespace moe
