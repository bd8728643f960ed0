// Expert histogram, exclusive prefix sum, and gather / scatter permutations.
//
// Expert-major grouping of the (token, slot) rows before the expert products (the
// grouped-expert step of the deployment's README, mynewscn.com translation).
// Three small kernels, all deterministic (integer work, no order-dependent atomics):
//   1. block_counts: a workgroup owns 1024 consecutive tokens (16 wavefronts x 64
//      tokens, one token per lane).  For each expert e a wavefront takes a ballot
//      of "my token's bit e is set"; the popcount is that wavefront's count.  The
//      workgroup's per-expert sum goes to the workspace.
//   2. scan: one workgroup; thread e turns the per-block counts of expert e into
//      exclusive per-block bases (in place) and the total counts[e]; a workgroup
//      scan over e gives offsets.
//   3. ranks: the same 1024-token workgroups recount per wavefront, prefix the
//      wavefront counts per expert in LDS, then ballot again: a lane whose token
//      chose e has rank popcount(ballot & lanes-below-me) among the wavefront's
//      tokens, so its row is p = offsets[e] + block base + wavefront base + rank
//      (tokens ascending within an expert).  The slot j comes from topk_ids.
#include "config.h"
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kWaves = kOffsBlockTokens / 64;   // 16

// Per-wavefront expert counts into cnt[wave][e]; returns nothing.
__device__ __forceinline__ void wave_expert_counts(const uint32_t* __restrict__ bm, int64_t t,
                                                   bool valid, int E, int words, int lane,
                                                   int* __restrict__ cnt_row) {
  int mine = 0;
  for (int w = 0; w < words; ++w) {
    const uint32_t word = valid ? bm[t * words + w] : 0u;
    const int nbits = (E - w * 32) < 32 ? (E - w * 32) : 32;
    for (int b = 0; b < nbits; ++b) {
      const int e = w * 32 + b;
      const unsigned long long m = __ballot((word >> b) & 1u);
      if (lane == (e & 63)) mine = __popcll(m);
      if ((e & 63) == 63 || e == E - 1) {
        if (lane <= (e & 63)) cnt_row[(e & ~63) + lane] = mine;
      }
    }
  }
}

__global__ __launch_bounds__(1024) void block_counts_kernel(const uint32_t* __restrict__ bm,
                                                            int64_t T, int E, int words,
                                                            int32_t* __restrict__ blk) {
  extern __shared__ int cnt[];   // [kWaves][E]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kOffsBlockTokens + threadIdx.x;
  wave_expert_counts(bm, t, t < T, E, words, lane, cnt + wave * E);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int s = 0;
    for (int w = 0; w < kWaves; ++w) s += cnt[w * E + e];
    blk[static_cast<int64_t>(blockIdx.x) * E + e] = s;
  }
}

__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ blk, int64_t n_blocks,
                                                    int E, int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets) {
  __shared__ int wave_tot[16];
  const int e = threadIdx.x;
  const int lane = e & 63, wave = e >> 6;
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
  // exclusive scan of run over e: wavefront inclusive scan, then wavefront totals
  int incl = run;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wave_tot[w];
  if (e < E) offsets[e] = base + incl - run;
  if (e == E - 1) offsets[E] = base + incl;
}

__global__ __launch_bounds__(1024) void ranks_kernel(const uint32_t* __restrict__ bm,
                                                     const int32_t* __restrict__ ids, int64_t T,
                                                     int E, int k, int words,
                                                     const int32_t* __restrict__ blk,
                                                     const int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ gather,
                                                     int32_t* __restrict__ scatter) {
  extern __shared__ int cnt[];   // [kWaves][E] -> row bases
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kOffsBlockTokens + threadIdx.x;
  const bool valid = t < T;
  wave_expert_counts(bm, t, valid, E, words, lane, cnt + wave * E);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int base = offsets[e] + blk[static_cast<int64_t>(blockIdx.x) * E + e];
    for (int w = 0; w < kWaves; ++w) {
      const int c = cnt[w * E + e];
      cnt[w * E + e] = base;
      base += c;
    }
  }
  __syncthreads();

  int my_ids[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) my_ids[j] = (valid && j < k) ? ids[t * k + j] : -1;
  const int64_t n_slots = T * k;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int w = 0; w < words; ++w) {
    const uint32_t word = valid ? bm[t * words + w] : 0u;
    const int nbits = (E - w * 32) < 32 ? (E - w * 32) : 32;
    for (int b = 0; b < nbits; ++b) {
      const bool mine = (word >> b) & 1u;
      const unsigned long long m = __ballot(mine);
      if (mine) {
        const int e = w * 32 + b;
        const int64_t p = static_cast<int64_t>(cnt[wave * E + e]) + __popcll(m & below);
        int j = -1;
#pragma unroll
        for (int q = 0; q < kMaxK; ++q)
          if (my_ids[q] == e) j = q;
        if (j >= 0 && p >= 0 && p < n_slots) {
          const int64_t s = t * k + j;
          gather[p] = static_cast<int32_t>(s);
          scatter[s] = static_cast<int32_t>(p);
        }
      }
    }
  }
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
                          void* ws, hipStream_t stream) {
  if (T == 0) {
    zero_counts_kernel<<<1, 256, 0, stream>>>(counts, offsets, E);
    return hipGetLastError();
  }
  const int words = (E + 31) / 32;
  const int64_t n_blocks = (T + kOffsBlockTokens - 1) / kOffsBlockTokens;
  int32_t* blk = static_cast<int32_t*>(ws);
  const size_t lds = static_cast<size_t>(kWaves) * E * sizeof(int);
  block_counts_kernel<<<dim3(static_cast<unsigned>(n_blocks)), dim3(kOffsBlockTokens), lds, stream>>>(
      bm, T, E, words, blk);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  scan_kernel<<<1, 1024, 0, stream>>>(blk, n_blocks, E, counts, offsets);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  ranks_kernel<<<dim3(static_cast<unsigned>(n_blocks)), dim3(kOffsBlockTokens), lds, stream>>>(
      bm, ids, T, E, k, words, blk, offsets, gather, scatter);
  return hipGetLastError();
}

}  // namespace moe
