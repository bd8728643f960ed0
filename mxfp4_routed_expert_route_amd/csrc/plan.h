// The grouped FFN's row-tile plan, written by one workgroup whose thread e holds
// expert e's row count and first row (the plan kernel, or the expert-offsets scan
// when it can write the plan itself): expert e is cut into ceil(count / tile_rows)
// tiles of consecutive rows, experts in index order, so only experts with rows get
// tiles.  Writes at most tile_bound tiles and their number.
#pragma once
#include "config.h"
#include "device.h"

namespace moe {

// blockDim.x <= 1024 threads (16 wavefronts), every thread of the workgroup calls
// this; wave_tot is a __shared__ int[16].  e >= E contributes no tiles.
__device__ __forceinline__ void write_tile_plan(int e, int E, int count, int begin, int tile_rows,
                                                int64_t tile_bound, int32_t* __restrict__ n_tiles,
                                                RowTile* __restrict__ tiles, int* wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nt = e < E ? (count + tile_rows - 1) / tile_rows : 0;
  int incl = nt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wave_tot[w];
  const int first = base + incl - nt;
  for (int i = 0; i < nt; ++i) {
    const int64_t slot = static_cast<int64_t>(first) + i;
    if (slot >= tile_bound) break;
    RowTile rt;
    rt.expert = e;
    rt.p_begin = begin + i * tile_rows;
    rt.p_end = (i + 1) * tile_rows < count ? begin + (i + 1) * tile_rows : begin + count;
    rt.multi = count > tile_rows ? 1 : 0;
    tiles[slot] = rt;
  }
  if (threadIdx.x == blockDim.x - 1) {
    const int64_t total = base + incl;
    *n_tiles = static_cast<int32_t>(total < tile_bound ? total : tile_bound);
  }
}

}  // namespace moe
