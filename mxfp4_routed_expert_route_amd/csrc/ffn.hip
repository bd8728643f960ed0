// Grouped expert FFN over MXFP4 weights: the row-tile plan and the dispatch of
// W1 (gate|up with the clamped SwiGLU epilogue) and W2.
//
// A plan kernel cuts each expert's rows [offsets[e], offsets[e+1]) into row tiles
// (1, 16, 32, 80 or 128 rows, chosen from T, the mean rows per expert and the
// dims); only experts with rows get tiles.  Fewer rows than experts (decode,
// verify): the GEMV kernel (ffn_gemv.hip), weights streamed past one row per
// tile on the vector ALUs.  Few rows per expert: the streaming kernel (ffn_stream.hip),
// bf16 MFMAs, bound by HBM.  Many rows: the tiled kernels (ffn_tile.hip),
// block-scaled FP4 x FP8 MFMAs on an LDS activation tile.
#include "ffn_common.h"
#include "launch.h"
#include "plan.h"
#include "validate.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- plan

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ counts,
                                                    const int32_t* __restrict__ offsets, int E,
                                                    int tile_rows, int64_t n_slots, int64_t tile_bound,
                                                    int32_t* __restrict__ n_tiles,
                                                    RowTile* __restrict__ tiles) {
  __shared__ int wave_tot[16];
  const int e = threadIdx.x;
  int c = 0, begin = 0;
  if (e < E) {
    c = counts[e];
    begin = offsets[e];
    if (c < 0 || begin < 0 || begin > n_slots) c = 0;
    if (static_cast<int64_t>(begin) + c > n_slots) c = static_cast<int>(n_slots - begin);
  }
  write_tile_plan(e, E, c, begin, tile_rows, tile_bound, n_tiles, tiles, wave_tot);
}

}  // namespace

hipError_t launch_ffn(const uint16_t* x, int64_t T, int H, int I, int E, int k,
                      const uint8_t* w1, const uint8_t* w1s, const uint8_t* w2,
                      const uint8_t* w2s, const int32_t* counts, const int32_t* offsets,
                      const int32_t* gather, float limit, uint16_t* y_sorted, void* ws,
                      const WsLayout& L, hipStream_t stream, hipEvent_t const* events,
                      bool plan_ready, const CombineArgs* combine, bool* combined,
                      bool split_ready) {
  if (combined) *combined = false;
  const int64_t n_slots = T * k;
  char* wsb = static_cast<char*>(ws);
  uint16_t* h = reinterpret_cast<uint16_t*>(wsb + L.ffn_h_offset);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(wsb + L.ffn_plan_offset);
  RowTile* tiles = reinterpret_cast<RowTile*>(wsb + L.ffn_plan_offset + 256);
  const bool clamp = limit > 0.f && limit <= 3.402823466e38f;   // finite and positive
  const int clamp_i = clamp ? 1 : 0;
  const int slots_i = static_cast<int>(n_slots);
  const uint32_t x_bytes = static_cast<uint32_t>(T * H * 2);         // < 2^32 - 2^20 (host check)
  const uint32_t h_bytes = static_cast<uint32_t>(n_slots * I * 2);

  // Few rows per expert -> weight streaming with 16- or 32-row tiles; else 80- or 128-row
  // tiles (ffn_tile_rows).  The plan may already be in the workspace (written by
  // the one-launch front-end of moe_forward_mxfp4 under the same rule).
  const int tile_rows = ffn_tile_rows(T, E, k, H, I);
  const int64_t tile_bound = ffn_tile_bound(n_slots, E, tile_rows);

  hipError_t err = hipSuccess;
  if (!plan_ready) {
    plan_kernel<<<1, 1024, 0, stream>>>(counts, offsets, E, tile_rows, n_slots, tile_bound,
                                        n_tiles, tiles);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const bool tiled = tile_rows >= 80;
  if (tiled && !split_ready) {   // x in two-part FP8 for the tiled kernels (ahead of the W1 event)
    err = launch_act_split(x, T, H, reinterpret_cast<uint8_t*>(wsb + L.ffn_xq_offset),
                           reinterpret_cast<uint8_t*>(wsb + L.ffn_xs_offset), stream);
    if (err != hipSuccess) return err;
  }
  if (events) {
    err = hipEventRecord(events[0], stream);
    if (err != hipSuccess) return err;
  }

  if (tile_rows == kFfnGemvTileRows) {
    // decode GEMV: W1 4 gate rows (and their up rows) per wavefront, W2 8 rows
    err = launch_gemv(true, tile_bound, stream, x, gather, k, slots_i, w1, w1s, tiles, n_tiles, H,
                      2 * I, I, limit, clamp_i, h, I);
    if (err != hipSuccess) return err;
    if (events) {
      err = hipEventRecord(events[1], stream);
      if (err != hipSuccess) return err;
    }
    if (combine) {   // W2 and the combine in one launch, token by token
      err = launch_gemv_w2_combine(T, k, E, slots_i, stream, h, combine->topk_ids,
                                   combine->topk_weights, combine->scatter, w2, w2s, I, H,
                                   y_sorted, combine->y);
      if (err == hipSuccess && combined) *combined = true;
    } else {
      err = launch_gemv(false, tile_bound, stream, h, nullptr, k, slots_i, w2, w2s, tiles,
                        n_tiles, I, H, 0, limit, 0, y_sorted, H);
    }
  } else if (tile_rows <= 32) {
    // W1: 8 * frags gate rows (and as many up rows) per wavefront; W2: 16 * frags rows
    const int frags = stream_frags(tile_rows / 16);
    const int wpt1 = I / (8 * frags), wpt2 = H / (16 * frags);
    unsigned g1 = static_cast<unsigned>((tile_bound * wpt1 + 3) / 4);
    unsigned g2 = static_cast<unsigned>((tile_bound * wpt2 + 3) / 4);
    if (tile_rows == 32) {   // whole tiles per XCD: grids in steps of 8 tiles
      const unsigned s1 = 8u * (wpt1 / 4), s2 = 8u * (wpt2 / 4);
      if (wpt1 % 4 == 0) g1 = (g1 + s1 - 1) / s1 * s1;
      if (wpt2 % 4 == 0) g2 = (g2 + s2 - 1) / s2 * s2;
    }
    const RowTile* t = tiles;
    const int msub = tile_rows / 16;
    err = launch_stream(true, msub, g1, stream, x, x_bytes, gather, k, slots_i, w1, w1s, t,
                        n_tiles, H, 2 * I, I, wpt1, limit, clamp_i, h, I);
    if (err != hipSuccess) return err;
    if (events) {
      err = hipEventRecord(events[1], stream);
      if (err != hipSuccess) return err;
    }
    err = launch_stream(false, msub, g2, stream, h, h_bytes, nullptr, k, slots_i, w2, w2s, t,
                        n_tiles, I, H, 0, wpt2, limit, 0, y_sorted, H);
  } else {
    // Tiled path: block-scaled FP4 x FP8 MFMAs on two-part FP8 activations (x was
    // split above); W1 writes h in that form, W2 reads it.
    uint8_t* xq = reinterpret_cast<uint8_t*>(wsb + L.ffn_xq_offset);
    uint8_t* xs = reinterpret_cast<uint8_t*>(wsb + L.ffn_xs_offset);
    uint8_t* hs = reinterpret_cast<uint8_t*>(wsb + L.ffn_hs_offset);
    // 80-row tiles with at most 64 rows per expert on average (most experts one
    // tile, so no weight slice to share between an expert's tiles): each XCD takes
    // whole tiles, and a tile's activation chunks are fetched into one L2
    const bool whole = tile_rows == 80 && T * k / E <= 64;
    TileArgs t1{tile_bound, xq, x_bytes, xs, static_cast<uint32_t>(T * (H / 32)), gather, k,
                slots_i, w1, w1s, tiles, n_tiles, H, 2 * I, I, limit, clamp_i, h, hs, I, whole};
    TileArgs t2{tile_bound, reinterpret_cast<const uint8_t*>(h), h_bytes, hs,
                static_cast<uint32_t>(n_slots * (I / 32)), nullptr, k, slots_i, w2, w2s, tiles,
                n_tiles, I, H, 0, limit, 0, y_sorted, nullptr, H, whole};
    err = launch_tile(true, tile_rows, t1, stream);
    if (err != hipSuccess) return err;
    if (events) {
      err = hipEventRecord(events[1], stream);
      if (err != hipSuccess) return err;
    }
    err = launch_tile(false, tile_rows, t2, stream);
  }
  if (err != hipSuccess || !events) return err;
  return hipEventRecord(events[2], stream);
}

}  // namespace moe
