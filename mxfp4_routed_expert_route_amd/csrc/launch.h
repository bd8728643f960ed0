// Internal launchers: each enqueues its kernels on `stream` and returns the
// launch status.  Arguments are already checked by validate.cpp.
#pragma once
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace moe {

// With bm != nullptr, also the bit matrix ([T][ceil(E/32)] words, every word of
// each row written).
// x (rows x K bf16) to the tiled FFN's two-part FP8 form (xq) and block scales (xs)
struct SplitArgs {
  const uint16_t* x;
  int64_t rows;
  int K;
  uint8_t* xq;
  uint8_t* xs;
};

// With split != nullptr the routing launch also converts x (extra workgroups after
// the routing ones: the conversion streams while routing waits on its latencies).
hipError_t launch_route(const float* logits, int64_t T, int E, int k, int32_t* ids,
                        float* weights, hipStream_t stream, uint32_t* bm = nullptr,
                        const SplitArgs* split = nullptr);

hipError_t launch_bitmatrix(const int32_t* ids, int64_t T, int E, int k, uint32_t* bm,
                            hipStream_t stream);

struct PlanOut;

// With plan != nullptr (and T > 0) the one-workgroup kernel (T <= 512) or the
// scan step (larger T) also writes the FFN's row-tile plan and sets *plan_written.
hipError_t launch_offsets(const uint32_t* bm, const int32_t* ids, int64_t T, int E, int k,
                          int32_t* counts, int32_t* offsets, int32_t* gather, int32_t* scatter,
                          void* ws, hipStream_t stream, const PlanOut* plan = nullptr,
                          bool* plan_written = nullptr);

struct WsLayout;

// The weighted combine's inputs and output, for an FFN launch that may fold the
// combine into its W2 step.
struct CombineArgs {
  const int32_t* topk_ids;
  const float* topk_weights;
  const int32_t* scatter;
  uint16_t* y;
};

// The grouped FFN; `L` is the workspace layout for these sizes (validate.h).  With
// `combine` set, the decode GEMV path (one-row tiles) also writes the combined y
// from its W2 step and sets *combined; other paths leave the combine to the caller.
// split_ready: x is already in the workspace's two-part FP8 form (routing launch).
hipError_t launch_ffn(const uint16_t* x, int64_t T, int H, int I, int E, int k,
                      const uint8_t* w1, const uint8_t* w1s, const uint8_t* w2,
                      const uint8_t* w2s, const int32_t* counts, const int32_t* offsets,
                      const int32_t* gather, float limit, uint16_t* y_sorted, void* ws,
                      const WsLayout& L, hipStream_t stream, hipEvent_t const* events = nullptr,
                      bool plan_ready = false, const CombineArgs* combine = nullptr,
                      bool* combined = nullptr, bool split_ready = false);

// Where the one-launch front-end also writes the FFN's row-tile plan (count, then
// the tile list; see ffn.hip).
struct PlanOut {
  int tile_rows;
  int64_t tile_bound;
  int32_t* n_tiles;
  void* tiles;   // RowTile[tile_bound]
};

// With plan != nullptr the one-launch path (T <= 64) also writes the FFN plan and
// sets *plan_written; larger T runs the routing kernel (writing the bit matrix
// too) and the offsets kernels, whose last step writes the plan.
// With split != nullptr and T above the one-launch front-end's limit the routing
// launch also converts x (launch_route) and sets *split_done.
hipError_t launch_route_and_group(const float* logits, int64_t T, int E, int k, int32_t* ids,
                                  float* weights, uint32_t* bm, int32_t* counts, int32_t* offsets,
                                  int32_t* gather, int32_t* scatter, void* ws, hipStream_t stream,
                                  const PlanOut* plan = nullptr, bool* plan_written = nullptr,
                                  const SplitArgs* split = nullptr, bool* split_done = nullptr);

// x [rows][K] bf16 -> two-part FP8 rows (xq: [rows][2K] bytes) and their E8M0 block
// scales (xs: [rows][K/32] bytes), the input form of the tiled FFN kernels.
hipError_t launch_act_split(const uint16_t* x, int64_t rows, int K, uint8_t* xq, uint8_t* xs,
                            hipStream_t stream);

// Streaming-read marker: kReadProbeBlocks workgroups, one sink word each.
constexpr int kReadProbeBlocks = 8192;
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

hipError_t launch_combine(const uint16_t* ys, const float* w, const int32_t* scatter, int64_t T,
                          int H, int k, uint16_t* y, hipStream_t stream);

}  // namespace moe

#include "../../include/moe_mxfp4.h"

namespace moe {

// The whole layer (moe_forward_mxfp4): the host checks of every step, then the
// launches with workspace `ws` (at least moe_workspace_bytes for these sizes).
moe_status check_forward(const float* logits, const uint16_t* x, int64_t T, int32_t H, int32_t I,
                         int32_t E, int32_t k, const uint8_t* w1, const uint8_t* w1_scale,
                         const uint8_t* w2, const uint8_t* w2_scale, const int32_t* topk_ids,
                         const float* topk_weights, const uint32_t* bitmatrix,
                         const int32_t* counts, const int32_t* offsets, const int32_t* gather,
                         const int32_t* scatter, const uint16_t* y_sorted, const uint16_t* y,
                         const void* ws, size_t ws_bytes);
moe_status forward_layer(const float* logits, const uint16_t* x, int64_t T, int32_t H, int32_t I,
                         int32_t E, int32_t k, const uint8_t* w1, const uint8_t* w1_scale,
                         const uint8_t* w2, const uint8_t* w2_scale, float swiglu_limit,
                         int32_t* topk_ids, float* topk_weights, uint32_t* bitmatrix,
                         int32_t* counts, int32_t* offsets, int32_t* gather, int32_t* scatter,
                         uint16_t* y_sorted, uint16_t* y, void* ws, hipStream_t st,
                         hipEvent_t const* events = nullptr);

}  // namespace moe
