// extern "C" entry points of libmoe_mxfp4.so: host-side checks, then launches.
#include <hip/hip_runtime.h>

#include "../../include/moe_mxfp4.h"
#include "../../include/moe_mxfp4_profiling.h"
#include "config.h"
#include "launch.h"
#include "validate.h"

namespace {

moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }
hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

namespace moe {

moe_status check_forward(const float* logits, const uint16_t* x, int64_t T, int32_t H, int32_t I,
                         int32_t E, int32_t k, const uint8_t* w1, const uint8_t* w1_scale,
                         const uint8_t* w2, const uint8_t* w2_scale, const int32_t* topk_ids,
                         const float* topk_weights, const uint32_t* bitmatrix,
                         const int32_t* counts, const int32_t* offsets, const int32_t* gather,
                         const int32_t* scatter, const uint16_t* y_sorted, const uint16_t* y,
                         const void* ws, size_t ws_bytes) {
  moe_status s = check_route(logits, T, E, k, topk_ids, topk_weights);
  if (s != MOE_OK) return s;
  s = check_bitmatrix(topk_ids, T, E, k, bitmatrix);
  if (s != MOE_OK) return s;
  s = check_offsets(bitmatrix, topk_ids, T, E, k, counts, offsets, gather, scatter, ws, ws_bytes);
  if (s != MOE_OK) return s;
  s = check_ffn(x, T, H, I, E, k, w1, w1_scale, w2, w2_scale, counts, offsets, gather, y_sorted,
                ws, ws_bytes);
  if (s != MOE_OK) return s;
  return check_combine(y_sorted, topk_weights, scatter, T, H, k, y);
}

moe_status forward_layer(const float* logits, const uint16_t* x, int64_t T, int32_t H, int32_t I,
                         int32_t E, int32_t k, const uint8_t* w1, const uint8_t* w1_scale,
                         const uint8_t* w2, const uint8_t* w2_scale, float swiglu_limit,
                         int32_t* topk_ids, float* topk_weights, uint32_t* bitmatrix,
                         int32_t* counts, int32_t* offsets, int32_t* gather, int32_t* scatter,
                         uint16_t* y_sorted, uint16_t* y, void* ws, hipStream_t st,
                         hipEvent_t const* events) {
  if (T == 0)
    return from_hip(launch_offsets(nullptr, nullptr, 0, E, k, counts, offsets, nullptr, nullptr,
                                   nullptr, st));
  WsLayout L;
  moe_status s = workspace_layout(T, E, k, H, I, &L);
  if (s != MOE_OK) return s;
  // the routing side writes the FFN's row-tile plan: the one-launch front-end
  // (T <= 64), else the expert-offsets kernel (T <= 512) or its scan step
  const int tile_rows = ffn_tile_rows(T, E, k, H, I);
  char* wsb = static_cast<char*>(ws);
  const PlanOut plan{tile_rows, ffn_tile_bound(T * k, E, tile_rows),
                     reinterpret_cast<int32_t*>(wsb + L.ffn_plan_offset),
                     wsb + L.ffn_plan_offset + 256};
  bool plan_written = false;
  // the tiled FFN reads x in two-part FP8: the routing launch converts it meanwhile
  const SplitArgs split{x, T, H, reinterpret_cast<uint8_t*>(wsb + L.ffn_xq_offset),
                        reinterpret_cast<uint8_t*>(wsb + L.ffn_xs_offset)};
  bool split_done = false;
  hipError_t e = launch_route_and_group(logits, T, E, k, topk_ids, topk_weights, bitmatrix,
                                        counts, offsets, gather, scatter, ws, st, &plan,
                                        &plan_written, ffn_tiled(T, E, k, H, I) ? &split : nullptr,
                                        &split_done);
  if (e != hipSuccess) return MOE_ERR_HIP;
  // on the decode GEMV path the W2 launch also writes y (same arithmetic as the combine)
  const CombineArgs fold{topk_ids, topk_weights, scatter, y};
  bool combined = false;
  e = launch_ffn(x, T, H, I, E, k, w1, w1_scale, w2, w2_scale, counts, offsets, gather,
                 swiglu_limit, y_sorted, ws, L, st, events, plan_written, &fold, &combined,
                 split_done);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (combined) return MOE_OK;
  return from_hip(launch_combine(y_sorted, topk_weights, scatter, T, H, k, y, st));
}

}  // namespace moe

extern "C" {

moe_status moe_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_ids,
                     float* topk_weights, void* stream) {
  moe_status s = moe::check_route(logits, T, E, k, topk_ids, topk_weights);
  if (s != MOE_OK || T == 0) return s;
  return from_hip(moe::launch_route(logits, T, E, k, topk_ids, topk_weights, as_stream(stream)));
}

moe_status moe_build_bitmatrix(const int32_t* topk_ids, int64_t T, int32_t E, int32_t k,
                               uint32_t* bitmatrix, void* stream) {
  moe_status s = moe::check_bitmatrix(topk_ids, T, E, k, bitmatrix);
  if (s != MOE_OK || T == 0) return s;
  return from_hip(moe::launch_bitmatrix(topk_ids, T, E, k, bitmatrix, as_stream(stream)));
}

moe_status moe_expert_offsets(const uint32_t* bitmatrix, const int32_t* topk_ids, int64_t T,
                              int32_t E, int32_t k, int32_t* counts, int32_t* offsets,
                              int32_t* gather, int32_t* scatter, void* ws, size_t ws_bytes,
                              void* stream) {
  moe_status s = moe::check_offsets(bitmatrix, topk_ids, T, E, k, counts, offsets, gather,
                                    scatter, ws, ws_bytes);
  if (s != MOE_OK) return s;
  return from_hip(moe::launch_offsets(bitmatrix, topk_ids, T, E, k, counts, offsets, gather,
                                      scatter, ws, as_stream(stream)));
}

moe_status moe_route_and_group(const float* logits, int64_t T, int32_t E, int32_t k,
                               int32_t* topk_ids, float* topk_weights, uint32_t* bitmatrix,
                               int32_t* counts, int32_t* offsets, int32_t* gather,
                               int32_t* scatter, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = moe::check_route(logits, T, E, k, topk_ids, topk_weights);
  if (s != MOE_OK) return s;
  s = moe::check_bitmatrix(topk_ids, T, E, k, bitmatrix);
  if (s != MOE_OK) return s;
  s = moe::check_offsets(bitmatrix, topk_ids, T, E, k, counts, offsets, gather, scatter, ws,
                         ws_bytes);
  if (s != MOE_OK) return s;
  if (T == 0)
    return from_hip(moe::launch_offsets(nullptr, nullptr, 0, E, k, counts, offsets, nullptr,
                                        nullptr, nullptr, as_stream(stream)));
  return from_hip(moe::launch_route_and_group(logits, T, E, k, topk_ids, topk_weights, bitmatrix,
                                              counts, offsets, gather, scatter, ws,
                                              as_stream(stream)));
}

moe_status moe_grouped_ffn_mxfp4(const uint16_t* x, int64_t T, int32_t H, int32_t I, int32_t E,
                                 int32_t k, const uint8_t* w1, const uint8_t* w1_scale,
                                 const uint8_t* w2, const uint8_t* w2_scale,
                                 const int32_t* counts, const int32_t* offsets,
                                 const int32_t* gather, float swiglu_limit, uint16_t* y_sorted,
                                 void* ws, size_t ws_bytes, void* stream) {
  moe_status s = moe::check_ffn(x, T, H, I, E, k, w1, w1_scale, w2, w2_scale, counts, offsets,
                                gather, y_sorted, ws, ws_bytes);
  if (s != MOE_OK || T == 0) return s;
  moe::WsLayout L;
  s = moe::workspace_layout(T, E, k, H, I, &L);
  if (s != MOE_OK) return s;
  return from_hip(moe::launch_ffn(x, T, H, I, E, k, w1, w1_scale, w2, w2_scale, counts, offsets,
                                  gather, swiglu_limit, y_sorted, ws, L, as_stream(stream)));
}

moe_status moe_forward_mxfp4(const float* logits, const uint16_t* x, int64_t T, int32_t H,
                             int32_t I, int32_t E, int32_t k, const uint8_t* w1,
                             const uint8_t* w1_scale, const uint8_t* w2, const uint8_t* w2_scale,
                             float swiglu_limit, int32_t* topk_ids, float* topk_weights,
                             uint32_t* bitmatrix, int32_t* counts, int32_t* offsets,
                             int32_t* gather, int32_t* scatter, uint16_t* y_sorted, uint16_t* y,
                             void* ws, size_t ws_bytes, void* stream) {
  moe_status s = moe::check_forward(logits, x, T, H, I, E, k, w1, w1_scale, w2, w2_scale,
                                    topk_ids, topk_weights, bitmatrix, counts, offsets, gather,
                                    scatter, y_sorted, y, ws, ws_bytes);
  if (s != MOE_OK) return s;
  return moe::forward_layer(logits, x, T, H, I, E, k, w1, w1_scale, w2, w2_scale, swiglu_limit,
                            topk_ids, topk_weights, bitmatrix, counts, offsets, gather, scatter,
                            y_sorted, y, ws, as_stream(stream));
}

moe_status moe_grouped_ffn_mxfp4_timed(const uint16_t* x, int64_t T, int32_t H, int32_t I,
                                       int32_t E, int32_t k, const uint8_t* w1,
                                       const uint8_t* w1_scale, const uint8_t* w2,
                                       const uint8_t* w2_scale, const int32_t* counts,
                                       const int32_t* offsets, const int32_t* gather,
                                       float swiglu_limit, uint16_t* y_sorted, void* ws,
                                       size_t ws_bytes, void* const* events, void* stream) {
  moe_status s = moe::check_ffn(x, T, H, I, E, k, w1, w1_scale, w2, w2_scale, counts, offsets,
                                gather, y_sorted, ws, ws_bytes);
  if (s != MOE_OK || T == 0) return s;
  if (!events || !events[0] || !events[1] || !events[2]) return MOE_ERR_INVALID_ARGUMENT;
  moe::WsLayout L;
  s = moe::workspace_layout(T, E, k, H, I, &L);
  if (s != MOE_OK) return s;
  hipEvent_t ev[3] = {static_cast<hipEvent_t>(events[0]), static_cast<hipEvent_t>(events[1]),
                      static_cast<hipEvent_t>(events[2])};
  return from_hip(moe::launch_ffn(x, T, H, I, E, k, w1, w1_scale, w2, w2_scale, counts, offsets,
                                  gather, swiglu_limit, y_sorted, ws, L, as_stream(stream), ev));
}

moe_status moe_forward_mxfp4_timed(const float* logits, const uint16_t* x, int64_t T, int32_t H,
                                   int32_t I, int32_t E, int32_t k, const uint8_t* w1,
                                   const uint8_t* w1_scale, const uint8_t* w2,
                                   const uint8_t* w2_scale, float swiglu_limit, int32_t* topk_ids,
                                   float* topk_weights, uint32_t* bitmatrix, int32_t* counts,
                                   int32_t* offsets, int32_t* gather, int32_t* scatter,
                                   uint16_t* y_sorted, uint16_t* y, void* ws, size_t ws_bytes,
                                   void* const* events, void* stream) {
  moe_status s = moe::check_forward(logits, x, T, H, I, E, k, w1, w1_scale, w2, w2_scale,
                                    topk_ids, topk_weights, bitmatrix, counts, offsets, gather,
                                    scatter, y_sorted, y, ws, ws_bytes);
  if (s != MOE_OK) return s;
  if (T > 0 && (!events || !events[0] || !events[1] || !events[2]))
    return MOE_ERR_INVALID_ARGUMENT;
  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
  if (T > 0)
    for (int i = 0; i < 3; ++i) ev[i] = static_cast<hipEvent_t>(events[i]);
  return moe::forward_layer(logits, x, T, H, I, E, k, w1, w1_scale, w2, w2_scale, swiglu_limit,
                            topk_ids, topk_weights, bitmatrix, counts, offsets, gather, scatter,
                            y_sorted, y, ws, as_stream(stream), T > 0 ? ev : nullptr);
}

moe_status moe_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  static_assert(moe::kReadProbeBlocks == MOE_READ_PROBE_SINK_WORDS, "one sink word per workgroup");
  if (sink == nullptr || (bytes > 0 && buf == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0) return MOE_ERR_MISALIGNED;
  if (bytes == 0) return MOE_OK;
  return from_hip(moe::launch_read_probe(buf, bytes, sink, as_stream(stream)));
}

moe_status moe_combine(const uint16_t* y_sorted, const float* topk_weights,
                       const int32_t* scatter, int64_t T, int32_t H, int32_t k, uint16_t* y,
                       void* stream) {
  moe_status s = moe::check_combine(y_sorted, topk_weights, scatter, T, H, k, y);
  if (s != MOE_OK || T == 0) return s;
  return from_hip(moe::launch_combine(y_sorted, topk_weights, scatter, T, H, k, y,
                                      as_stream(stream)));
}

size_t moe_workspace_bytes(int64_t T, int32_t E, int32_t k, int32_t H, int32_t I) {
  moe::WsLayout L;
  if (moe::workspace_layout(T, E, k, H, I, &L) != MOE_OK) return 0;
  return L.total;
}

const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_MISALIGNED: return "MOE_ERR_MISALIGNED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

}  // extern "C"
