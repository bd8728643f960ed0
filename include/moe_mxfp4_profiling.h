/*
 * moe_mxfp4_profiling.h -- instrumented variants of moe_grouped_ffn_mxfp4 and
 * moe_forward_mxfp4 for measurement tools.
 *
 * For callers that time the grouped FFN's kernels one by one (benchmarks, the
 * roofline report): it does exactly what moe_grouped_ffn_mxfp4 does (same
 * arguments, checks, kernels and stream; see moe_mxfp4.h) and additionally
 * records three caller-owned events on `stream`:
 *   events[0]  after the row-tile plan, just before the W1 (gate|up + SwiGLU) kernel
 *   events[1]  after the W1 kernel, just before the W2 kernel
 *   events[2]  after the W2 kernel
 * Each entry is a hipEvent_t created by the caller (passed as void*); all three
 * must be non-NULL when T > 0.  Elapsed time between consecutive events is the
 * duration of one kernel.  T = 0 records nothing.
 *
 * moe_forward_mxfp4_timed is the same for the whole layer: exactly what
 * moe_forward_mxfp4 does (same arguments, checks, kernels and stream), with the
 * three events recorded inside its FFN step:
 *   events[0]  after the routing front-end and the row-tile plan, before W1
 *   events[1]  after the W1 kernel, before the W2 kernel
 *   events[2]  after the W2 kernel.  Where the decode GEMV path (fewer routed rows
 *              than experts) folds the weighted combine into its W2 launch, that
 *              launch is the W2 kernel here; on the other paths the combine
 *              follows events[2].
 * All three must be non-NULL when T > 0; T = 0 records nothing.
 *
 * moe_read_probe is the "achievable read bandwidth" marker measured beside the
 * FFN kernels: a plain streaming read of `bytes` bytes of device memory at `buf`
 * (8192 workgroups, each reading one contiguous slab with non-temporal 16-byte
 * loads, eight in flight per lane), enqueued on `stream`.
 * Workgroup b writes the XOR of the 32-bit words it read to sink[b], so the XOR
 * of all MOE_READ_PROBE_SINK_WORDS sink words is the XOR of every 32-bit word of
 * the buffer (a check that every byte was read).  `buf` and `sink` are device
 * pointers owned by the caller; sink holds MOE_READ_PROBE_SINK_WORDS uint32.
 * Errors: NULL buf (bytes > 0) or NULL sink -> MOE_ERR_INVALID_ARGUMENT; buf not
 * 16-byte aligned or bytes not a multiple of 16 -> MOE_ERR_MISALIGNED; a failed
 * launch -> MOE_ERR_HIP.  bytes = 0 enqueues nothing.
 */
#ifndef MOE_MXFP4_PROFILING_H
#define MOE_MXFP4_PROFILING_H

#include "moe_mxfp4.h"

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_READ_PROBE_SINK_WORDS 8192

moe_status moe_grouped_ffn_mxfp4_timed(const uint16_t* x, int64_t T, int32_t H, int32_t I,
                                       int32_t E, int32_t k, const uint8_t* w1,
                                       const uint8_t* w1_scale, const uint8_t* w2,
                                       const uint8_t* w2_scale, const int32_t* counts,
                                       const int32_t* offsets, const int32_t* gather,
                                       float swiglu_limit, uint16_t* y_sorted, void* ws,
                                       size_t ws_bytes, void* const* events, void* stream);

moe_status moe_forward_mxfp4_timed(const float* logits, const uint16_t* x, int64_t T, int32_t H,
                                   int32_t I, int32_t E, int32_t k, const uint8_t* w1,
                                   const uint8_t* w1_scale, const uint8_t* w2,
                                   const uint8_t* w2_scale, float swiglu_limit, int32_t* topk_ids,
                                   float* topk_weights, uint32_t* bitmatrix, int32_t* counts,
                                   int32_t* offsets, int32_t* gather, int32_t* scatter,
                                   uint16_t* y_sorted, uint16_t* y, void* ws, size_t ws_bytes,
                                   void* const* events, void* stream);

moe_status moe_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_PROFILING_H */
