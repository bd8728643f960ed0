// Host-side argument checks and workspace layout.  Pure C++: no HIP calls, so the
// same code builds and runs on a machine without a GPU.
#pragma once
#include <cstddef>
#include <cstdint>

#include "../../include/moe_mxfp4.h"

namespace moe {

struct WsLayout {
  size_t offsets_bytes;   // per-block expert counts for moe_expert_offsets
  size_t ffn_h_offset;    // [T*k][I] intermediate activations: bf16, or two-part FP8 (2 bytes
                          // per value) on the tiled path
  size_t ffn_hs_offset;   // tiled path: [T*k][I/32] E8M0 scales of h
  size_t ffn_xq_offset;   // tiled path: [T][2H] bytes, x in two-part FP8
  size_t ffn_xs_offset;   // tiled path: [T][H/32] E8M0 scales of x
  size_t ffn_plan_offset; // row-tile count + RowTile list
  size_t ffn_bytes;
  size_t total;
  int64_t n_blocks;       // moe_expert_offsets workgroups
  int64_t tile_bound;     // upper bound on FFN row tiles
};

// Fills `out` for valid sizes (E, k as for moe_route; H, I as for the FFN; H or I
// may be 0 when only the routing part is wanted) and returns MOE_OK.
moe_status workspace_layout(int64_t T, int32_t E, int32_t k, int32_t H, int32_t I, WsLayout* out);

moe_status check_route(const void* logits, int64_t T, int32_t E, int32_t k, const void* ids,
                       const void* weights);
moe_status check_bitmatrix(const void* ids, int64_t T, int32_t E, int32_t k, const void* bm);
moe_status check_offsets(const void* bm, const void* ids, int64_t T, int32_t E, int32_t k,
                         const void* counts, const void* offsets, const void* gather,
                         const void* scatter, const void* ws, size_t ws_bytes);
moe_status check_ffn(const void* x, int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                     const void* w1, const void* w1s, const void* w2, const void* w2s,
                     const void* counts, const void* offsets, const void* gather,
                     const void* y_sorted, const void* ws, size_t ws_bytes);
moe_status check_combine(const void* y_sorted, const void* w, const void* scatter, int64_t T,
                         int32_t H, int32_t k, const void* y);

}  // namespace moe
