// Host-side argument checks and workspace layout (no HIP calls).
#include "validate.h"

#include <climits>

#include "config.h"

namespace moe {
namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

moe_status check_sizes(int64_t T, int32_t E, int32_t k) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARGUMENT;
  if (E > kMaxE || k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (T > INT32_MAX / k) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_dims(int32_t H, int32_t I) {
  if (H <= 0 || I <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (H % 128 != 0 || I % 128 != 0 || H > kMaxDim || I > kMaxDim) return MOE_ERR_UNSUPPORTED;
  // the FFN kernels address one expert's W1 codes (2I rows of H/2 bytes) through a
  // buffer resource with a 32-bit size: below 4 GiB (only H = I = 65536 reaches it)
  if (static_cast<int64_t>(H) * I >= (int64_t{1} << 32)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Activation buffers (x: T*H bf16, h: T*k*I bf16) are addressed with 32-bit byte
// offsets; keep them below 3.5 GiB.
bool activations_fit(int64_t T, int32_t k, int32_t H, int32_t I) {
  const int64_t lim = static_cast<int64_t>(kMaxActivationBytes);
  return T * H * 2 <= lim && T * k * static_cast<int64_t>(I) * 2 <= lim &&
         T * k * static_cast<int64_t>(H) * 2 <= lim;
}

}  // namespace

moe_status workspace_layout(int64_t T, int32_t E, int32_t k, int32_t H, int32_t I, WsLayout* out) {
  moe_status s = check_sizes(T, E, k);
  if (s != MOE_OK) return s;
  if (H < 0 || I < 0) return MOE_ERR_INVALID_ARGUMENT;
  WsLayout L{};
  const int64_t slots = T * k;
  L.n_blocks = (T + kOffsBlockTokens - 1) / kOffsBlockTokens;
  L.offsets_bytes = align_up(static_cast<size_t>(L.n_blocks) * E * sizeof(int32_t), 256);
  {   // plan room for the smallest tile the FFN can take at these sizes
    const int rows = ffn_tile_rows(T, E, k, H, I);
    L.tile_bound = ffn_tile_bound(slots, E, rows < kFfnMinTileRows ? rows : kFfnMinTileRows);
  }
  L.ffn_h_offset = 0;
  size_t end = align_up(static_cast<size_t>(slots) * static_cast<size_t>(I) * 2, 256);
  L.ffn_hs_offset = L.ffn_xq_offset = L.ffn_xs_offset = end;
  if (ffn_tiled(T, E, k, H, I)) {   // two-part FP8 activations: scales of h, then x and its scales
    L.ffn_hs_offset = end;
    end = align_up(end + static_cast<size_t>(slots) * static_cast<size_t>(I / 32), 256);
    L.ffn_xq_offset = end;
    end = align_up(end + static_cast<size_t>(T) * static_cast<size_t>(H) * 2, 256);
    L.ffn_xs_offset = end;
    end = align_up(end + static_cast<size_t>(T) * static_cast<size_t>(H / 32), 256);
  }
  L.ffn_plan_offset = end;
  L.ffn_bytes = L.ffn_plan_offset + align_up(256 + static_cast<size_t>(L.tile_bound) * sizeof(RowTile), 256);
  L.total = L.offsets_bytes > L.ffn_bytes ? L.offsets_bytes : L.ffn_bytes;
  *out = L;
  return MOE_OK;
}

moe_status check_route(const void* logits, int64_t T, int32_t E, int32_t k, const void* ids,
                       const void* weights) {
  moe_status s = check_sizes(T, E, k);
  if (s != MOE_OK || T == 0) return s;
  if (!logits || !ids || !weights) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(weights, 4)) return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

moe_status check_bitmatrix(const void* ids, int64_t T, int32_t E, int32_t k, const void* bm) {
  moe_status s = check_sizes(T, E, k);
  if (s != MOE_OK || T == 0) return s;
  if (!ids || !bm) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(ids, 4) || !aligned(bm, 4)) return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

moe_status check_offsets(const void* bm, const void* ids, int64_t T, int32_t E, int32_t k,
                         const void* counts, const void* offsets, const void* gather,
                         const void* scatter, const void* ws, size_t ws_bytes) {
  moe_status s = check_sizes(T, E, k);
  if (s != MOE_OK) return s;
  if (!counts || !offsets) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(counts, 4) || !aligned(offsets, 4)) return MOE_ERR_MISALIGNED;
  if (T == 0) return MOE_OK;
  if (!bm || !ids || !gather || !scatter || !ws) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(bm, 4) || !aligned(ids, 4) || !aligned(gather, 4) || !aligned(scatter, 4) ||
      !aligned(ws, 16))
    return MOE_ERR_MISALIGNED;
  WsLayout L;
  s = workspace_layout(T, E, k, 0, 0, &L);
  if (s != MOE_OK) return s;
  if (ws_bytes < L.offsets_bytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return MOE_OK;
}

moe_status check_ffn(const void* x, int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                     const void* w1, const void* w1s, const void* w2, const void* w2s,
                     const void* counts, const void* offsets, const void* gather,
                     const void* y_sorted, const void* ws, size_t ws_bytes) {
  moe_status s = check_sizes(T, E, k);
  if (s != MOE_OK) return s;
  s = check_dims(H, I);
  if (s != MOE_OK || T == 0) return s;
  if (!activations_fit(T, k, H, I)) return MOE_ERR_UNSUPPORTED;
  if (!x || !w1 || !w1s || !w2 || !w2s || !counts || !offsets || !gather || !y_sorted || !ws)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w1s, 16) || !aligned(w2, 16) ||
      !aligned(w2s, 16) || !aligned(y_sorted, 16) || !aligned(ws, 16) || !aligned(counts, 4) ||
      !aligned(offsets, 4) || !aligned(gather, 4))
    return MOE_ERR_MISALIGNED;
  WsLayout L;
  s = workspace_layout(T, E, k, H, I, &L);
  if (s != MOE_OK) return s;
  if (ws_bytes < L.ffn_bytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return MOE_OK;
}

moe_status check_combine(const void* y_sorted, const void* w, const void* scatter, int64_t T,
                         int32_t H, int32_t k, const void* y) {
  if (T < 0 || k < 1 || H <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (k > kMaxK || H % 8 != 0 || T > INT32_MAX / k) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y_sorted || !w || !scatter || !y) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(y_sorted, 16) || !aligned(y, 16) || !aligned(w, 4) || !aligned(scatter, 4))
    return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

}  // namespace moe
