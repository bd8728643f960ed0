// Tiling constants shared by the host launch code and the kernels.
#pragma once
#include <cstddef>
#include <cstdint>

namespace moe {

constexpr int kMaxE = 1024;           // experts per layer
constexpr int kMaxK = 8;              // experts per token
constexpr int kWave = 64;             // CDNA wavefront width
constexpr int kMaxDim = 65536;        // largest H or I
constexpr int64_t kMaxActivationBytes = 3758096384LL;   // 3.5 GiB: 32-bit buffer offsets

// moe_expert_offsets: tokens per workgroup (8 wavefronts of 64 tokens)
constexpr int kOffsBlockTokens = 512;

// grouped FFN: the smallest row tile of the MFMA paths (16, 32, 80 or 128 rows;
// the decode GEMV path cuts 1-row tiles), and the K chunk per step
constexpr int kFfnMinTileRows = 16;
constexpr int kFfnGemvTileRows = 1;
constexpr int kFfnKChunk = 128;
// streaming path: LDS for the staged E8M0 scales of a workgroup (4 wavefronts x
// 64 rows x K/32 bytes); above this the scales are read from memory
constexpr size_t kStreamMaxScaleLds = 64 * 1024;
// streaming path: row tiles whose activation rows (all of K) fit beside the
// staged scales within this much LDS per workgroup (three per CU: 16-row tiles
// with four fragments per wavefront) keep them in LDS
constexpr size_t kStreamMaxLds = 53 * 1024;
// the same with 32-row tiles (two workgroups per CU)
constexpr size_t kStreamMaxLds2 = 80 * 1024;
// 16-row tiles with two weight fragments per wavefront (four workgroups per CU)
constexpr size_t kStreamMaxLds4 = 40 * 1024;

// Upper bound on the row tiles of n_slots rows over E experts cut into tiles of
// R = tile_rows rows: an expert with c rows has ceil(c / R) <= (c + R - 1) / R
// tiles, and at most min(n_slots, E) experts have rows, so the tiles number at
// most (n_slots + (R - 1) min(n_slots, E)) / R.
inline int64_t ffn_tile_bound(int64_t n_slots, int E, int tile_rows) {
  const int64_t touched = n_slots < E ? n_slots : E;
  return (n_slots + (tile_rows - 1) * touched) / tile_rows;
}

// The decode GEMV kernels (ffn_gemv.hip) take K = H (W1) and K = I (W2) of 2048 or
// 4096: one or two 1 KB slices per weight row.
inline bool ffn_gemv_dims(int H, int I) {
  return (H == 2048 || H == 4096) && (I == 2048 || I == 4096);
}

// Rows per FFN row tile for T tokens, E experts, k experts per token.  A token
// picks an expert at most once, so no expert has more than T rows.  Fewer rows
// than experts (T k < E, decode and verify steps: most touched experts hold one
// row) with K of 2048 or 4096: 1-row tiles on the GEMV kernels.  Up to 8 rows
// per expert on average: 16-row streaming tiles (decode: the tiles' rows fit in
// LDS for all of K); up to 24: 32-row streaming tiles (measured on the 512-token
// burst, 12 rows per expert: 671 us per layer against 715 with 16-row tiles,
// whose experts past 16 rows read their weights twice); up to 95: 80-row tiles of
// the LDS-tiled kernel (HBM-bound: each expert's weights read about once; at 48
// rows per expert on average the largest experts stay within one tile); from 96
// on, 128-row tiles of the 128 x 512 tiled kernel (the products bound the batch).
inline int ffn_tile_rows(int64_t T, int E, int k, int H, int I) {
  if (T * k < E && ffn_gemv_dims(H, I)) return kFfnGemvTileRows;
  const int64_t avg_rows = T * k / E;
  if (T <= 16 || avg_rows <= 8) return 16;
  if (avg_rows <= 24) return 32;
  return avg_rows < 96 ? 80 : 128;
}

// The tiled kernels (80- and 128-row tiles) run the block-scaled FP8 x FP4 MFMAs
// on two-part FP8 activations; the streaming kernels run bf16 MFMAs.
inline bool ffn_tiled(int64_t T, int E, int k, int H, int I) {
  return ffn_tile_rows(T, E, k, H, I) >= 80;
}

struct RowTile {
  int32_t expert;
  int32_t p_begin;
  int32_t p_end;
  int32_t multi;   // 1 when the expert's rows span more than one tile
};

}  // namespace moe
