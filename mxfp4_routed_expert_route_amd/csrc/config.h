// Tiling constants shared by the host launch code and the kernels.
#pragma once
#include <cstdint>

namespace moe {

constexpr int kMaxE = 1024;           // experts per layer
constexpr int kMaxK = 8;              // experts per token
constexpr int kWave = 64;             // CDNA wavefront width

// moe_expert_offsets: tokens per workgroup (16 wavefronts of 64 tokens)
constexpr int kOffsBlockTokens = 1024;

// grouped FFN: rows per row tile (4 MFMA subtiles of 16 rows), K chunk per step
constexpr int kFfnTileRows = 64;
constexpr int kFfnKChunk = 128;
constexpr int kFfnW1ColsPerBlock = 64;   // gate columns per workgroup (plus the matching up columns)
constexpr int kFfnW2ColsPerBlock = 128;  // output columns per workgroup

struct RowTile {
  int32_t expert;
  int32_t p_begin;
  int32_t p_end;
  int32_t pad;
};

}  // namespace moe
