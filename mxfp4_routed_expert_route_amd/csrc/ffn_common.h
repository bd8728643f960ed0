// Shared pieces of the grouped MXFP4 FFN kernels (streaming and tiled).
//
// Weight format (txtmix.com article, §1 and §3; OCP MX v1.0): E2M1 codes, two per
// byte (element 2i low nibble), one E8M0 scale per 32 elements along K.  The
// clamp (txtmix.com article, §9): gate capped at +limit, up clamped to
// [-limit, +limit], both before the SwiGLU product.
//
// Every GEMM wavefront owns weight rows of one row tile's expert as 16-column MFMA
// fragments -- four (64 rows) in the tiled kernel and the 32-row streaming tiles,
// two (32 rows) in the 16-row streaming tiles; for W1 half of them gate rows and
// half the matching up rows, so each SwiGLU pair meets in one lane.  Codes are
// dequantised in registers with the gfx950 scaled FP4->BF16 convert (scale passed
// as an fp32 whose exponent field is the E8M0 byte; 0xFF maps to a NaN scale) and
// fed to v_mfma_f32_16x16x32_bf16 as the B operand; activations are the A
// operand.  Within one MFMA the K order of the 32 products does not matter as long
// as A and B agree, which frees the lane-to-K assignment for memory efficiency.
// fp32 accumulation throughout.
#pragma once
#include "config.h"
#include "device.h"

namespace moe {

// E8M0 byte -> fp32 whose exponent field holds it; 0xFF becomes a NaN.
__device__ __forceinline__ float e8m0_as_f32(uint32_t s) {
  return __uint_as_float((s << 23) | (((s + 1u) & 0x100u) << 14));
}

// 8 E2M1 codes (one dword, element 2i in the low nibble of byte i) -> 8 bf16.
__device__ __forceinline__ bf16x8 dequant8(uint32_t q, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 3);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ float swiglu(float g, float u, float limit, bool clamp) {
  if (clamp) {
    g = g > limit ? limit : g;                       // NaN passes through
    u = u > limit ? limit : (u < -limit ? -limit : u);
  }
  return g / (1.0f + __expf(-g)) * u;
}

// Weight rows per streaming wavefront: 16-row tiles (decode) give each wavefront
// two 16-row fragments (W1: 16 gate + 16 up rows; W2: 32 output rows), 32-row
// tiles four.  Measured with a read-only probe of the W1 decode pattern (46
// experts x 4096 rows of 2 KB, 12 wavefronts per CU): 5,888 wavefronts of 32 rows
// read the 377 MB in 66.7 us against 73.2 us for 2,944 wavefronts of 64 rows.
constexpr int kStreamFrags16 = 2;
inline int stream_frags(int msub) { return msub == 1 ? kStreamFrags16 : 4; }

// A K chunk is 128 elements: 64 bytes of codes and 4 scale bytes per weight row.
// Launchers (arguments are checked by the caller; they return the launch status).
// kW1 selects W1 (x rows gathered through `gather`, SwiGLU epilogue into h) or
// W2 (h rows in order, plain epilogue into y_sorted).
hipError_t launch_stream(bool w1, int msub, unsigned grid, hipStream_t stream, const uint16_t* act,
                         uint32_t act_bytes, const int32_t* gather, int k_top, int n_slots,
                         const uint8_t* wq, const uint8_t* wsc, const RowTile* tiles,
                         const int32_t* n_tiles, int K, int n_rows, int half, int wpt, float limit,
                         int clamp, uint16_t* out, int ld_out);
// tile_rows: 80 (80 x 256 workgroups) or 128 (128 x 512 workgroups)
hipError_t launch_tile(bool w1, int tile_rows, int64_t tile_bound, hipStream_t stream,
                       const uint16_t* act, uint32_t act_bytes, const int32_t* gather, int k_top,
                       int n_slots, const uint8_t* wq, const uint8_t* wsc, const RowTile* tiles,
                       const int32_t* n_tiles, int K, int n_rows, int half, float limit, int clamp,
                       uint16_t* out, int ld_out, bool whole_tiles);

}  // namespace moe
