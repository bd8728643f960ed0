// Shared pieces of the grouped MXFP4 FFN kernels (streaming and tiled).
//
// Weight format (txtmix.com article, §1 and §3; OCP MX v1.0): E2M1 codes, two per
// byte (element 2i low nibble), one E8M0 scale per 32 elements along K.  The
// clamp (txtmix.com article, §9): gate capped at +limit, up clamped to
// [-limit, +limit], both before the SwiGLU product.
//
// Every GEMM wavefront owns weight rows of one row tile's expert as 16-row MFMA
// fragments -- four (64 rows) in the tiled kernels and the 32-row streaming tiles,
// two (32 rows) in the 16-row streaming tiles; for W1 half of them gate rows and
// half the matching up rows, so each SwiGLU pair meets in one lane.  Streaming
// kernels (decode shapes) dequantise the codes in registers with the gfx950 scaled
// FP4->BF16 convert (scale passed as an fp32 whose exponent field is the E8M0 byte;
// 0xFF maps to a NaN scale) and feed them to v_mfma_f32_16x16x32_bf16 as the B
// operand, activations being the A operand; within one MFMA the K order of the 32
// products does not matter as long as A and B agree, which frees the lane-to-K
// assignment for memory efficiency.  Tiled kernels (prefill shapes) feed codes and
// scales as stored to the block-scaled FP4 x FP8 MFMA (ffn_tile.hip) with the
// activations in the two-part FP8 form below.  fp32 accumulation throughout.
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

// ---- two-part FP8 activations (the input form of the block-scaled MFMA path)
//
// An activation row of K values is stored as 2K bytes plus K/32 scale bytes.
// Per 32-element block along K (natural order, block b = elements 32b..32b+31) an
// E8M0 scale s puts the block's largest magnitude m in [128, 256): s = 127 +
// floor(log2 m) - 7.  Each element v (scaled: v' = v * 2^(127-s)) is held as
// hi = E4M3(v') and lo = E4M3(v' - hi), both rounded to nearest even (OCP E4M3,
// 3 mantissa bits).  A bf16 value has 8 significant bits and each part holds 4,
// so hi + lo equals v' exactly whenever the remainder v' - hi is a multiple of
// the smallest E4M3 step 2^-9, i.e. for |v'| >= 2^-2 (|v| >= m * 2^-9); below
// that the error is at most 2^-10, i.e. 2^-17 of the block maximum.
// Byte layout of a row: per 128-element chunk c, 128 bytes of hi then 128 bytes
// of lo, each in the lane order of v_mfma_scale_f32_16x16x128_f8f6f4's FP8
// operand (measured on gfx950): lane group g (lanes 16g .. 16g+15) takes chunk
// elements 16g .. 16g+15 and 64+16g .. 64+16g+15 as its 32 bytes, so element kk
// of the chunk sits at byte a8_pos(kk).  The scales of a row are K/32 bytes in
// natural block order (one dword per chunk).
__host__ __device__ constexpr int a8_pos(int kk) {
  return kk < 64 ? 32 * (kk / 16) + kk % 16 : 32 * ((kk - 64) / 16) + 16 + (kk - 64) % 16;
}

// E8M0 scale byte for a block whose largest magnitude has fp32 bits `absbits`
// (sign cleared): 127 + floor(log2 m) - 7, or 0 for tiny blocks; 127 for a block
// holding an infinity or NaN (those stay non-finite through the conversion).
__device__ __forceinline__ uint32_t a8_scale_byte(uint32_t absbits) {
  const uint32_t e = absbits >> 23;   // biased exponent of m
  if (e == 255u) return 127u;
  return e >= 7u ? e - 7u : 0u;
}

// 2^(127 - s) as fp32 (exact for every s the scale rule produces: 0 .. 247).
__device__ __forceinline__ float a8_inv_scale(uint32_t s) {
  return __uint_as_float((254u - s) << 23);
}

// 8 scaled values -> 8 hi bytes and 8 lo bytes (element i in byte i % 4 of word i / 4).
__device__ __forceinline__ void a8_split8(const float (&v)[8], uint2& hi, uint2& lo) {
  uint32_t h[2], l[2];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    int pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * w + 0], v[4 * w + 1], 0, false);
    pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * w + 2], v[4 * w + 3], pk, true);
    h[w] = static_cast<uint32_t>(pk);
    const auto b01 = __builtin_amdgcn_cvt_pk_f32_fp8(pk, false);
    const auto b23 = __builtin_amdgcn_cvt_pk_f32_fp8(pk, true);
    int lk = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * w + 0] - b01[0], v[4 * w + 1] - b01[1], 0, false);
    lk = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * w + 2] - b23[0], v[4 * w + 3] - b23[1], lk, true);
    l[w] = static_cast<uint32_t>(lk);
  }
  hi = make_uint2(h[0], h[1]);
  lo = make_uint2(l[0], l[1]);
}

// SiLU(min(g, L)) * clamp(u, -L, L) in fp32.  SiLU's quotient is taken as g times
// the hardware reciprocal of 1 + exp(-g) (v_rcp_f32, ~1 ulp), not an IEEE division:
// the full division's fix-up sequence made the 128-row W1 epilogue ~1.6% of the
// hot experts' W1 time slower.  For g -> -inf the reciprocal of +inf is 0 and the
// result -0, the same limit.
__device__ __forceinline__ float swiglu(float g, float u, float limit, bool clamp) {
  if (clamp) {
    g = g > limit ? limit : g;                       // NaN passes through
    u = u > limit ? limit : (u < -limit ? -limit : u);
  }
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Weight rows per streaming wavefront: 16-row tiles (decode) give each wavefront
// two 16-row fragments (W1: 16 gate + 16 up rows; W2: 32 output rows), 32-row
// tiles four.  Measured with a read-only probe of the W1 decode pattern (46
// experts x 4096 rows of 2 KB, 12 wavefronts per CU): 5,888 wavefronts of 32 rows
// read the 377 MB in 66.7 us against 73.2 us for 2,944 wavefronts of 64 rows.
constexpr int kStreamFrags16 = 2;
// 32-row streaming tiles: LDS per wavefront for the weight transit (two 16-row
// fragments x 128 bytes), and the weight loads' cache-policy operand
constexpr size_t kStreamTransitBytes = 4096;
constexpr int kStreamWeightAux = 2;   // non-temporal
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
// Tiled GEMM arguments.  act: two-part FP8 rows (2K bytes each; W1: x's, gathered
// through `gather`; W2: h's, in order) with E8M0 block scales asc ([rows][K/32]).
// out: W1 writes h as two-part FP8 ([n_slots][2 ld_out] bytes) and its scales to
// out_sc ([n_slots][ld_out/32]); W2 writes bf16 y_sorted ([n_slots][ld_out]).
struct TileArgs {
  int64_t tile_bound;
  const uint8_t* act;
  uint32_t act_bytes;
  const uint8_t* asc;
  uint32_t asc_bytes;
  const int32_t* gather;
  int k_top, n_slots;
  const uint8_t* wq;
  const uint8_t* wsc;
  const RowTile* tiles;
  const int32_t* n_tiles;
  int K, n_rows, half;
  float limit;
  int clamp;
  void* out;
  uint8_t* out_sc;
  int ld_out;
  bool whole_tiles;
};
// tile_rows: 80 (80 x 256 workgroups) or 128 (128 x 512 workgroups)
hipError_t launch_tile(bool w1, int tile_rows, const TileArgs& args, hipStream_t stream);
// Decode GEMV (1-row tiles, K = 2048 or 4096, ffn_gemv_dims): act as for
// launch_stream (bf16 rows; W1 gathered through `gather`), out bf16 [n_slots][ld_out].
hipError_t launch_gemv(bool w1, int64_t tile_bound, hipStream_t stream, const uint16_t* act,
                       const int32_t* gather, int k_top, int n_slots, const uint8_t* wq,
                       const uint8_t* wsc, const RowTile* tiles, const int32_t* n_tiles, int K,
                       int n_rows, int half, float limit, int clamp, uint16_t* out, int ld_out);

// W2 of the decode GEMV path with the weighted combine folded in (ffn_gemv.hip):
// y_sorted as launch_gemv(false, ...) writes it and y as the combine kernel does,
// one wavefront per (token, 8 output columns).
hipError_t launch_gemv_w2_combine(int64_t T, int k_top, int E, int n_slots, hipStream_t stream,
                                  const uint16_t* h, const int32_t* ids, const float* topw,
                                  const int32_t* scatter, const uint8_t* wq, const uint8_t* wsc,
                                  int K, int n_rows, uint16_t* y_sorted, uint16_t* y);

}  // namespace moe
