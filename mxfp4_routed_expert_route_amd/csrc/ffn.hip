// Grouped expert FFN over MXFP4 weights: W1 (gate|up) with the clamped SwiGLU
// epilogue, then W2.
//
// Weight format (txtmix.com article, §1 and §3; OCP MX v1.0): E2M1 codes, two per
// byte (element 2i low nibble), one E8M0 scale per 32 elements along K.  The
// clamp (txtmix.com article, §9): gate capped at +limit, up clamped to
// [-limit, +limit], both before the SwiGLU product.
//
// Work decomposition.  A plan kernel cuts each expert's rows [offsets[e],
// offsets[e+1]) into row tiles of up to 64 rows; only experts with rows get
// tiles.  A GEMM workgroup owns one (row tile, column block): 4 wavefronts, each
// with two 16-column weight fragments (W1: 16 gate rows and the 16 matching up
// rows, so the SwiGLU pairs meet in one lane; W2: 32 output rows) and all rows of
// the tile as up to four 16-row MFMA subtiles.
//
// Inner step (K chunk of 128): every lane streams 16 bytes (32 codes, exactly one
// scale block) of one weight row straight from HBM, so a fragment row is read as
// one 64-byte run per chunk.  The codes are dequantised in registers with the
// gfx950 scaled FP4->BF16 convert (scale passed as an fp32 whose exponent field
// is the E8M0 byte; 0xFF maps to a NaN scale) and fed to
// v_mfma_f32_16x16x32_bf16 as the B operand; activations are the A operand.
// Within one MFMA the K order of the 32 products does not matter as long as A
// and B agree, so lane group g (lanes 16g..16g+15) takes K = chunk + 32g + 8s ..
// +7 for sub-step s on both operands.  fp32 accumulation throughout.
#include "config.h"
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- plan

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ counts,
                                                    const int32_t* __restrict__ offsets, int E,
                                                    int64_t n_slots, int64_t tile_bound,
                                                    int32_t* __restrict__ n_tiles,
                                                    RowTile* __restrict__ tiles) {
  __shared__ int wave_tot[16];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  int c = 0, begin = 0;
  if (e < E) {
    c = counts[e];
    begin = offsets[e];
    if (c < 0 || begin < 0 || begin > n_slots) c = 0;
    if (static_cast<int64_t>(begin) + c > n_slots) c = static_cast<int>(n_slots - begin);
  }
  const int nt = (c + kFfnTileRows - 1) / kFfnTileRows;
  int incl = nt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wave_tot[w];
  const int first = base + incl - nt;
  for (int i = 0; i < nt; ++i) {
    const int64_t slot = static_cast<int64_t>(first) + i;
    if (slot >= tile_bound) break;
    RowTile rt;
    rt.expert = e;
    rt.p_begin = begin + i * kFfnTileRows;
    rt.p_end = (i + 1) * kFfnTileRows < c ? begin + (i + 1) * kFfnTileRows : begin + c;
    rt.pad = 0;
    tiles[slot] = rt;
  }
  if (e == blockDim.x - 1) {
    const int64_t total = base + incl;
    *n_tiles = static_cast<int32_t>(total < tile_bound ? total : tile_bound);
  }
}

// ---------------------------------------------------------------- GEMM

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

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ float swiglu(float g, float u, float limit, bool clamp) {
  if (clamp) {
    g = g > limit ? limit : g;                       // NaN passes through
    u = u > limit ? limit : (u < -limit ? -limit : u);
  }
  return g / (1.0f + __expf(-g)) * u;
}

// kW1: act = x [T][K] gathered through gather[p] / k_top; out = h [n_slots][I] with
//      column block of 64 gate columns; B fragments = gate rows and up rows.
// !kW1: act = h [n_slots][K]; out = y_sorted [n_slots][N]; column block of 128.
template <bool kW1>
__global__ __launch_bounds__(256) void gemm_kernel(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ gather, int k_top,
    int n_slots, const uint8_t* __restrict__ wq, const uint8_t* __restrict__ wsc,
    const RowTile* __restrict__ tiles, const int32_t* __restrict__ n_tiles, int K, int n_rows,
    int half, int blocks_per_tile, float limit, int clamp, uint16_t* __restrict__ out,
    int ld_out) {
  const int tile_id = blockIdx.x / blocks_per_tile;
  const int nb = blockIdx.x - tile_id * blocks_per_tile;
  if (tile_id >= *n_tiles) return;
  const RowTile rt = tiles[tile_id];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int rows = rt.p_end - rt.p_begin;
  const int msub = (rows + 15) >> 4;

  // activation rows this lane feeds (A operand row r16 of each subtile)
  const uint16_t* arow[4];
  bool aval[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int p = rt.p_begin + mi * 16 + r16;
    aval[mi] = p < rt.p_end;
    int64_t src = 0;
    if (aval[mi]) {
      if (kW1) {
        const int slot = gather[p];   // a slot id outside [0, T*k) feeds zeros, never an address
        aval[mi] = static_cast<unsigned>(slot) < static_cast<unsigned>(n_slots);
        src = aval[mi] ? slot / k_top : 0;
      } else {
        src = p;
      }
    }
    arow[mi] = act + src * K + 32 * g;
  }

  // weight rows this lane streams (B operand column r16 of each fragment)
  int n0, n1;
  if (kW1) {
    n0 = nb * kFfnW1ColsPerBlock + wave * 16 + r16;   // gate row
    n1 = half + n0;                                   // matching up row
  } else {
    n0 = nb * kFfnW2ColsPerBlock + wave * 32 + r16;
    n1 = n0 + 16;
  }
  const size_t row_q = static_cast<size_t>(K / 2), row_s = static_cast<size_t>(K / 32);
  const size_t e_rows = static_cast<size_t>(rt.expert) * n_rows;
  const uint8_t* bq0 = wq + (e_rows + n0) * row_q + 16 * g;
  const uint8_t* bq1 = wq + (e_rows + n1) * row_q + 16 * g;
  const uint8_t* bs0 = wsc + (e_rows + n0) * row_s + g;
  const uint8_t* bs1 = wsc + (e_rows + n1) * row_s + g;

  floatx4 acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) acc[mi][0] = acc[mi][1] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int n_chunks = K / kFfnKChunk;
  for (int kc = 0; kc < n_chunks; ++kc) {
    const uint4 q0 = *reinterpret_cast<const uint4*>(bq0 + kc * 64);
    const uint4 q1 = *reinterpret_cast<const uint4*>(bq1 + kc * 64);
    const float s0 = e8m0_as_f32(bs0[kc * 4]);
    const float s1 = e8m0_as_f32(bs1[kc * 4]);
    const uint32_t w0[4] = {q0.x, q0.y, q0.z, q0.w};
    const uint32_t w1[4] = {q1.x, q1.y, q1.z, q1.w};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 b0 = dequant8(w0[s], s0);
      const bf16x8 b1 = dequant8(w1[s], s1);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        if (mi < msub) {
          const bf16x8 a = aval[mi] ? load_bf16x8(arow[mi] + kc * kFfnKChunk + 8 * s) : bf16x8{};
          acc[mi][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b0, acc[mi][0], 0, 0, 0);
          acc[mi][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b1, acc[mi][1], 0, 0, 0);
        }
      }
    }
  }

  // D layout of a 16x16 MFMA tile: lane holds column (lane & 15), rows 4*(lane>>4) + i.
  const bool do_clamp = clamp != 0;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    if (mi >= msub) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = rt.p_begin + mi * 16 + 4 * g + i;
      if (p >= rt.p_end) continue;
      uint16_t* orow = out + static_cast<int64_t>(p) * ld_out;
      if (kW1) {
        orow[n0] = f32_to_bf16_bits(swiglu(acc[mi][0][i], acc[mi][1][i], limit, do_clamp));
      } else {
        orow[n0] = f32_to_bf16_bits(acc[mi][0][i]);
        orow[n1] = f32_to_bf16_bits(acc[mi][1][i]);
      }
    }
  }
}

}  // namespace

hipError_t launch_ffn(const uint16_t* x, int64_t T, int H, int I, int E, int k,
                      const uint8_t* w1, const uint8_t* w1s, const uint8_t* w2,
                      const uint8_t* w2s, const int32_t* counts, const int32_t* offsets,
                      const int32_t* gather, float limit, uint16_t* y_sorted, void* ws,
                      size_t h_offset, size_t plan_offset, int64_t tile_bound,
                      hipStream_t stream, hipEvent_t const* events) {
  const int64_t n_slots = T * k;
  uint16_t* h = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + h_offset);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + plan_offset);
  RowTile* tiles = reinterpret_cast<RowTile*>(static_cast<char*>(ws) + plan_offset + 256);
  const bool clamp = limit > 0.f && limit <= 3.402823466e38f;   // finite and positive

  plan_kernel<<<1, 1024, 0, stream>>>(counts, offsets, E, n_slots, tile_bound, n_tiles, tiles);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  if (events) {
    err = hipEventRecord(events[0], stream);
    if (err != hipSuccess) return err;
  }
  const int bpt1 = I / kFfnW1ColsPerBlock;
  gemm_kernel<true><<<dim3(static_cast<unsigned>(tile_bound * bpt1)), dim3(256), 0, stream>>>(
      x, gather, k, static_cast<int>(n_slots), w1, w1s, tiles, n_tiles, H, 2 * I, I, bpt1, limit, clamp ? 1 : 0, h, I);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (events) {
    err = hipEventRecord(events[1], stream);
    if (err != hipSuccess) return err;
  }

  const int bpt2 = H / kFfnW2ColsPerBlock;
  gemm_kernel<false><<<dim3(static_cast<unsigned>(tile_bound * bpt2)), dim3(256), 0, stream>>>(
      h, nullptr, k, static_cast<int>(n_slots), w2, w2s, tiles, n_tiles, I, H, 0, bpt2, limit, 0, y_sorted, H);
  err = hipGetLastError();
  if (err != hipSuccess || !events) return err;
  return hipEventRecord(events[2], stream);
}

}  // namespace moe
