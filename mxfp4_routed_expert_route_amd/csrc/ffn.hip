// Grouped expert FFN over MXFP4 weights: W1 (gate|up) with the clamped SwiGLU
// epilogue, then W2.
//
// Weight format (txtmix.com article, §1 and §3; OCP MX v1.0): E2M1 codes, two per
// byte (element 2i low nibble), one E8M0 scale per 32 elements along K.  The
// clamp (txtmix.com article, §9): gate capped at +limit, up clamped to
// [-limit, +limit], both before the SwiGLU product.
//
// Work decomposition.  A plan kernel cuts each expert's rows [offsets[e],
// offsets[e+1]) into row tiles (16, 32 or 64 rows, chosen from T and the mean
// rows per expert); only experts with rows get tiles.  A wavefront always owns
// 64 weight rows of one tile's expert -- for W1 32 gate rows and the 32 matching
// up rows, so each SwiGLU pair meets in one lane; for W2 64 output rows -- as four
// 16-column MFMA fragments.  Few rows per expert (decode shapes): the streaming
// kernel, one independent wavefront per (tile, 64 weight rows), bound by HBM.
// Many rows: the tiled kernel, four wavefronts sharing an LDS activation tile.
//
// Inner step (K chunk of 128): every lane loads 16 bytes (32 codes, exactly one
// scale block) of one weight row straight from HBM, so a weight row is read in
// 64-byte runs.  The codes are dequantised in registers with the gfx950 scaled
// FP4->BF16 convert (scale passed as an fp32 whose exponent field is the E8M0
// byte; 0xFF maps to a NaN scale) and fed to v_mfma_f32_16x16x32_bf16 as the B
// operand; activations are the A operand.  Within one MFMA the K order of the 32
// products does not matter as long as A and B agree, so lane group g (lanes
// 16g..16g+15) takes K = chunk + 32g + 8s .. +7 for sub-step s on both operands.
// fp32 accumulation throughout.
#include "config.h"
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- plan

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ counts,
                                                    const int32_t* __restrict__ offsets, int E,
                                                    int tile_rows, int64_t n_slots, int64_t tile_bound,
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
  const int nt = (c + tile_rows - 1) / tile_rows;
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
    rt.p_begin = begin + i * tile_rows;
    rt.p_end = (i + 1) * tile_rows < c ? begin + (i + 1) * tile_rows : begin + c;
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

// ---------------------------------------------------------------- streaming GEMM (few rows)
//
// For row tiles of at most 16*MSUB rows (decode-shaped batches, where each
// expert has a handful of rows and the weights are read once): one wavefront
// owns a row tile and 64 weight rows (W1: 32 gate rows and the 32 matching up
// rows; W2: 64 output rows) and needs no barrier, so many wavefronts stay
// resident per CU.  Per K chunk of 128 each lane loads 16 bytes from each of its
// four weight rows (one scale block per row).
//
// Memory pipeline.  Vector-memory loads retire in issue order, and a wait is a
// count of loads still allowed in flight, so the order of issue decides what a
// wait drains.  Per chunk c the loop issues the activations of chunk c+1, then
// the weights of chunk c+3, then computes chunk c: the wait for c's activations
// leaves the weights of c+2 and c+3 in flight.  Every load in the loop is
// unconditional (rows past the tile read zeros through a bounded buffer
// resource; prefetches past the end re-read the last chunk), which keeps those
// wait counts exact.  The E8M0 scales of the wavefront's 64 rows are staged in
// LDS once, transposed so that one 16-byte LDS read per chunk gives a lane the
// scale of each of its four rows; they never enter the vector-memory queue.
// kDeep selects that pipeline (K a multiple of 512); otherwise a one-chunk
// prefetch with scales read from memory.
template <bool kW1, int MSUB, bool kDeep>
__global__ __launch_bounds__(256) void gemm_stream_kernel(
    const uint16_t* __restrict__ act, uint32_t act_bytes, const int32_t* __restrict__ gather,
    int k_top, int n_slots, const uint8_t* __restrict__ wq, const uint8_t* __restrict__ wsc,
    const RowTile* __restrict__ tiles, const int32_t* __restrict__ n_tiles, int K, int n_rows,
    int half, int waves_per_tile, float limit, int clamp, uint16_t* __restrict__ out,
    int ld_out) {
  extern __shared__ uint32_t scale_lds[];   // kDeep: per wavefront [K/128][16][4] dwords
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int tile_id = gw / waves_per_tile;
  const int cg = gw - tile_id * waves_per_tile;
  if (tile_id >= *n_tiles) return;   // per wavefront: no workgroup barrier in this kernel
  const RowTile rt = tiles[tile_id];
  const int r16 = lane & 15, g = lane >> 4;
  const int n_chunks = K / kFfnKChunk;

  const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(act, act_bytes);
  uint32_t aoff[MSUB];   // byte offset of this lane's activation run in chunk 0
#pragma unroll
  for (int mi = 0; mi < MSUB; ++mi) {
    const int p = rt.p_begin + mi * 16 + r16;
    bool valid = p < rt.p_end;
    uint32_t row = 0;
    if (valid) {
      if (kW1) {
        const int slot = gather[p];   // a slot id outside [0, T*k) feeds zeros, never an address
        valid = static_cast<unsigned>(slot) < static_cast<unsigned>(n_slots);
        row = valid ? static_cast<uint32_t>(slot / k_top) : 0u;
      } else {
        row = static_cast<uint32_t>(p);
      }
    }
    // lane group g starts at element 32g (128-element chunks) or 64g (256-element chunks)
    aoff[mi] = valid ? row * static_cast<uint32_t>(K) * 2u + (kDeep ? 128u : 64u) * g
                     : kRsrcOutOfRange;
  }

  // weight row of fragment f for a lane whose MFMA column is c16
  auto wrow = [&](int f, int c16) {
    return kW1 ? (f >= 2 ? half : 0) + cg * 32 + (f & 1) * 16 + c16   // gate, gate, up, up
               : cg * 64 + f * 16 + c16;
  };
  int nrow[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) nrow[f] = wrow(f, r16);
  const size_t row_q = static_cast<size_t>(K / 2), row_s = static_cast<size_t>(K / 32);
  const size_t e_rows = static_cast<size_t>(rt.expert) * n_rows;
  const uint8_t* bq[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) bq[f] = wq + (e_rows + nrow[f]) * row_q + (kDeep ? 0 : 16 * g);

  uint32_t* my_scales = scale_lds + (threadIdx.x >> 6) * (n_chunks * 64);
  if (kDeep) {
    // lane L stages the scales of row (f = L/16, column L%16).  The 8 scale bytes
    // of a 256-element chunk c2 (2 per lane group) go to the two dwords
    // my_scales[((c2*16 + L%16)*4 + f)*2 + {0,1}]
    const int f = lane >> 4;
    const uint8_t* srow = wsc + (e_rows + wrow(f, r16)) * row_s;
    for (int c = 0; c < n_chunks; c += 4) {   // c counts 128-element chunks
      const uint4 d = *reinterpret_cast<const uint4*>(srow + c * 4);
      const int c2 = c / 2;
      my_scales[(((c2 + 0) * 16 + r16) * 4 + f) * 2 + 0] = d.x;
      my_scales[(((c2 + 0) * 16 + r16) * 4 + f) * 2 + 1] = d.y;
      my_scales[(((c2 + 1) * 16 + r16) * 4 + f) * 2 + 0] = d.z;
      my_scales[(((c2 + 1) * 16 + r16) * 4 + f) * 2 + 1] = d.w;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  const uint8_t* bs[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) bs[f] = wsc + (e_rows + nrow[f]) * row_s + g;

  floatx4 acc[MSUB][4];
#pragma unroll
  for (int mi = 0; mi < MSUB; ++mi)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[mi][f] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto load_w = [&](uint4 (&q)[4], int kc) {
#pragma unroll
    for (int f = 0; f < 4; ++f) q[f] = *reinterpret_cast<const uint4*>(bq[f] + kc * 64);
  };
  auto load_s = [&](uint32_t (&sc)[4], int kc) {   // from memory (shallow pipeline)
#pragma unroll
    for (int f = 0; f < 4; ++f) sc[f] = bs[f][kc * 4];
  };
  auto lds_s = [&](uint32_t (&sc)[4], int kc) {    // from the staged copy
    const uint4 d = *reinterpret_cast<const uint4*>(my_scales + (kc * 16 + r16) * 4);
    const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int f = 0; f < 4; ++f) sc[f] = (dw[f] >> (8 * g)) & 0xFFu;
  };
  auto load_a = [&](bf16x8 (&a)[MSUB][4], int kc) {
#pragma unroll
    for (int mi = 0; mi < MSUB; ++mi)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        a[mi][s] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(arsrc, aoff[mi] + kc * 256 + 16 * s, 0, 0));
  };
  auto compute = [&](const uint4 (&q)[4], const uint32_t (&sc)[4], const bf16x8 (&a)[MSUB][4]) {
    const uint32_t w[4][4] = {{q[0].x, q[0].y, q[0].z, q[0].w},
                              {q[1].x, q[1].y, q[1].z, q[1].w},
                              {q[2].x, q[2].y, q[2].z, q[2].w},
                              {q[3].x, q[3].y, q[3].z, q[3].w}};
    float scl[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) scl[f] = e8m0_as_f32(sc[f]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const bf16x8 b = dequant8(w[f][s], scl[f]);
#pragma unroll
        for (int mi = 0; mi < MSUB; ++mi)
          acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mi][s], b, acc[mi][f], 0, 0, 0);
      }
    }
  };

  if constexpr (kDeep) {
    // 256-element chunks: each lane takes 32 bytes (two scale blocks) of each of its
    // four rows, so a row is visited 128 bytes at a time (about 20% more HBM
    // throughput than 64-byte visits for this many concurrent rows).  Weights:
    // two register stages (the next chunk streams in while this one computes).
    // Activations: loaded for the current chunk, issued before the weight
    // prefetch, so waiting for them leaves the prefetch in flight.
    const int n2 = n_chunks / 2;   // 256-element chunks (even: n_chunks % 4 == 0)
    auto load_w2 = [&](uint4 (&q)[4][2], int c2) {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const uint8_t* src = bq[f] + c2 * 128 + 32 * g;   // lane group g: bytes 32g..32g+31
        q[f][0] = *reinterpret_cast<const uint4*>(src);
        q[f][1] = *reinterpret_cast<const uint4*>(src + 16);
      }
    };
    auto load_a2 = [&](bf16x8 (&a)[MSUB][8], int c2) {
#pragma unroll
      for (int mi = 0; mi < MSUB; ++mi)
#pragma unroll
        for (int t = 0; t < 8; ++t)
          a[mi][t] = __builtin_bit_cast(
              bf16x8, __builtin_amdgcn_raw_buffer_load_b128(arsrc, aoff[mi] + c2 * 512 + 16 * t, 0, 0));
    };
    auto compute2 = [&](const uint4 (&q)[4][2], const bf16x8 (&a)[MSUB][8], int c2) {
      const uint4 d0 = *reinterpret_cast<const uint4*>(my_scales + ((c2 * 16 + r16) * 4) * 2);
      const uint4 d1 = *reinterpret_cast<const uint4*>(my_scales + ((c2 * 16 + r16) * 4) * 2 + 4);
      const uint32_t sd[4][2] = {{d0.x, d0.y}, {d0.z, d0.w}, {d1.x, d1.y}, {d1.z, d1.w}};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float scl[4];
#pragma unroll
        for (int f = 0; f < 4; ++f)   // block 2g + j of the chunk: byte (2g+j)%4 of dword (2g+j)/4
          scl[f] = e8m0_as_f32((sd[f][(2 * g + j) >> 2] >> (8 * ((2 * g + j) & 3))) & 0xFFu);
        const uint32_t w[4][4] = {{q[0][j].x, q[0][j].y, q[0][j].z, q[0][j].w},
                                  {q[1][j].x, q[1][j].y, q[1][j].z, q[1][j].w},
                                  {q[2][j].x, q[2][j].y, q[2][j].z, q[2][j].w},
                                  {q[3][j].x, q[3][j].y, q[3][j].z, q[3][j].w}};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            const bf16x8 b = dequant8(w[f][s], scl[f]);
#pragma unroll
            for (int mi = 0; mi < MSUB; ++mi)
              acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mi][4 * j + s], b, acc[mi][f],
                                                                   0, 0, 0);
          }
        }
      }
    };
    uint4 q0[4][2], q1[4][2];
    load_w2(q0, 0);
    __builtin_amdgcn_sched_barrier(0);
    for (int c2 = 0; c2 < n2; c2 += 2) {
#define MOE_STREAM_STEP(Q_NEXT, KQ, Q_CUR, KC) \
  {                                           \
    bf16x8 a[MSUB][8];                        \
    load_a2(a, KC);                           \
    __builtin_amdgcn_sched_barrier(0);        \
    load_w2(Q_NEXT, KQ);                      \
    __builtin_amdgcn_sched_barrier(0);        \
    compute2(Q_CUR, a, KC);                   \
    __builtin_amdgcn_sched_barrier(0);        \
  }
      MOE_STREAM_STEP(q1, c2 + 1, q0, c2)
      MOE_STREAM_STEP(q0, c2 + 2 < n2 ? c2 + 2 : n2 - 1, q1, c2 + 1)
#undef MOE_STREAM_STEP
    }
  } else {
    uint4 qa[4], qb[4];
    uint32_t sa[4], sb[4];
    load_w(qa, 0);
    load_s(sa, 0);
    int kc = 0;
    for (; kc + 2 <= n_chunks; kc += 2) {
      bf16x8 a0[MSUB][4];
      load_a(a0, kc);
      __builtin_amdgcn_sched_barrier(0);
      load_w(qb, kc + 1);
      load_s(sb, kc + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(qa, sa, a0);
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 a1[MSUB][4];
      load_a(a1, kc + 1);
      __builtin_amdgcn_sched_barrier(0);
      const int kn = kc + 2 < n_chunks ? kc + 2 : kc + 1;   // last pass re-reads a valid chunk
      load_w(qa, kn);
      load_s(sa, kn);
      __builtin_amdgcn_sched_barrier(0);
      compute(qb, sb, a1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kc < n_chunks) {   // odd chunk count: the last chunk is in qa
      bf16x8 a0[MSUB][4];
      load_a(a0, kc);
      compute(qa, sa, a0);
    }
  }

  // D layout of a 16x16 MFMA tile: lane holds column (lane & 15), rows 4*(lane>>4) + i.
  const bool do_clamp = clamp != 0;
#pragma unroll
  for (int mi = 0; mi < MSUB; ++mi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = rt.p_begin + mi * 16 + 4 * g + i;
      if (p >= rt.p_end) continue;
      uint16_t* orow = out + static_cast<int64_t>(p) * ld_out;
      if (kW1) {
        orow[nrow[0]] = f32_to_bf16_bits(swiglu(acc[mi][0][i], acc[mi][2][i], limit, do_clamp));
        orow[nrow[1]] = f32_to_bf16_bits(swiglu(acc[mi][1][i], acc[mi][3][i], limit, do_clamp));
      } else {
#pragma unroll
        for (int f = 0; f < 4; ++f) orow[nrow[f]] = f32_to_bf16_bits(acc[mi][f][i]);
      }
    }
  }
}

// ---------------------------------------------------------------- tiled GEMM (many rows)
//
// For row tiles of 64 or 128 rows (prefill-shaped batches).  A workgroup of four
// wavefronts owns one row tile and 256 weight rows; each wavefront has 64 weight
// rows (same split as the streaming kernel: W1 32 gate + 32 up rows, W2 64 output
// rows) and all 16-row MFMA subtiles of the tile (kMSub = 4 or 8), so each
// dequantised weight fragment feeds kMSub MFMAs.  The activation tile of each K
// chunk (kMSub*16 rows x 128 bf16) is loaded once per workgroup into LDS
// (double-buffered; rows padded by 16 bytes so that the 16 lanes of a read group
// hit distinct banks) and read by all four wavefronts.  Weights go straight to
// registers, issued right after the chunk that frees their registers.  With 64-row
// tiles the E8M0 scales are staged in LDS as in the streaming kernel; with
// 128-row tiles the LDS holds only activations and the scales come with the
// weights.
//
// Per chunk c: issue the activation loads of c+1 (128 rows) or c+2 (64 rows),
// compute c, issue the weights of c+2, store the activations of c+1 to the other
// LDS buffer, barrier.
//
// Workgroup order.  The hardware deals consecutive workgroups to the 8 XCDs in
// turn, and each XCD has its own 4 MB L2.  Launch order (row tile major) gives
// each XCD 2 of the 16 column blocks of every tile: a small weight slice per L2,
// but every tile's activations fetched into all 8 L2s.  Measured alternatives:
// whole tiles per XCD (each L2 then cycles an expert's full 8.9 MB W1) was 40%
// slower; 4 column blocks x half the tiles per XCD is ~1% faster than launch
// order and is what is used.
constexpr int kARowBytes = kFfnKChunk * 2 + 16;   // 256 B of bf16 + 16 B pad
constexpr int kXcds = 8;

template <int kMSub>
constexpr int a_buf_bytes() { return kMSub * 16 * kARowBytes; }

template <bool kW1, int kMSub>
__global__ __launch_bounds__(256, 2) void gemm_tile_kernel(
    const uint16_t* __restrict__ act, uint32_t act_bytes, const int32_t* __restrict__ gather,
    int k_top, int n_slots, const uint8_t* __restrict__ wq, const uint8_t* __restrict__ wsc,
    const RowTile* __restrict__ tiles, const int32_t* __restrict__ n_tiles, int K, int n_rows,
    int half, int waves_per_tile, int blocks_per_tile, float limit, int clamp,
    uint16_t* __restrict__ out, int ld_out) {
  constexpr bool kLdsScales = kMSub == 4;
  constexpr int kRows = kMSub * 16;
  constexpr int kABuf = a_buf_bytes<kMSub>();
  constexpr int kThreadsPerRow = 256 / kRows;          // 4 (64 rows) or 2 (128 rows)
  constexpr int kPieces = kMSub;                       // 16-byte pieces per thread per chunk
  extern __shared__ __attribute__((aligned(16))) unsigned char tile_lds[];

  // work id: with 16 column blocks per tile, XCD x takes column blocks
  // 4(x%4)..4(x%4)+3 of the row tiles of parity x/4 (its weight slice stays in its
  // L2 while each tile's activations go to 4 XCDs, not 8); otherwise launch order
  int work = blockIdx.x;
  if (blocks_per_tile == 16) {
    const int x = blockIdx.x % kXcds, l = blockIdx.x / kXcds;
    work = ((l / 4) * 2 + x / 4) * 16 + (x % 4) * 4 + (l % 4);
  }
  const int tile_id = work / blocks_per_tile;
  const int nb = work - tile_id * blocks_per_tile;
  if (tile_id >= *n_tiles) return;   // uniform over the workgroup
  const RowTile rt = tiles[tile_id];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int n_chunks = K / kFfnKChunk;
  const int rows = rt.p_end - rt.p_begin;
  const int msub = (rows + 15) >> 4;   // subtiles that hold rows

  // column group of this wavefront; a wavefront past the last group repeats the
  // last one (it still stages activations and meets every barrier) and stores nothing
  const int cg_raw = nb * 4 + wave;
  const bool store_cols = cg_raw < waves_per_tile;
  const int cg = store_cols ? cg_raw : waves_per_tile - 1;

  // --- activation staging: thread -> (row ar, part aq) of the chunk
  const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(act, act_bytes);
  const int ar = tid / kThreadsPerRow, aq = tid % kThreadsPerRow;
  uint32_t aoff;
  {
    const int p = rt.p_begin + ar;
    bool valid = p < rt.p_end;
    uint32_t row = 0;
    if (valid) {
      if (kW1) {
        const int slot = gather[p];
        valid = static_cast<unsigned>(slot) < static_cast<unsigned>(n_slots);
        row = valid ? static_cast<uint32_t>(slot / k_top) : 0u;
      } else {
        row = static_cast<uint32_t>(p);
      }
    }
    aoff = valid ? row * static_cast<uint32_t>(K) * 2u + 16u * kPieces * aq : kRsrcOutOfRange;
  }
  unsigned char* a_lds = tile_lds;                       // [2][kRows][kARowBytes]
  const int a_store = ar * kARowBytes + aq * 16 * kPieces;
  auto load_a = [&](uint4 (&ra)[kPieces], int kc) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i)
      ra[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            arsrc, aoff + kc * 256 + 16 * i, 0, 0));
  };
  auto store_a = [&](const uint4 (&ra)[kPieces], int buf) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i)
      *reinterpret_cast<uint4*>(a_lds + buf * kABuf + a_store + 16 * i) = ra[i];
  };

  // --- weights: four fragments of 16 rows, this lane's row in each
  auto wrow = [&](int f, int c16) {
    return kW1 ? (f >= 2 ? half : 0) + cg * 32 + (f & 1) * 16 + c16 : cg * 64 + f * 16 + c16;
  };
  int nrow[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) nrow[f] = wrow(f, r16);
  const size_t row_q = static_cast<size_t>(K / 2), row_s = static_cast<size_t>(K / 32);
  const size_t e_rows = static_cast<size_t>(rt.expert) * n_rows;
  const uint8_t* bq[4];
  const uint32_t* bs[4];   // scale dword of (row, chunk): one byte per lane group
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    bq[f] = wq + (e_rows + nrow[f]) * row_q + 16 * g;
    bs[f] = reinterpret_cast<const uint32_t*>(wsc + (e_rows + nrow[f]) * row_s);
  }
  auto load_w = [&](uint4 (&q)[4], uint32_t (&sd)[4], int kc) {
#pragma unroll
    for (int f = 0; f < 4; ++f) q[f] = *reinterpret_cast<const uint4*>(bq[f] + kc * 64);
    if constexpr (!kLdsScales) {
#pragma unroll
      for (int f = 0; f < 4; ++f) sd[f] = bs[f][kc];
    }
  };

  // --- 64-row tiles: scales of the wavefront's 64 rows, staged as [chunk][16][4] dwords
  uint32_t* my_scales =
      reinterpret_cast<uint32_t*>(tile_lds + 2 * kABuf) + wave * (n_chunks * 64);
  if constexpr (kLdsScales) {
    const int f = lane >> 4;
    const uint8_t* srow = wsc + (e_rows + wrow(f, r16)) * row_s;
    int c = 0;
    for (; c + 4 <= n_chunks; c += 4) {
      const uint4 d = *reinterpret_cast<const uint4*>(srow + c * 4);
      my_scales[((c + 0) * 16 + r16) * 4 + f] = d.x;
      my_scales[((c + 1) * 16 + r16) * 4 + f] = d.y;
      my_scales[((c + 2) * 16 + r16) * 4 + f] = d.z;
      my_scales[((c + 3) * 16 + r16) * 4 + f] = d.w;
    }
    for (; c < n_chunks; ++c)
      my_scales[(c * 16 + r16) * 4 + f] = *reinterpret_cast<const uint32_t*>(srow + c * 4);
  }

  floatx4 acc[kMSub][4];
#pragma unroll
  for (int mi = 0; mi < kMSub; ++mi)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[mi][f] = floatx4{0.f, 0.f, 0.f, 0.f};

  // one chunk: activations from LDS buffer `buf`, weights in q, scale dwords in sd
  auto compute = [&](const uint4 (&q)[4], const uint32_t (&sd)[4], int kc, int buf) {
    uint32_t dw[4];
    if constexpr (kLdsScales) {
      const uint4 d = *reinterpret_cast<const uint4*>(my_scales + (kc * 16 + r16) * 4);
      dw[0] = d.x; dw[1] = d.y; dw[2] = d.z; dw[3] = d.w;
    } else {
#pragma unroll
      for (int f = 0; f < 4; ++f) dw[f] = sd[f];
    }
    float scl[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) scl[f] = e8m0_as_f32((dw[f] >> (8 * g)) & 0xFFu);
    const uint32_t w[4][4] = {{q[0].x, q[0].y, q[0].z, q[0].w},
                              {q[1].x, q[1].y, q[1].z, q[1].w},
                              {q[2].x, q[2].y, q[2].z, q[2].w},
                              {q[3].x, q[3].y, q[3].z, q[3].w}};
    const unsigned char* abase = a_lds + buf * kABuf + r16 * kARowBytes + 64 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 b[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) b[f] = dequant8(w[f][s], scl[f]);
      // every subtile, also those past the tile's rows (they hold zeros): a branch
      // here would cut the MFMA stream into blocks that each wait on one LDS read
#pragma unroll
      for (int mi = 0; mi < kMSub; ++mi) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(abase + mi * 16 * kARowBytes + 16 * s);
#pragma unroll
        for (int f = 0; f < 4; ++f)
          acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[f], acc[mi][f], 0, 0, 0);
      }
    }
  };

  const int last = n_chunks - 1;
  uint4 q0[4], q1[4];
  uint32_t s0[4], s1[4];
  int kc = 0;
  if constexpr (kMSub == 4) {
    // activations two chunks ahead in registers (ra0/ra1), one chunk ahead in LDS
    uint4 ra0[kPieces], ra1[kPieces];
    load_a(ra0, 0);
    load_w(q0, s0, 0);
    load_w(q1, s1, last >= 1 ? 1 : 0);
    load_a(ra1, last >= 1 ? 1 : 0);
    store_a(ra0, 0);
    __syncthreads();
    for (; kc + 2 <= n_chunks; kc += 2) {
      load_a(ra0, kc + 2 <= last ? kc + 2 : last);
      compute(q0, s0, kc, 0);
      load_w(q0, s0, kc + 2 <= last ? kc + 2 : last);
      store_a(ra1, 1);
      __syncthreads();
      load_a(ra1, kc + 3 <= last ? kc + 3 : last);
      compute(q1, s1, kc + 1, 1);
      load_w(q1, s1, kc + 3 <= last ? kc + 3 : last);
      store_a(ra0, 0);
      __syncthreads();
    }
  } else {
    // activations one chunk ahead (registers ra, then LDS)
    uint4 ra[kPieces];
    load_a(ra, 0);
    load_w(q0, s0, 0);
    load_w(q1, s1, last >= 1 ? 1 : 0);
    store_a(ra, 0);
    __syncthreads();
    for (; kc + 2 <= n_chunks; kc += 2) {
      load_a(ra, kc + 1);
      compute(q0, s0, kc, 0);
      load_w(q0, s0, kc + 2 <= last ? kc + 2 : last);
      store_a(ra, 1);
      __syncthreads();
      load_a(ra, kc + 2 <= last ? kc + 2 : last);
      compute(q1, s1, kc + 1, 1);
      load_w(q1, s1, kc + 3 <= last ? kc + 3 : last);
      store_a(ra, 0);
      __syncthreads();
    }
  }
  if (kc < n_chunks) compute(q0, s0, kc, 0);   // odd chunk count: last chunk in buffer 0 / q0

  if (!store_cols) return;
  const bool do_clamp = clamp != 0;
#pragma unroll
  for (int mi = 0; mi < kMSub; ++mi) {
    if (mi >= msub) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = rt.p_begin + mi * 16 + 4 * g + i;
      if (p >= rt.p_end) continue;
      uint16_t* orow = out + static_cast<int64_t>(p) * ld_out;
      if (kW1) {
        orow[nrow[0]] = f32_to_bf16_bits(swiglu(acc[mi][0][i], acc[mi][2][i], limit, do_clamp));
        orow[nrow[1]] = f32_to_bf16_bits(swiglu(acc[mi][1][i], acc[mi][3][i], limit, do_clamp));
      } else {
#pragma unroll
        for (int f = 0; f < 4; ++f) orow[nrow[f]] = f32_to_bf16_bits(acc[mi][f][i]);
      }
    }
  }
}

template <bool kW1, int kMSub>
hipError_t launch_tile(int64_t tile_bound, hipStream_t stream, const uint16_t* act,
                       uint32_t act_bytes, const int32_t* gather, int k_top, int n_slots,
                       const uint8_t* wq, const uint8_t* wsc, const RowTile* tiles,
                       const int32_t* n_tiles, int K, int n_rows, int half, int wpt, float limit,
                       int clamp, uint16_t* out, int ld_out) {
  const int bpt = (wpt + 3) / 4;
  size_t lds = 2 * static_cast<size_t>(a_buf_bytes<kMSub>());
  if (kMSub == 4) lds += static_cast<size_t>(4) * (K / kFfnKChunk) * 64 * sizeof(uint32_t);
  // the column-block/XCD split covers row tiles in pairs: round up to whole pairs
  const int64_t blocks = bpt == 16 ? (tile_bound + 1) / 2 * 2 * bpt : tile_bound * bpt;
  gemm_tile_kernel<kW1, kMSub><<<static_cast<unsigned>(blocks), 256, lds, stream>>>(
      act, act_bytes, gather, k_top, n_slots, wq, wsc, tiles, n_tiles, K, n_rows, half, wpt, bpt,
      limit, clamp, out, ld_out);
  return hipGetLastError();
}

// Launch one streaming GEMM; picks the deep pipeline when K allows it.
template <bool kW1, int MSUB>
hipError_t launch_stream(unsigned grid, hipStream_t stream, const uint16_t* act, uint32_t act_bytes,
                         const int32_t* gather, int k_top, int n_slots, const uint8_t* wq,
                         const uint8_t* wsc, const RowTile* tiles, const int32_t* n_tiles, int K,
                         int n_rows, int half, int wpt, float limit, int clamp, uint16_t* out,
                         int ld_out) {
  const int n_chunks = K / kFfnKChunk;
  const size_t lds = static_cast<size_t>(4) * n_chunks * 64 * sizeof(uint32_t);
  if (n_chunks % 4 == 0 && lds <= kStreamMaxScaleLds)
    gemm_stream_kernel<kW1, MSUB, true><<<grid, 256, lds, stream>>>(
        act, act_bytes, gather, k_top, n_slots, wq, wsc, tiles, n_tiles, K, n_rows, half, wpt,
        limit, clamp, out, ld_out);
  else
    gemm_stream_kernel<kW1, MSUB, false><<<grid, 256, 0, stream>>>(
        act, act_bytes, gather, k_top, n_slots, wq, wsc, tiles, n_tiles, K, n_rows, half, wpt,
        limit, clamp, out, ld_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn(const uint16_t* x, int64_t T, int H, int I, int E, int k,
                      const uint8_t* w1, const uint8_t* w1s, const uint8_t* w2,
                      const uint8_t* w2s, const int32_t* counts, const int32_t* offsets,
                      const int32_t* gather, float limit, uint16_t* y_sorted, void* ws,
                      size_t h_offset, size_t plan_offset, int64_t /*tile_bound_min_rows*/,
                      hipStream_t stream, hipEvent_t const* events) {
  const int64_t n_slots = T * k;
  uint16_t* h = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + h_offset);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + plan_offset);
  RowTile* tiles = reinterpret_cast<RowTile*>(static_cast<char*>(ws) + plan_offset + 256);
  const bool clamp = limit > 0.f && limit <= 3.402823466e38f;   // finite and positive
  const int clamp_i = clamp ? 1 : 0;
  const int slots_i = static_cast<int>(n_slots);
  const uint32_t x_bytes = static_cast<uint32_t>(T * H * 2);         // < 2^32 - 2^20 (host check)
  const uint32_t h_bytes = static_cast<uint32_t>(n_slots * I * 2);

  // Path: a token picks an expert at most once, so no expert has more than T rows.
  // Few rows per expert -> weight streaming with 16- or 32-row tiles; else 64-row tiles.
  const int64_t avg_rows = n_slots / E;
  int tile_rows;
  if (T <= 16)
    tile_rows = 16;
  else if (avg_rows <= 24)
    tile_rows = 32;
  else
    tile_rows = 64;
  const int64_t tile_bound = ffn_tile_bound(n_slots, E, tile_rows);

  plan_kernel<<<1, 1024, 0, stream>>>(counts, offsets, E, tile_rows, n_slots, tile_bound, n_tiles,
                                      tiles);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (events) {
    err = hipEventRecord(events[0], stream);
    if (err != hipSuccess) return err;
  }

  if (tile_rows <= 32) {
    const int wpt1 = I / 32, wpt2 = H / 64;
    const unsigned g1 = static_cast<unsigned>((tile_bound * wpt1 + 3) / 4);
    const unsigned g2 = static_cast<unsigned>((tile_bound * wpt2 + 3) / 4);
    const RowTile* t = tiles;
    err = tile_rows == 16
              ? launch_stream<true, 1>(g1, stream, x, x_bytes, gather, k, slots_i, w1, w1s, t,
                                       n_tiles, H, 2 * I, I, wpt1, limit,
                                       clamp_i, h, I)
              : launch_stream<true, 2>(g1, stream, x, x_bytes, gather, k, slots_i, w1, w1s, t,
                                       n_tiles, H, 2 * I, I, wpt1, limit,
                                       clamp_i, h, I);
    if (err != hipSuccess) return err;
    if (events) {
      err = hipEventRecord(events[1], stream);
      if (err != hipSuccess) return err;
    }
    err = tile_rows == 16
              ? launch_stream<false, 1>(g2, stream, h, h_bytes, nullptr, k, slots_i, w2, w2s, t,
                                        n_tiles, I, H, 0, wpt2, limit, 0,
                                        y_sorted, H)
              : launch_stream<false, 2>(g2, stream, h, h_bytes, nullptr, k, slots_i, w2, w2s, t,
                                        n_tiles, I, H, 0, wpt2, limit, 0,
                                        y_sorted, H);
  } else {
    const int wpt1 = I / 32, wpt2 = H / 64;
    err = launch_tile<true, 4>(tile_bound, stream, x, x_bytes, gather, k, slots_i, w1, w1s, tiles,
                               n_tiles, H, 2 * I, I, wpt1, limit, clamp_i, h, I);
    if (err != hipSuccess) return err;
    if (events) {
      err = hipEventRecord(events[1], stream);
      if (err != hipSuccess) return err;
    }
    err = launch_tile<false, 4>(tile_bound, stream, h, h_bytes, nullptr, k, slots_i, w2, w2s,
                                tiles, n_tiles, I, H, 0, wpt2, limit, 0, y_sorted, H);
  }
  if (err != hipSuccess || !events) return err;
  return hipEventRecord(events[2], stream);
}

}  // namespace moe
