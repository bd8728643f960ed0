// Streaming grouped GEMM for decode-shaped batches (row tiles of <= 32 rows).
#include "ffn_common.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- streaming GEMM (few rows)
//
// For row tiles of at most 16*MSUB rows (decode and small batches, where each
// expert has few rows and the weights are read once): one wavefront owns a row
// tile and 16*kFrag weight rows (W1: 8*kFrag gate rows and the matching up rows;
// W2: 16*kFrag output rows), so many wavefronts stay resident per CU.  16-row
// tiles use two fragments per wavefront: finer work units balance the CUs
// better (5,888 wavefronts instead of 2,944 for the verify step's W1).
//
// Memory pipeline (kDeep, K a multiple of 512).  K advances in chunks of 256
// elements: each lane takes 32 bytes (two scale blocks) of each of its kFrag
// rows, so a weight row is visited 128 bytes at a time -- measured on MI355X,
// 128-byte visits of this many concurrent rows stream about 20% faster than
// 64-byte ones.  With 32-row tiles the loads themselves read 8 rows x 128
// contiguous bytes each (non-temporal) and the chunk reaches the MFMA layout
// through 4 KB of LDS per wavefront (the burst step: W1 406 -> 385 us, W2 225 ->
// 217-221 us, bit-identical).  Two register stages of weights: the next chunk
// streams in while this one computes.  The E8M0 scales of the wavefront's 16*kFrag rows are staged
// in LDS once, laid out so that one (two fragments) or two (four) 16-byte LDS
// reads per chunk give a lane the scales of its rows; they never enter the
// vector-memory queue.  Activations take one of
// three routes (the host enables the first two only when the four wavefronts of
// a workgroup share one tile):
//   * rows in LDS: a tile whose rows fit beside the scales is staged once, for
//     all of K, behind one workgroup barrier (decode: one or two rows);
//   * ring: larger tiles are staged chunk by chunk, once per workgroup, through
//     a two-slot LDS ring with one barrier per chunk;
//   * per wavefront: each wavefront loads its chunk's activations itself, issued
//     before the weight prefetch, so waiting for them leaves the prefetch in
//     flight (vector-memory loads retire in issue order).
// Every load in the loop is unconditional (rows past the tile read zeros through
// a bounded buffer resource; the last prefetch re-reads the last chunk), which
// keeps the compiler's wait counts exact.
// Otherwise (small K): 128-element chunks, one-chunk prefetch, scales from memory.
// Four wavefronts per SIMD (16 per CU) with 16-row tiles (two fragments per
// wavefront, 113 VGPRs, workgroups within 40 KB of LDS), two with 32-row tiles.
template <bool kW1, int MSUB, bool kDeep, int kFrag>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MSUB == 1 ? 3 : 2)))
void gemm_stream_kernel(
    const uint16_t* __restrict__ act, uint32_t act_bytes, const int32_t* __restrict__ gather,
    int k_top, int n_slots, const uint8_t* __restrict__ wq, const uint8_t* __restrict__ wsc,
    const RowTile* __restrict__ tiles, const int32_t* __restrict__ n_tiles, int K, int n_rows,
    int half, int waves_per_tile, float limit, int clamp, uint16_t* __restrict__ out,
    int ld_out, int a_lds_rows, int a_ring, int wt_off) {
  // kDeep: per wavefront [K/128][16][4] dwords of scales; after the four
  // wavefronts' scales, either a_lds_rows activation rows of K bf16 and a
  // 512-byte zero block, or the ring (two slots of 16*MSUB rows of 512 bytes)
  extern __shared__ uint32_t scale_lds[];
  const int lane = threadIdx.x & 63;
  // 32-row tiles: each XCD takes whole tiles (tile x, x+8, ... for XCD x, the
  // hardware dealing consecutive workgroups to the 8 XCDs in turn), so the tile's
  // activation chunks, staged by each of its workgroups, are fetched into one L2
  int blk = blockIdx.x;
  if constexpr (MSUB == 2) {
    const int bpt = waves_per_tile >> 2;
    if ((waves_per_tile & 3) == 0 && gridDim.x % (8 * bpt) == 0) {   // uniform
      const int x = blockIdx.x % 8, l = blockIdx.x / 8;
      blk = ((l / bpt) * 8 + x) * bpt + l % bpt;
    }
  }
  const int gw = blk * 4 + (threadIdx.x >> 6);
  const int tile_id = gw / waves_per_tile;
  const int cg = gw - tile_id * waves_per_tile;
  // A workgroup's four wavefronts share one tile exactly when waves_per_tile is a
  // multiple of 4; only then may the kernel take the paths with workgroup barriers
  // (activation rows in LDS, the ring), and only then is this return uniform over
  // the workgroup.  Otherwise each wavefront returns on its own, and no barrier
  // follows.
  const bool shared_tile = (waves_per_tile & 3) == 0;
  if (tile_id >= *n_tiles) return;
  const RowTile rt = tiles[tile_id];
  const int r16 = lane & 15, g = lane >> 4;
  const int n_chunks = K / kFfnKChunk;
  static_assert(kFrag == 2 || kFrag == 4, "two or four 16-row weight fragments per wavefront");
  constexpr int kGate = kFrag / 2;   // W1: gate fragments (the up fragments follow)

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

  // Row tiles of at most a_lds_rows rows (decode: mostly one or two): the four
  // wavefronts share the tile (the host enables this only when the wavefronts per
  // tile are a multiple of 4), so the workgroup stages its activation rows for all
  // of K in LDS once and the K loop reads them there.  This drops the activation
  // loads -- as many 16-byte loads per chunk as the weights, mostly of rows past
  // the tile -- from the vector-memory queue.
  const int nvalid = rt.p_end - rt.p_begin;
  const bool small_a = kDeep && MSUB == 1 && shared_tile && a_lds_rows > 0 && nvalid <= a_lds_rows;
  const bool ring = kDeep && shared_tile && a_ring != 0 && !small_a;   // uniform (one tile)
  unsigned char* a_lds = reinterpret_cast<unsigned char*>(scale_lds + 4 * n_chunks * 16 * kFrag);
  const int a_row_bytes = K * 2;
  if (small_a) {   // uniform over the workgroup (one tile)
    // the tile's rows, then the zero block at row a_lds_rows
    const int row_pieces = nvalid * (a_row_bytes / 16);
    for (int i = threadIdx.x; i < row_pieces + 32; i += 256) {
      const bool is_row = i < row_pieces;
      const int byte = is_row ? i * 16 : a_lds_rows * a_row_bytes + (i - row_pieces) * 16;
      const int r = byte / a_row_bytes;
      uint32_t off = kRsrcOutOfRange;
      if (is_row) {
        const int p = rt.p_begin + r;
        if (kW1) {
          const int slot = gather[p];
          if (static_cast<unsigned>(slot) < static_cast<unsigned>(n_slots))
            off = static_cast<uint32_t>(slot / k_top) * static_cast<uint32_t>(a_row_bytes) +
                  static_cast<uint32_t>(byte - r * a_row_bytes);
        } else {
          off = static_cast<uint32_t>(p) * static_cast<uint32_t>(a_row_bytes) +
                static_cast<uint32_t>(byte - r * a_row_bytes);
        }
      }
      *reinterpret_cast<uint4*>(a_lds + byte) =
          __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(arsrc, off, 0, 0));
    }
    __syncthreads();
  }
  // this lane's activation run in LDS: its row, or the zero block (which does
  // not advance with the chunk)
  const unsigned char* a_mine = r16 < nvalid ? a_lds + r16 * a_row_bytes + 128 * g
                                             : a_lds + a_lds_rows * a_row_bytes + 128 * g;
  const int a_step = r16 < nvalid ? 512 : 0;

  // weight row of fragment f for a lane whose MFMA column is c16
  auto wrow = [&](int f, int c16) {   // W1: gate fragments, then the matching up fragments
    return kW1 ? (f >= kGate ? half : 0) + cg * (16 * kGate) + (f % kGate) * 16 + c16
               : cg * (16 * kFrag) + f * 16 + c16;
  };
  int nrow[kFrag];
#pragma unroll
  for (int f = 0; f < kFrag; ++f) nrow[f] = wrow(f, r16);
  const size_t row_q = static_cast<size_t>(K / 2), row_s = static_cast<size_t>(K / 32);
  const size_t e_rows = static_cast<size_t>(rt.expert) * n_rows;
  const uint8_t* bq[kFrag];
#pragma unroll
  for (int f = 0; f < kFrag; ++f) bq[f] = wq + (e_rows + nrow[f]) * row_q + (kDeep ? 0 : 16 * g);

  uint32_t* my_scales = scale_lds + (threadIdx.x >> 6) * (n_chunks * 16 * kFrag);
  if (kDeep && (lane >> 4) < kFrag) {
    // lane L stages the scales of row (f = L/16, column L%16); with two fragments
    // per wavefront lanes 32..63 have no row.  The 8 scale bytes of a 256-element
    // chunk c2 (2 per lane group) go to the two dwords
    // my_scales[(((c2*kFrag/2 + f/2)*16 + L%16)*2 + f%2)*2 + {0,1}]: each 16-byte
    // LDS read of the K loop (fragments 2h, 2h+1 of one row) then sits at quad
    // L%16 of its 256-byte block, a bank pattern without read conflicts (see the
    // tiled kernel's activation layout)
    const int f = lane >> 4;
    const uint8_t* srow = wsc + (e_rows + wrow(f, r16)) * row_s;
    auto put = [&](int c, const uint4& d) {   // c counts 128-element chunks
      const int c2 = c / 2;
      uint32_t* s0 = my_scales + ((((c2 + 0) * (kFrag / 2) + f / 2) * 16 + r16) * 2 + f % 2) * 2;
      uint32_t* s1 = my_scales + ((((c2 + 1) * (kFrag / 2) + f / 2) * 16 + r16) * 2 + f % 2) * 2;
      s0[0] = d.x;
      s0[1] = d.y;
      s1[0] = d.z;
      s1[1] = d.w;
    };
    // four 16-byte loads in flight before their stores (a load-then-store loop
    // waits one memory latency per iteration, with every wavefront of the grid
    // in this prologue at once; eight would exceed the register budget)
    int c = 0;
    for (; c + 16 <= n_chunks; c += 16) {
      uint4 d[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) d[j] = *reinterpret_cast<const uint4*>(srow + (c + 4 * j) * 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) put(c + 4 * j, d[j]);
    }
    for (; c < n_chunks; c += 4) put(c, *reinterpret_cast<const uint4*>(srow + c * 4));
  }
  if (kDeep) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  const uint8_t* bs[kFrag];
#pragma unroll
  for (int f = 0; f < kFrag; ++f) bs[f] = wsc + (e_rows + nrow[f]) * row_s + g;

  floatx4 acc[MSUB][kFrag];
#pragma unroll
  for (int mi = 0; mi < MSUB; ++mi)
#pragma unroll
    for (int f = 0; f < kFrag; ++f) acc[mi][f] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto load_w = [&](uint4 (&q)[kFrag], int kc) {
#pragma unroll
    for (int f = 0; f < kFrag; ++f) q[f] = *reinterpret_cast<const uint4*>(bq[f] + kc * 64);
  };
  auto load_s = [&](uint32_t (&sc)[kFrag], int kc) {   // from memory (shallow pipeline)
#pragma unroll
    for (int f = 0; f < kFrag; ++f) sc[f] = bs[f][kc * 4];
  };
  auto load_a = [&](bf16x8 (&a)[MSUB][4], int kc) {
#pragma unroll
    for (int mi = 0; mi < MSUB; ++mi)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        a[mi][s] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(arsrc, aoff[mi] + kc * 256 + 16 * s, 0, 0));
  };
  auto compute = [&](const uint4 (&q)[kFrag], const uint32_t (&sc)[kFrag],
                     const bf16x8 (&a)[MSUB][4]) {
    uint32_t w[kFrag][4];
#pragma unroll
    for (int f = 0; f < kFrag; ++f) {
      w[f][0] = q[f].x; w[f][1] = q[f].y; w[f][2] = q[f].z; w[f][3] = q[f].w;
    }
    float scl[kFrag];
#pragma unroll
    for (int f = 0; f < kFrag; ++f) scl[f] = e8m0_as_f32(sc[f]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int f = 0; f < kFrag; ++f) {
        const bf16x8 b = dequant8(w[f][s], scl[f]);
#pragma unroll
        for (int mi = 0; mi < MSUB; ++mi)
          acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mi][s], b, acc[mi][f], 0, 0, 0);
      }
    }
  };

  if constexpr (kDeep) {
    // 256-element chunks, two weight register stages; `run` is the K loop for the
    // LDS-held rows and the per-wavefront activation loads, `run_ring` for the ring.
    const int n2 = n_chunks / 2;   // 256-element chunks (even: n_chunks % 4 == 0)
    // 32-row tiles: each weight load instruction reads 8 rows x 128 contiguous bytes
    // (lane l: row 8h + l/8 of fragment f, bytes 16 (l%8) .. +15 of the chunk), and
    // the wavefront moves the chunk through LDS into the MFMA layout (transit).
    // Measured on MI355X with a read-only probe of W2's bytes (1 GiB, 64 rows per
    // wavefront, eight loads in flight): this pattern reads 6.9 TB/s, the MFMA
    // layout's own pattern (16 rows x 4 runs of 16 bytes per instruction) 5.6.
    constexpr bool kR8 = MSUB == 2;
    // (the expert made visibly wavefront-uniform: a scalar resource, no per-load loop)
    const size_t e_rows_u =
        static_cast<size_t>(__builtin_amdgcn_readfirstlane(rt.expert)) * n_rows;
    const __amdgpu_buffer_rsrc_t wrs =
        make_rsrc(wq + e_rows_u * row_q, static_cast<uint32_t>(n_rows * row_q));
    uint32_t r8off[kFrag][2];
#pragma unroll
    for (int f = 0; f < kFrag; ++f)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        r8off[f][h] = static_cast<uint32_t>(wrow(f, 8 * h + (lane >> 3))) *
                          static_cast<uint32_t>(row_q) + 16u * (lane & 7);
    auto load_w2 = [&](uint4 (&q)[kFrag][2], int c2) {
      if constexpr (kR8) {
#pragma unroll
        for (int f = 0; f < kFrag; ++f)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            q[f][h] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs, r8off[f][h], c2 * 128,
                                                             kStreamWeightAux));
      } else {
#pragma unroll
        for (int f = 0; f < kFrag; ++f) {
          const uint8_t* src = bq[f] + c2 * 128 + 32 * g;   // lane group g: bytes 32g..32g+31
          q[f][0] = *reinterpret_cast<const uint4*>(src);
          q[f][1] = *reinterpret_cast<const uint4*>(src + 16);
        }
      }
    };
    // Transit of one chunk, two fragments at a time through the wavefront's 4 KB of
    // LDS: row r's 16-byte block b (of 8) of fragment pair member m sits in 256-byte
    // line 8m + r/2 at quad 8 (r%2) + (b ^ r/2), so the stores (8 lanes: one row's 8
    // blocks) and the loads (16 lanes: rows 0..15, one block each) each touch
    // distinct quads.  LDS operations of a wavefront execute in order, so the loads
    // see the stores and the next stores follow the loads; the empty asm statements
    // keep the compiler from moving them across each other.
    unsigned char* wt = reinterpret_cast<unsigned char*>(scale_lds) + wt_off +
                        (threadIdx.x >> 6) * kStreamTransitBytes;
    uint32_t wt_st[2], wt_ld[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 8 * h + (lane >> 3), b = lane & 7;
      wt_st[h] = static_cast<uint32_t>((r >> 1) * 256 + ((r & 1) * 8 + (b ^ (r >> 1))) * 16);
      const int bj = 2 * g + h;   // the MFMA layout: row r16, blocks 2g and 2g + 1
      wt_ld[h] = static_cast<uint32_t>((r16 >> 1) * 256 + ((r16 & 1) * 8 + (bj ^ (r16 >> 1))) * 16);
    }
    auto transit = [&](uint4 (&q)[kFrag][2]) __attribute__((always_inline)) {
      if constexpr (kR8) {
#pragma unroll
        for (int fp = 0; fp < kFrag; fp += 2) {
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int h = 0; h < 2; ++h)
              *reinterpret_cast<uint4*>(wt + m * 2048 + wt_st[h]) = q[fp + m][h];
          asm volatile("" ::: "memory");
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              q[fp + m][j] = *reinterpret_cast<const uint4*>(wt + m * 2048 + wt_ld[j]);
          asm volatile("" ::: "memory");
        }
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
    auto load_a2_lds = [&](bf16x8 (&a)[MSUB][8], int c2) {   // small_a (MSUB == 1)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        a[0][t] = *reinterpret_cast<const bf16x8*>(a_mine + c2 * a_step + 16 * t);
    };
    auto compute2 = [&](const uint4 (&q)[kFrag][2], const bf16x8 (&a)[MSUB][8], int c2) {
      // one 16-byte read per two fragments (2 dwords each) of the lane's row
      const uint4 d0 =
          *reinterpret_cast<const uint4*>(my_scales + ((c2 * (kFrag / 2) + 0) * 16 + r16) * 4);
      uint4 d1 = d0;
      if constexpr (kFrag == 4)
        d1 = *reinterpret_cast<const uint4*>(my_scales + ((c2 * (kFrag / 2) + 1) * 16 + r16) * 4);
      const uint32_t sd[4][2] = {{d0.x, d0.y}, {d0.z, d0.w}, {d1.x, d1.y}, {d1.z, d1.w}};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float scl[kFrag];
#pragma unroll
        for (int f = 0; f < kFrag; ++f)   // block 2g + j of the chunk: byte (2g+j)%4 of dword (2g+j)/4
          scl[f] = e8m0_as_f32((sd[f][(2 * g + j) >> 2] >> (8 * ((2 * g + j) & 3))) & 0xFFu);
        uint32_t w[kFrag][4];
#pragma unroll
        for (int f = 0; f < kFrag; ++f) {
          w[f][0] = q[f][j].x; w[f][1] = q[f][j].y; w[f][2] = q[f][j].z; w[f][3] = q[f][j].w;
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
          for (int f = 0; f < kFrag; ++f) {
            const bf16x8 b = dequant8(w[f][s], scl[f]);
#pragma unroll
            for (int mi = 0; mi < MSUB; ++mi)
              acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mi][4 * j + s], b, acc[mi][f],
                                                                   0, 0, 0);
          }
        }
      }
    };
    auto run = [&](auto&& load_a) __attribute__((always_inline)) {
      uint4 q0[kFrag][2], q1[kFrag][2];
      load_w2(q0, 0);
      __builtin_amdgcn_sched_barrier(0);
      for (int c2 = 0; c2 < n2; c2 += 2) {
#define MOE_STREAM_STEP(Q_NEXT, KQ, Q_CUR, KC) \
  {                                           \
    bf16x8 a[MSUB][8];                        \
    load_a(a, KC);                            \
    __builtin_amdgcn_sched_barrier(0);        \
    load_w2(Q_NEXT, KQ);                      \
    __builtin_amdgcn_sched_barrier(0);        \
    transit(Q_CUR);                           \
    compute2(Q_CUR, a, KC);                   \
    __builtin_amdgcn_sched_barrier(0);        \
  }
        MOE_STREAM_STEP(q1, c2 + 1, q0, c2)
        MOE_STREAM_STEP(q0, c2 + 2 < n2 ? c2 + 2 : n2 - 1, q1, c2 + 1)
#undef MOE_STREAM_STEP
      }
    };
    // Larger tiles with a_ring: the workgroup stages each 256-element activation
    // chunk once (16*MSUB rows x 512 bytes; 16/MSUB threads per row, each load
    // instruction reading 256/MSUB contiguous bytes of every row) into a two-slot
    // LDS ring, one barrier per chunk; the chunk after next is in flight in
    // registers meanwhile.  A slot is piece-major: 16-byte piece q (0..31) of row r
    // at (q * 16*MSUB + (r ^ (q & 7))) * 16, so the reads of a K step (piece 8g + t
    // of each lane's row) sit at bank quad r ^ t, a function of the row alone, and
    // eight consecutive lanes storing one row's pieces hit distinct quads (the
    // tiled kernel's activation layout states the measured rule).
    auto run_ring = [&]() __attribute__((always_inline)) {
      constexpr int kRR = 16 * MSUB, kSlot = 32 * kRR * 16;
      constexpr int kTpr = 16 / MSUB, kPc = 2 * MSUB;   // threads per row, pieces per thread
      const int sr = threadIdx.x / kTpr, sp = threadIdx.x % kTpr;
      uint32_t srow = kRsrcOutOfRange;
      {
        const int p = rt.p_begin + sr;
        if (p < rt.p_end) {
          if (kW1) {
            const int slot = gather[p];
            if (static_cast<unsigned>(slot) < static_cast<unsigned>(n_slots))
              srow = static_cast<uint32_t>(slot / k_top) * static_cast<uint32_t>(K) * 2u;
          } else {
            srow = static_cast<uint32_t>(p) * static_cast<uint32_t>(K) * 2u;
          }
        }
      }
      auto stage_load = [&](uint4 (&r)[kPc], int c2) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kPc; ++i)
          r[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                               arsrc, srow + 16 * (sp + kTpr * i), c2 * 512, 0));
      };
      auto stage_store = [&](const uint4 (&r)[kPc], int slot) __attribute__((always_inline)) {
        // piece sp + kTpr * i of row sr; kTpr is a multiple of 8, so the row XOR is sp & 7
        unsigned char* d = a_lds + slot * kSlot + (sp * kRR + (sr ^ (sp & 7))) * 16;
#pragma unroll
        for (int i = 0; i < kPc; ++i) *reinterpret_cast<uint4*>(d + kTpr * i * kRR * 16) = r[i];
      };
      auto read_a = [&](bf16x8 (&a)[MSUB][8], int c2) __attribute__((always_inline)) {
        const unsigned char* base = a_lds + (c2 & 1) * kSlot;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int off = ((8 * g + t) * kRR + (r16 ^ t)) * 16;   // piece 8g + t
#pragma unroll
          for (int mi = 0; mi < MSUB; ++mi)
            a[mi][t] = *reinterpret_cast<const bf16x8*>(base + off + mi * 256);
        }
      };
      uint4 sa[kPc];
      uint4 q0[kFrag][2], q1[kFrag][2];
      stage_load(sa, 0);
      __builtin_amdgcn_sched_barrier(0);
      load_w2(q0, 0);
      __builtin_amdgcn_sched_barrier(0);
      stage_store(sa, 0);
      __builtin_amdgcn_sched_barrier(0);
      stage_load(sa, n2 > 1 ? 1 : 0);
      __syncthreads();
      for (int c2 = 0; c2 < n2; c2 += 2) {
#define MOE_RING_STEP(Q_NEXT, KQ, Q_CUR, KC)                  \
  {                                                           \
    load_w2(Q_NEXT, KQ);                                      \
    __builtin_amdgcn_sched_barrier(0);                        \
    transit(Q_CUR);                                           \
    bf16x8 a[MSUB][8];                                        \
    read_a(a, KC);                                            \
    compute2(Q_CUR, a, KC);                                   \
    __builtin_amdgcn_sched_barrier(0);                        \
    stage_store(sa, (KC + 1) & 1);                            \
    __builtin_amdgcn_sched_barrier(0);                        \
    stage_load(sa, KC + 2 < n2 ? KC + 2 : n2 - 1);            \
    __syncthreads();                                          \
  }
        MOE_RING_STEP(q1, c2 + 1, q0, c2)
        MOE_RING_STEP(q0, c2 + 2 < n2 ? c2 + 2 : n2 - 1, q1, c2 + 1)
#undef MOE_RING_STEP
      }
    };
    if (small_a)
      run(load_a2_lds);
    else if (ring)
      run_ring();
    else
      run(load_a2);
  } else {
    uint4 qa[kFrag], qb[kFrag];
    uint32_t sa[kFrag], sb[kFrag];
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
  // Non-temporal stores: h and y_sorted are read once, by the next launch (burst
  // layer 609 -> 598 us in a rotated one-process A/B, bit-identical).
  const bool do_clamp = clamp != 0;
#pragma unroll
  for (int mi = 0; mi < MSUB; ++mi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = rt.p_begin + mi * 16 + 4 * g + i;
      if (p >= rt.p_end) continue;
      uint16_t* orow = out + static_cast<int64_t>(p) * ld_out;
      if (kW1) {
#pragma unroll
        for (int f = 0; f < kGate; ++f)
          __builtin_nontemporal_store(
              f32_to_bf16_bits(swiglu(acc[mi][f][i], acc[mi][f + kGate][i], limit, do_clamp)),
              orow + nrow[f]);
      } else {
#pragma unroll
        for (int f = 0; f < kFrag; ++f)
          __builtin_nontemporal_store(f32_to_bf16_bits(acc[mi][f][i]), orow + nrow[f]);
      }
    }
  }
}

// Launch one streaming GEMM; picks the deep pipeline when K allows it.
template <bool kW1, int MSUB, int kFrag>
hipError_t launch_stream_t(unsigned grid, hipStream_t stream, const uint16_t* act, uint32_t act_bytes,
                         const int32_t* gather, int k_top, int n_slots, const uint8_t* wq,
                         const uint8_t* wsc, const RowTile* tiles, const int32_t* n_tiles, int K,
                         int n_rows, int half, int wpt, float limit, int clamp, uint16_t* out,
                         int ld_out) {
  const int n_chunks = K / kFfnKChunk;
  const size_t lds = static_cast<size_t>(4) * n_chunks * 16 * kFrag * sizeof(uint32_t);
  // 16-row tiles with two fragments per wavefront fit four workgroups per CU
  const size_t max_lds = MSUB == 1 ? (kFrag == 2 ? kStreamMaxLds4 : kStreamMaxLds) : kStreamMaxLds2;
  // activation rows in LDS for row tiles that fit: one tile per workgroup, and
  // room for four workgroups per CU with 16-row tiles (W1 at H = 4096: 2 rows; W2
  // at I = 2048: 7), two with 32-row tiles
  int a_rows = 0;
  if (MSUB == 1 && wpt % 4 == 0 && lds + 512 < max_lds) {
    const size_t fit = (max_lds - lds - 512) / (static_cast<size_t>(K) * 2);
    a_rows = static_cast<int>(fit < 16 ? fit : 16);
  }
  size_t a_bytes = a_rows > 0 ? static_cast<size_t>(a_rows) * K * 2 + 512 : 0;
  // the ring: two chunks of 16*MSUB padded rows, within the workgroup's share of
  // LDS
  // 32-row tiles: the weight transit, 4 KB per wavefront, after the activations
  const size_t wt_bytes = MSUB == 2 ? 4 * kStreamTransitBytes : 0;
  const size_t ring_bytes = 2 * 16 * MSUB * 512;
  const size_t budget = max_lds - wt_bytes;
  const int a_ring = wpt % 4 == 0 && lds + ring_bytes <= budget ? 1 : 0;
  if (a_ring && ring_bytes > a_bytes) a_bytes = ring_bytes;
  if (n_chunks % 4 == 0 && lds <= kStreamMaxScaleLds)
    gemm_stream_kernel<kW1, MSUB, true, kFrag><<<grid, 256, lds + a_bytes + wt_bytes, stream>>>(
        act, act_bytes, gather, k_top, n_slots, wq, wsc, tiles, n_tiles, K, n_rows, half, wpt,
        limit, clamp, out, ld_out, a_rows, a_ring, static_cast<int>(lds + a_bytes));
  else
    gemm_stream_kernel<kW1, MSUB, false, kFrag><<<grid, 256, 0, stream>>>(
        act, act_bytes, gather, k_top, n_slots, wq, wsc, tiles, n_tiles, K, n_rows, half, wpt,
        limit, clamp, out, ld_out, 0, 0, 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_stream(bool w1, int msub, unsigned grid, hipStream_t stream, const uint16_t* act,
                         uint32_t act_bytes, const int32_t* gather, int k_top, int n_slots,
                         const uint8_t* wq, const uint8_t* wsc, const RowTile* tiles,
                         const int32_t* n_tiles, int K, int n_rows, int half, int wpt, float limit,
                         int clamp, uint16_t* out, int ld_out) {
  if (w1)
    return msub == 1
               ? launch_stream_t<true, 1, kStreamFrags16>(grid, stream, act, act_bytes, gather,
                                                          k_top, n_slots, wq, wsc, tiles, n_tiles,
                                                          K, n_rows, half, wpt, limit, clamp, out,
                                                          ld_out)
               : launch_stream_t<true, 2, 4>(grid, stream, act, act_bytes, gather, k_top, n_slots,
                                             wq, wsc, tiles, n_tiles, K, n_rows, half, wpt, limit,
                                             clamp, out, ld_out);
  return msub == 1
             ? launch_stream_t<false, 1, kStreamFrags16>(grid, stream, act, act_bytes, gather,
                                                         k_top, n_slots, wq, wsc, tiles, n_tiles,
                                                         K, n_rows, half, wpt, limit, clamp, out,
                                                         ld_out)
             : launch_stream_t<false, 2, 4>(grid, stream, act, act_bytes, gather, k_top, n_slots,
                                            wq, wsc, tiles, n_tiles, K, n_rows, half, wpt, limit,
                                            clamp, out, ld_out);
}

}  // namespace moe
