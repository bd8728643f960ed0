// Tiled grouped GEMM for prefill-shaped batches (80- and 128-row tiles).
#include <type_traits>

#include "ffn_common.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- tiled GEMM (many rows)
//
// For row tiles of 80 or 128 rows (prefill-shaped batches).  A workgroup of kWaves
// wavefronts owns one row tile and kWaves x 16 x kFrag weight rows.  A wavefront
// holds kFrag 16-row weight fragments (W1: kFrag/2 gate fragments and the
// matching up fragments, so each SwiGLU pair meets in one lane; W2: kFrag output
// fragments) and all kMSub 16-row MFMA subtiles of the tile, so each weight
// fragment feeds kMSub MFMAs.  The products are gfx950's block-scaled FP4 x FP8
// MFMAs (v_mfma_scale_f32_16x16x128_f8f6f4): the weights' E2M1 codes and E8M0
// scales go in as they are stored -- no dequantisation -- and the activations as
// two-part FP8 (hi + lo with an E8M0 scale per 32 elements, exact for bf16
// inputs; ffn_common.h), one MFMA per part, so the products run at the FP8 rate
// twice, i.e. the bf16 rate, without the dequantisation instructions of a bf16
// MFMA path.  The activation tile of each K chunk (kMSub*16 rows x 128 elements,
// 256 bytes a row) is loaded once per workgroup into LDS (double-buffered, in the
// layout described at kAPieces) and read by all its wavefronts.  W1's weights go
// straight to registers in the operand layout, issued right after the chunk that
// frees their registers, and the E8M0 scales of the wavefronts' weight rows are
// staged in LDS for all of K while they fit beside the activation buffers (K <=
// 4096 for both shapes; staging them took the 128-row kernel's loop off four
// scale loads per chunk, 11% of the skewed layer); beyond that they come with the
// weights.  W2 (on 128-row tiles: those with fewer than eight subtiles) reads its
// weights 8 rows x 128 contiguous bytes per load and moves them into the operand
// layout through a per-wavefront LDS transit, scales with them (see load_pair).
// Each tile runs only the 16-row subtiles that hold rows and stages only their
// activation rows (the K loop and the epilogue are instantiated per subtile count).
//
// Two shapes are used:
//  * 80 x 256 (kMSub 5, four wavefronts, two workgroups per CU) for experts of
//    ~25-95 rows, where the weights are read from HBM about once per expert and
//    the batch is bound by HBM.  80 rather than 64 rows: with uniform routing at
//    48 rows per expert the largest experts reach the high 60s, and each one past
//    the tile size would re-read its 13.4 MB of weights for a few rows -- and
//    its extra workgroups run as a near-empty last round of the grid;
//  * 128 x 512 (kMSub 8, eight wavefronts, one workgroup per CU) for experts with
//    hundreds of rows, where the products bound the batch: per K chunk it moves
//    half the activation and weight bytes per product of the 64 x 256 shape.  Its
//    128 accumulator registers leave no room for the compiler to hoist every LDS
//    read and dequantisation of a chunk; a scheduling barrier between the 32-wide
//    K steps keeps it within 256 VGPRs without spills.
//
// Per chunk c: issue the activation loads of c+1 (128 rows) or c+2 (80 rows),
// compute c, issue the weights of c+2, store the activations of c+1 to the other
// LDS buffer, barrier.
//
// Workgroup order.  The hardware deals consecutive workgroups to the 8 XCDs in
// turn, and each XCD has its own 4 MB L2.  Launch order (row tile major) gives
// each XCD 2 of the 16 column blocks of every tile (256-column blocks of W1): a
// small weight slice per L2, but every tile's activations fetched into all 8 L2s.
// Measured alternatives: whole tiles per XCD (each L2 then cycles an expert's full
// 8.9 MB W1) was 40% slower on an earlier version of this kernel and is neutral on
// the present 128-row kernel (skewed-8191: 2,514-2,532 against 2,524-2,528 us per
// layer); 4 column blocks x half the tiles per XCD is ~1% faster than launch order
// and is what is used there.  With 8 column blocks per
// tile (128 x 512 tiles) the same split gives each XCD 2 column blocks of half
// the tiles: a 1 MB activation tile goes to 4 L2s instead of 8, and the XCD's
// slice of a hot expert (2 x 1.1 MB of W1) stays in its L2 across that expert's
// many row tiles.  With 80-row tiles and at most 64 rows per expert on average
// (prefill batches: most experts are one tile, so there is no slice to share)
// each XCD takes whole tiles instead: all 16 column blocks of a tile read its
// activation chunks from one L2 (prefill-2048 W1 ~566 -> ~549 us).
//
// LDS layout of a staged activation chunk.  A chunk row is 256 bytes, 16 pieces
// of 16 bytes: pieces 0..7 hold the row's 128 hi bytes, 8..15 its lo bytes, in
// the MFMA's FP8 lane order (a8_pos).  Lane group g reads hi pieces 2g, 2g+1 and
// lo pieces 8+2g, 9+2g of its row, so the chunk is stored piece-major -- [q][row]
// -- with bit 2 of the row index flipped in odd pieces: byte offset
// (q * rows + (row ^ 4(q & 1))) * 16.  Measured on gfx950 (a probe of
// ds_read_b128 / ds_write_b128 patterns with the SQ_LDS_BANK_CONFLICT counter), a
// 128-bit read spends no conflict cycles when a lane's bank quad (address / 16
// mod 16) depends only on its MFMA row (lane & 15), and extra cycles whenever it
// also depends on the lane group (272-byte padded rows, quad (row + 4g + s) mod
// 16, cost 4 cycles per read); here a read's quad is row or row ^ 4.  A 128-bit
// write takes 8 lanes at a time over 32 banks.
constexpr int kAPieces = kFfnKChunk * 2 / 16;
constexpr int kXcds = 8;

template <int kMSub>
constexpr int a_buf_bytes() { return kMSub * 16 * kAPieces * 16; }
// LDS a wavefront's weights pass through (kR8): one pair of chunks of its four
// fragments (4 x 16 rows x 128 bytes of codes) and the scale dwords of two pairs
// (4 chunks x 16 rows x 4 fragments)
constexpr int kTileTransitBytes = 4 * 2048 + 4 * 16 * 4 * 4;
// LDS of the staged E8M0 scales (without kR8): per wavefront, one dword per
// (128-element chunk, weight row) of its 64 rows
inline size_t tile_scale_lds_bytes(int K, int waves) {
  return static_cast<size_t>(waves) * (K / kFfnKChunk) * 64 * sizeof(uint32_t);
}
constexpr size_t kTileLdsPerWorkgroup = 80 * 1024;   // two workgroups per CU
constexpr size_t kCuLds = 160 * 1024;                 // one workgroup per CU
// LDS of a workgroup: two activation buffers, the rows' block scales (a dword per
// thread for each buffer, or with tile_ascales all of K for each row), and the
// wavefronts' weight transit areas (r8) and/or staged weight scales (lds_scales)
inline size_t tile_lds_bytes(int msub, int K, int waves, bool r8, bool lds_scales, bool tile_ascales) {
  const size_t rows = static_cast<size_t>(msub) * 16;
  const size_t ascales = tile_ascales ? rows * (K / 128 + 1) * 4 : 2 * static_cast<size_t>(64 * waves) * 4;
  // transit areas and staged weight scales share one region (a tile uses one)
  const size_t transit = r8 ? static_cast<size_t>(waves) * kTileTransitBytes : 0;
  const size_t staged = lds_scales ? tile_scale_lds_bytes(K, waves) : 0;
  const size_t weights = transit > staged ? transit : staged;
  return 2 * rows * kAPieces * 16 + ascales + weights;
}

// Which K loop a tile with NS subtiles runs: the weight transit (kR8) for every
// 80-row tile and for 128-row tiles with at most four subtiles; 128-row tiles with
// eight subtiles keep the operand-layout loads (their 128 accumulators leave no
// registers for a pair in flight beside the transit's operands).
template <bool kR8, int kMSub, int NS>
constexpr bool tile_r8_path() { return kR8 && (kMSub == 5 || NS < kMSub); }

template <bool kW1, int kMSub, int kFrag, int kWaves, bool kR8, bool kLdsScales, bool kTileAScales>
__global__ __launch_bounds__(64 * kWaves, 8 / kWaves) void gemm_tile_kernel(
    const uint8_t* __restrict__ act, uint32_t act_bytes, const uint8_t* __restrict__ asc,
    uint32_t asc_bytes, const int32_t* __restrict__ gather, int k_top, int n_slots,
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ wsc,
    const RowTile* __restrict__ tiles, const int32_t* __restrict__ n_tiles, int K, int n_rows,
    int half, int waves_per_tile, int blocks_per_tile, float limit, int clamp,
    void* __restrict__ out, uint8_t* __restrict__ out_sc, int ld_out, int whole_tiles) {
  // the fragment count is a parameter of the indexing below, but only four
  // fragments per wavefront (64 weight rows) are instantiated and tested
  static_assert(kFrag == 4, "four weight fragments per wavefront");
  constexpr int kRows = kMSub * 16;
  constexpr int kABuf = a_buf_bytes<kMSub>();
  constexpr int kThreads = 64 * kWaves;
  constexpr int kRowStride = kThreads / 16;            // rows apart of a thread's pieces
  constexpr int kPieces = kRows / kRowStride;          // 16-byte pieces per thread per chunk
  static_assert(kPieces * kRowStride == kRows, "activation staging covers each row exactly");
  constexpr int kGate = kFrag / 2;                     // W1: gate fragments per wavefront
  extern __shared__ __attribute__((aligned(16))) unsigned char tile_lds[];

  // work id: with 16 column blocks per tile, XCD x takes column blocks
  // 4(x%4)..4(x%4)+3 of the row tiles of parity x/4 (its weight slice stays in its
  // L2 while each tile's activations go to 4 XCDs, not 8); otherwise launch order
  // (same with 8 column blocks: XCD x takes column blocks 2(x%4), 2(x%4)+1)
  int work = blockIdx.x;
  if (whole_tiles) {   // XCD x takes row tiles x, x+8, ... (grid: whole 8-tile groups)
    const int x = blockIdx.x % kXcds, l = blockIdx.x / kXcds;
    work = ((l / blocks_per_tile) * kXcds + x) * blocks_per_tile + l % blocks_per_tile;
  } else if (blocks_per_tile == 16 || blocks_per_tile == 8) {
    const int x = blockIdx.x % kXcds, l = blockIdx.x / kXcds;
    const int per = blocks_per_tile / 4;   // column blocks per XCD and tile
    work = ((l / per) * 2 + x / 4) * blocks_per_tile + (x % 4) * per + (l % per);
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
  const int cg_raw = nb * kWaves + wave;
  const bool store_cols = cg_raw < waves_per_tile;
  const int cg = store_cols ? cg_raw : waves_per_tile - 1;

  // --- activation staging: a chunk row is 256 bytes (128 hi, 128 lo; see a8_pos).
  // Thread t stages piece aq = 4((t >> 3) & 3) + (t & 3) of rows ar + kRowStride * i,
  // ar = 2(t >> 5) + ((t >> 2) & 1): four consecutive lanes read 64 contiguous
  // bytes of one row, 32 lanes two whole rows; kRowStride rows per piece index i,
  // so any multiple of 16 rows maps onto the workgroup.  (Measured: a mapping
  // whose eight-lane groups take four rows x two pieces, conflict-free for the LDS
  // writes below, but with four different rows per four lanes, made the prefill
  // kernels ~10% slower; this one pays a 2-way LDS write conflict instead.)
  // Thread t < kRows also stages the scale dword (the four E8M0 block scales of the
  // chunk) of tile row t.
  const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(act, act_bytes);
  const __amdgpu_buffer_rsrc_t srsrc = make_rsrc(asc, asc_bytes);
  const int ar = 2 * (tid >> 5) + ((tid >> 2) & 1), aq = 4 * ((tid >> 3) & 3) + (tid & 3);
  uint32_t aoff[kPieces];
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const int p = rt.p_begin + ar + kRowStride * i;
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
    aoff[i] = valid ? row * static_cast<uint32_t>(K) * 2u + 16u * aq : kRsrcOutOfRange;
  }
  // Activation block scales: with kTileAScales every thread stages K/512 dwords of
  // tile row tid / 4 (all of K) once, before the K loop; otherwise thread tid < kRows
  // stages the scale dword of tile row tid with each chunk
  const int srow_t = kTileAScales ? tid / 4 : tid;
  uint32_t soff = kRsrcOutOfRange;   // byte offset of tile row srow_t's scales
  if (srow_t < kRows) {
    const int p = rt.p_begin + srow_t;
    if (p < rt.p_end) {
      if (kW1) {
        const int slot = gather[p];
        if (static_cast<unsigned>(slot) < static_cast<unsigned>(n_slots))
          soff = static_cast<uint32_t>(slot / k_top) * static_cast<uint32_t>(K / 32);
      } else {
        soff = static_cast<uint32_t>(p) * static_cast<uint32_t>(K / 32);
      }
    }
  }
  unsigned char* a_lds = tile_lds;                       // [2][kAPieces][kRows][16 B]
  // [2][kThreads] dwords, or with kTileAScales [kRows][a_scl_stride] for all of K
  uint32_t* a_scl = reinterpret_cast<uint32_t*>(tile_lds + 2 * kABuf);
  const int a_scl_stride = K / 128 + 1;   // dwords per row: odd, so 16 rows hit 16 banks
  const int a_store = (aq * kRows + (ar ^ (4 * (aq & 1)))) * 16;
  // np: the pieces that hold rows of the subtiles a tile runs (a constant at each
  // call site); pieces past them are neither loaded nor stored
  // ra: the thread's pieces; rs: its scale dword.  Every thread loads and stores
  // one (threads >= kRows read the out-of-range offset, i.e. zero, into slots
  // nobody reads): a branch on the thread index inside the K loop would split the
  // loop body and the register allocator then spills the accumulators.
  auto load_a = [&](uint4 (&ra)[kPieces], uint32_t& rs, int kc, int np) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i)
      if (i < np)
        ra[i] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(arsrc, aoff[i] + kc * 256, 0, 0));
    if constexpr (!kTileAScales) rs = __builtin_amdgcn_raw_buffer_load_b32(srsrc, soff + kc * 4, 0, 0);
  };
  auto store_a = [&](const uint4 (&ra)[kPieces], uint32_t rs, int buf, int np) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i)
      if (i < np)
        *reinterpret_cast<uint4*>(a_lds + buf * kABuf + a_store + kRowStride * i * 16) = ra[i];
    if constexpr (!kTileAScales) a_scl[buf * kThreads + tid] = rs;
  };
  if constexpr (kTileAScales) {
    // K/128 dwords per row, four threads per row, K/512 consecutive dwords each
    // (the host takes this path for K a multiple of 2048: whole 16-byte groups)
    const int n_dw = K / 512, d0 = (tid & 3) * n_dw;
    for (int j = 0; j < n_dw; j += 4) {
      const uint4 v = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(srsrc, soff + 4 * (d0 + j), 0, 0));
      if (srow_t < kRows) {
        uint32_t* d = a_scl + srow_t * a_scl_stride + d0 + j;
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
      }
    }
  }

  // --- weights: kFrag fragments of 16 rows, this lane's row in each
  // The weights are the MFMA's A operand and the activations its B operand, so a
  // lane of D holds rows 4g .. 4g+3 of each fragment (weight rows, i.e. output
  // columns) for one activation row (lane & 15).  Lane m of fragment f loads weight
  // row wrow(f, m), chosen so that a lane's D values are consecutive output
  // columns: W2, 16 columns 16g .. 16g+15 of the wavefront's 64 (fragment f, row
  // i at 16g + 4f + i); W1, 8 gate columns 8g .. 8g+7 of its 32 and the matching up
  // columns.  The epilogue then stores 16 bytes per lane and instruction.
  auto wrow = [&](int f, int c16) {
    return kW1 ? (f >= kGate ? half : 0) + cg * (16 * kGate) + (c16 >> 2) * (4 * kGate) +
                     (f % kGate) * 4 + (c16 & 3)
               : cg * (16 * kFrag) + (c16 >> 2) * (4 * kFrag) + f * 4 + (c16 & 3);
  };
  const size_t row_q = static_cast<size_t>(K / 2), row_s = static_cast<size_t>(K / 32);
  // The wavefront reads its rows 256 K elements at a time (a pair of 128-element
  // chunks: 128 bytes of codes and 8 scale bytes per row).  Each load instruction
  // covers 8 rows x 128 contiguous bytes -- lane l takes row 8h + l/8 of a
  // fragment (h = 0, 1), bytes 16 (l % 8) .. +15 -- the read shape that streams
  // fastest on MI355X (the FP4 operand's own shape, 16 rows x 64 bytes, reads
  // ~20% slower).  The pair reaches the operand layout through kTileTransitBytes
  // of LDS per wavefront: lane (r16, g) reads row r16's 16-byte block 4j + g for
  // chunk j of the pair.  Row r's block b sits in 256-byte line r/2 at 16-byte
  // quad 8 (r % 2) + (b ^ r/2) of its fragment's 2 KB, so the stores (8 lanes at
  // a time) and the reads (16 lanes at a time) each meet 8 or 16 different quads.
  // Lane l loads the 8 scale bytes of row (fragment l/16, row l%16), kept as
  // [j][16][kFrag] dwords: one 16-byte read gives a lane its fragments' scale
  // dwords for chunk j.  The transit area is the wavefront's own and its LDS
  // operations run in order, so a pair is stored right after the reads of the
  // one before, with no barrier.  Loads go through a buffer resource on the
  // expert's slab: with an odd chunk count the last pair's second half reads the
  // next row's codes, or zeros past the slab, which no product uses.
  const int expert_u = __builtin_amdgcn_readfirstlane(rt.expert);
  const size_t e_rows = static_cast<size_t>(expert_u) * n_rows;
  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(wq + e_rows * row_q, static_cast<uint32_t>(static_cast<size_t>(n_rows) * row_q));
  const __amdgpu_buffer_rsrc_t srs =
      make_rsrc(wsc + e_rows * row_s, static_cast<uint32_t>(static_cast<size_t>(n_rows) * row_s));
  // fragment f's rows are wrow(f, 0) + (wrow(0, c) - wrow(0, 0)): a wave-uniform
  // fragment base plus a lane offset shared by all fragments
  const int row0 = wrow(0, 0);
  uint32_t fq[kFrag];
#pragma unroll
  for (int f = 0; f < kFrag; ++f)
    fq[f] = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(wrow(f, 0))) * static_cast<uint32_t>(row_q);
  const uint32_t vq0 = static_cast<uint32_t>((wrow(0, lane >> 3) - row0) * row_q) + 16u * (lane & 7);
  const uint32_t vq1 = static_cast<uint32_t>((wrow(0, 8 + (lane >> 3)) - row0) * row_q) + 16u * (lane & 7);
  const uint32_t vs = static_cast<uint32_t>(wrow(lane >> 4, r16) * row_s);
  const int last_pair = (n_chunks - 1) >> 1;
  uint4 wr[kFrag][2];
  uint4 sr;
  // pair p's codes into wr; for even pairs (with_scales) also the scales of pairs
  // p and p + 1 into sr (16 bytes a row: half the scale-line visits of one load
  // per pair).  The K loop advances two pairs per iteration, so which pairs carry
  // scales is fixed at compile time (a branch inside the loop would split its body
  // and spill the accumulators).
  auto load_pair = [&](int p, auto with_scales) {
#pragma unroll
    for (int f = 0; f < kFrag; ++f)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        wr[f][h] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs, h ? vq1 : vq0, fq[f] + 128u * p, 0));
    if constexpr (decltype(with_scales)::value)
      sr = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(srs, vs, 8u * p, 0));
  };
  const size_t a_scl_bytes =
      kTileAScales ? static_cast<size_t>(kRows) * (K / 128 + 1) * 4 : 2 * static_cast<size_t>(kThreads) * 4;
  unsigned char* wt = tile_lds + 2 * kABuf + a_scl_bytes + wave * kTileTransitBytes;
  uint32_t* wts = reinterpret_cast<uint32_t*>(wt + kFrag * 2048);   // [chunk % 4][16][kFrag]
  auto put_pair = [&](auto with_scales) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int f = 0; f < kFrag; ++f)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 8 * h + (lane >> 3), b = lane & 7;
        *reinterpret_cast<uint4*>(wt + f * 2048 + (r >> 1) * 256 + ((r & 1) * 8 + (b ^ (r >> 1))) * 16) =
            wr[f][h];
      }
    if constexpr (decltype(with_scales)::value) {
      wts[r16 * kFrag + (lane >> 4)] = sr.x;
      wts[(16 + r16) * kFrag + (lane >> 4)] = sr.y;
      wts[(32 + r16) * kFrag + (lane >> 4)] = sr.z;
      wts[(48 + r16) * kFrag + (lane >> 4)] = sr.w;
    }
    asm volatile("" ::: "memory");
  };

  // Without kR8 (128-row tiles): each fragment row is loaded in the FP4 operand's
  // own layout, 64 bytes per chunk, two chunks ahead; the weight scales are staged
  // in LDS for all of K (kLdsScales) or come with the weights.  Addresses: a
  // wave-uniform base (the expert's slab and the fragment's first row) plus one
  // 32-bit lane offset within the slab, so each load takes the scalar-base form
  // and costs the wavefront one VGPR of address.
  const uint8_t* wbase = wq + e_rows * row_q;
  const uint8_t* sbase = wsc + e_rows * row_s;
  const int lane_row0 = wrow(0, r16);
  const uint32_t lane_q = static_cast<uint32_t>(lane_row0 * row_q) + 16u * g;
  const uint32_t lane_s = static_cast<uint32_t>(lane_row0 * row_s);
  size_t dq[kFrag], ds[kFrag];   // fragment f's rows start wrow(f) - wrow(0) rows further on
#pragma unroll
  for (int f = 0; f < kFrag; ++f) {
    const int d = __builtin_amdgcn_readfirstlane(wrow(f, 0) - wrow(0, 0));
    dq[f] = static_cast<size_t>(d) * row_q;
    ds[f] = static_cast<size_t>(d) * row_s;
  }
  auto load_w = [&](uint4 (&q)[kFrag], uint32_t (&sd)[kFrag], int kc) {
#pragma unroll
    for (int f = 0; f < kFrag; ++f)
      q[f] = *reinterpret_cast<const uint4*>(wbase + (dq[f] + kc * 64) + lane_q);
    if constexpr (!kLdsScales) {
#pragma unroll
      for (int f = 0; f < kFrag; ++f)
        sd[f] = *reinterpret_cast<const uint32_t*>(sbase + (ds[f] + kc * 4) + lane_s);
    }
  };

  // staged scales of the wavefront's 64 weight rows, [chunk][16][4] dwords (in the
  // region the transit areas use on the other path)
  uint32_t* my_scales =
      reinterpret_cast<uint32_t*>(tile_lds + 2 * kABuf + a_scl_bytes) + wave * (n_chunks * 64);
  auto stage_scales = [&]() {
    const int f = lane >> 4;
    const uint8_t* srow = wsc + (e_rows + wrow(f, r16)) * row_s;
    // eight 16-byte loads in flight before their stores: a load-then-store loop
    // would wait one memory latency per iteration
    auto put = [&](int c, const uint4& d) {
      my_scales[((c + 0) * 16 + r16) * 4 + f] = d.x;
      my_scales[((c + 1) * 16 + r16) * 4 + f] = d.y;
      my_scales[((c + 2) * 16 + r16) * 4 + f] = d.z;
      my_scales[((c + 3) * 16 + r16) * 4 + f] = d.w;
    };
    int c = 0;
    for (; c + 32 <= n_chunks; c += 32) {
      uint4 d[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) d[j] = *reinterpret_cast<const uint4*>(srow + (c + 4 * j) * 4);
#pragma unroll
      for (int j = 0; j < 8; ++j) put(c + 4 * j, d[j]);
    }
    for (; c + 4 <= n_chunks; c += 4) put(c, *reinterpret_cast<const uint4*>(srow + c * 4));
    for (; c < n_chunks; ++c)
      my_scales[(c * 16 + r16) * 4 + f] = *reinterpret_cast<const uint32_t*>(srow + c * 4);
  };

  floatx4 acc[kMSub][kFrag];
#pragma unroll
  for (int mi = 0; mi < kMSub; ++mi)
#pragma unroll
    for (int f = 0; f < kFrag; ++f) acc[mi][f] = floatx4{0.f, 0.f, 0.f, 0.f};

  // one chunk: activations (two-part FP8) and their block scales from LDS buffer
  // `buf`, weights (FP4 codes) and their scale dwords from the transit area (chunk
  // kc is half kc % 2 of the pair stored there); subtiles 0 .. NS-1
  // (NS = kMSub, or fewer when the tile's rows end earlier).  Per subtile and
  // fragment two block-scaled MFMAs (16 x 16 x 128: FP4 weights x FP8 activations),
  // one on the hi parts and one on the lo parts.  The MFMA takes lane 16b + c's
  // scale for row / column c and 32-element block b: a lane of group g passes the
  // scales of block g.
  typedef int v8i __attribute__((ext_vector_type(8)));
  auto compute = [&](auto ns_c, int kc, int buf, const uint4 (&q)[kFrag], const uint32_t (&sd)[kFrag]) {
    constexpr int NS = decltype(ns_c)::value;
    int wsc_g[kFrag];   // byte 0: the scale of this lane's weight row, block g
    v8i wb[kFrag];      // 32 FP4 codes of this lane's weight row: elements 32g .. 32g+31
    if constexpr (tile_r8_path<kR8, kMSub, NS>()) {
      const int j = kc & 1, bj = 4 * j + g;
      const int off = (r16 >> 1) * 256 + ((r16 & 1) * 8 + (bj ^ (r16 >> 1))) * 16;
      const uint4 d = *reinterpret_cast<const uint4*>(wts + (16 * (kc & 3) + r16) * kFrag);
      const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
      for (int f = 0; f < kFrag; ++f) {
        const uint4 w = *reinterpret_cast<const uint4*>(wt + f * 2048 + off);
        wsc_g[f] = static_cast<int>(dw[f] >> (8 * g));
        wb[f] = v8i{static_cast<int>(w.x), static_cast<int>(w.y), static_cast<int>(w.z),
                    static_cast<int>(w.w), 0, 0, 0, 0};
      }
    } else {
      uint32_t dw[kFrag];
      if constexpr (kLdsScales) {
        const uint4 d = *reinterpret_cast<const uint4*>(my_scales + (kc * 16 + r16) * 4);
        dw[0] = d.x; dw[1] = d.y; dw[2] = d.z; dw[3] = d.w;
      } else {
#pragma unroll
        for (int f = 0; f < kFrag; ++f) dw[f] = sd[f];
      }
#pragma unroll
      for (int f = 0; f < kFrag; ++f) {
        wsc_g[f] = static_cast<int>(dw[f] >> (8 * g));
        wb[f] = v8i{static_cast<int>(q[f].x), static_cast<int>(q[f].y), static_cast<int>(q[f].z),
                    static_cast<int>(q[f].w), 0, 0, 0, 0};
      }
    }
    const unsigned char* abase = a_lds + buf * kABuf;
    const uint32_t* ascl = kTileAScales ? a_scl + kc : a_scl + buf * kThreads;
    const int ascl_row = kTileAScales ? a_scl_stride : 1;
    // one subtile's operands: hi pieces 2g, 2g+1 (bytes 32g .. 32g+31 of the chunk's
    // hi half), lo pieces 8 further, and the block scale of row 16 mi + r16
    auto read_sub = [&](int mi, v8i& ah, v8i& al, int& asc_g) {
      const int row = 16 * mi + r16;
      const uint4 h0 = *reinterpret_cast<const uint4*>(abase + ((2 * g) * kRows + row) * 16);
      const uint4 h1 = *reinterpret_cast<const uint4*>(abase + ((2 * g + 1) * kRows + (row ^ 4)) * 16);
      const uint4 l0 = *reinterpret_cast<const uint4*>(abase + ((8 + 2 * g) * kRows + row) * 16);
      const uint4 l1 = *reinterpret_cast<const uint4*>(abase + ((9 + 2 * g) * kRows + (row ^ 4)) * 16);
      asc_g = static_cast<int>(ascl[row * ascl_row] >> (8 * g));
      ah = v8i{static_cast<int>(h0.x), static_cast<int>(h0.y), static_cast<int>(h0.z),
               static_cast<int>(h0.w), static_cast<int>(h1.x), static_cast<int>(h1.y),
               static_cast<int>(h1.z), static_cast<int>(h1.w)};
      al = v8i{static_cast<int>(l0.x), static_cast<int>(l0.y), static_cast<int>(l0.z),
               static_cast<int>(l0.w), static_cast<int>(l1.x), static_cast<int>(l1.y),
               static_cast<int>(l1.z), static_cast<int>(l1.w)};
    };
    // Every subtile up to NS, also those past the tile's rows (they hold zeros).
    // The next subtile's operands are read into the other register set before this
    // subtile's MFMAs, so the LDS reads are in flight while they run and never write
    // registers an issued MFMA still reads (which costs wait states); the hi MFMAs
    // of all fragments go before the lo ones, so no MFMA waits on the one before it.
    // (Not in the 128-row kernel that loads the weight scales with the weights:
    // there the second register set does not fit beside its other registers.)
    constexpr bool kTwoSets =
        tile_r8_path<kR8, kMSub, NS>() ? NS <= 4 : !(kMSub == 8 && !kLdsScales);
    v8i ah0, al0, ah1, al1;
    int as0 = 0, as1 = 0;
    read_sub(0, ah0, al0, as0);
#pragma unroll
    for (int mi = 0; mi < NS; ++mi) {
      if constexpr (kTwoSets) {
        if (mi + 1 < NS) {
          if (mi & 1)
            read_sub(mi + 1, ah0, al0, as0);
          else
            read_sub(mi + 1, ah1, al1, as1);
        }
      } else if (mi > 0) {
        read_sub(mi, ah0, al0, as0);
      }
      const bool second = kTwoSets && (mi & 1);
      const v8i ah = second ? ah1 : ah0;
      const v8i al = second ? al1 : al0;
      const int asc_g = second ? as1 : as0;
      // formats: A (weights) FP4 E2M1 = 4, B (activations) FP8 E4M3 = 0
#pragma unroll
      for (int f = 0; f < kFrag; ++f)
        acc[mi][f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wb[f], ah, acc[mi][f], 4, 0, 0,
                                                                       wsc_g[f], 0, asc_g);
#pragma unroll
      for (int f = 0; f < kFrag; ++f)
        acc[mi][f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wb[f], al, acc[mi][f], 4, 0, 0,
                                                                       wsc_g[f], 0, asc_g);
      // at most two subtiles' operands live at a time (the compiler would otherwise
      // hoist every subtile's LDS reads next to the 128 accumulators and spill)
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int last = n_chunks - 1;
  int kc = 0;
  // D of the tile's subtiles 0 .. NS-1 to the output (the accumulators of
  // subtiles past NS are never touched on that path)
  auto epilogue = [&](auto ns_c) {
    constexpr int NS = decltype(ns_c)::value;
    if (!store_cols) return;
    // D of fragment f, lane (r16, g), element i: activation row 16 mi + r16, output
    // column wrow(f, 4g + i); per lane these are consecutive from column wrow(0, 4g)
    const bool do_clamp = clamp != 0;
    const int col0 = wrow(0, 4 * g);
#pragma unroll
    for (int mi = 0; mi < NS; ++mi) {
      if (mi >= msub) continue;   // uniform over the workgroup
      const int p = rt.p_begin + mi * 16 + r16;
      if constexpr (kW1) {
        // h in two-part FP8: the wavefront's 32 gate columns cg*32 .. cg*32+31 are one
        // 32-element block of h's row, held by the four lanes r16 + 16g (8 each); the
        // block's largest magnitude comes from two lane exchanges, which every lane
        // takes part in
        float hv[8];
        uint32_t m = 0;
#pragma unroll
        for (int f = 0; f < kGate; ++f)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            hv[4 * f + i] = swiglu(acc[mi][f][i], acc[mi][f + kGate][i], limit, do_clamp);
            const uint32_t a = __float_as_uint(hv[4 * f + i]) & 0x7FFFFFFFu;
            m = a > m ? a : m;
          }
        uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 16, 64));
        m = o > m ? o : m;
        o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 32, 64));
        m = o > m ? o : m;
        const uint32_t s = a8_scale_byte(m);
        const float inv = a8_inv_scale(s);
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[i] *= inv;
        uint2 hi, lo;
        a8_split8(hv, hi, lo);
        if (p >= rt.p_end) continue;
        // block cg = chunk cg / 4, block cg % 4 of it; this lane's 8 elements are
        // elements 8g .. 8g+7 of the block
        uint8_t* orow = static_cast<uint8_t*>(out) + static_cast<int64_t>(p) * (2 * ld_out) +
                        (cg / 4) * 256;
        const int pos = a8_pos(32 * (cg % 4) + 16 * (g >> 1)) + 8 * (g & 1);
        *reinterpret_cast<uint2*>(orow + pos) = hi;
        *reinterpret_cast<uint2*>(orow + 128 + pos) = lo;
        if (g == 0) out_sc[static_cast<int64_t>(p) * (ld_out / 32) + cg] = static_cast<uint8_t>(s);
      } else {
        if (p >= rt.p_end) continue;
        uint16_t* orow = static_cast<uint16_t*>(out) + static_cast<int64_t>(p) * ld_out + col0;
        uint32_t w[2 * kFrag];
#pragma unroll
        for (int f = 0; f < kFrag; ++f)
#pragma unroll
          for (int i = 0; i < 4; i += 2)
            w[2 * f + i / 2] = pack_bf16x2(acc[mi][f][i], acc[mi][f][i + 1]);
        *reinterpret_cast<uint4*>(orow) = make_uint4(w[0], w[1], w[2], w[3]);
        *reinterpret_cast<uint4*>(orow + 8) = make_uint4(w[4], w[5], w[6], w[7]);
      }
    }
  };

  // Activations one chunk ahead (registers ra, then LDS).  Weights one pair ahead
  // (registers wr, then the transit area), or, on the operand-layout path, two
  // chunks ahead in registers.  The K loop is instantiated per subtile count --
  // 80-row tiles: 2 .. 5; 128-row tiles: 2, 4, 8 -- and the tile takes the
  // smallest that covers its rows (a uniform branch outside the loop): the last
  // tile of an expert, and every tile of an expert with few rows, runs only the
  // MFMAs of its rows.
  auto run = [&](auto ns_c) {
    constexpr int NS = decltype(ns_c)::value;
    constexpr int NP = (NS * 16 + kRowStride - 1) / kRowStride;   // pieces in use
    if constexpr (tile_r8_path<kR8, kMSub, NS>()) {
      const std::true_type sc{};
      const std::false_type no_sc{};
      uint4 ra[kPieces];
      uint32_t rs = 0;
      const uint4 qd[kFrag] = {};
      const uint32_t sdd[kFrag] = {};
      load_pair(0, sc);
      load_a(ra, rs, 0, NP);
      put_pair(sc);
      load_pair(last_pair >= 1 ? 1 : 0, no_sc);
      store_a(ra, rs, 0, NP);
      __syncthreads();
      // four chunks (pairs P, P + 1) per iteration; each pair is stored after the
      // last reads of the one before.  Past the last pair the loads repeat it; what
      // they store is never read.
      for (; kc + 4 <= n_chunks; kc += 4) {
        const int P = kc >> 1;
        load_a(ra, rs, kc + 1, NP);
        compute(ns_c, kc, 0, qd, sdd);
        store_a(ra, rs, 1, NP);
        __syncthreads();
        load_a(ra, rs, kc + 2, NP);
        compute(ns_c, kc + 1, 1, qd, sdd);
        put_pair(no_sc);   // pair P + 1 (its scales came with pair P)
        load_pair(P + 2 <= last_pair ? P + 2 : last_pair, sc);
        store_a(ra, rs, 0, NP);
        __syncthreads();
        load_a(ra, rs, kc + 3, NP);
        compute(ns_c, kc + 2, 0, qd, sdd);
        store_a(ra, rs, 1, NP);
        __syncthreads();
        load_a(ra, rs, kc + 4 <= last ? kc + 4 : last, NP);
        compute(ns_c, kc + 3, 1, qd, sdd);
        put_pair(sc);      // pair P + 2 and the scales of P + 2, P + 3
        load_pair(P + 3 <= last_pair ? P + 3 : last_pair, no_sc);
        store_a(ra, rs, 0, NP);
        __syncthreads();
      }
      // the last one to three chunks: pair P (stored, with the scales of P + 1) and
      // pair P + 1 (in wr)
      if (kc < n_chunks) {
        const bool c1 = kc + 1 < n_chunks, c2 = kc + 2 < n_chunks;
        load_a(ra, rs, c1 ? kc + 1 : last, NP);
        compute(ns_c, kc, 0, qd, sdd);
        if (c1) {
          store_a(ra, rs, 1, NP);
          __syncthreads();
          load_a(ra, rs, c2 ? kc + 2 : last, NP);
          compute(ns_c, kc + 1, 1, qd, sdd);
          if (c2) {
            put_pair(no_sc);
            store_a(ra, rs, 0, NP);
            __syncthreads();
            compute(ns_c, kc + 2, 0, qd, sdd);
          }
        }
      }
    } else {
      uint4 q0[kFrag], q1[kFrag];
      uint32_t s0[kFrag], s1[kFrag];
      if constexpr (kLdsScales) stage_scales();
      if constexpr (kWaves == 4) {
        // 80-row tiles: activations two chunks ahead in registers, one in LDS
        uint4 ra0[kPieces], ra1[kPieces];
        uint32_t rs0 = 0, rs1 = 0;
        load_a(ra0, rs0, 0, NP);
        load_w(q0, s0, 0);
        load_w(q1, s1, last >= 1 ? 1 : 0);
        load_a(ra1, rs1, last >= 1 ? 1 : 0, NP);
        store_a(ra0, rs0, 0, NP);
        __syncthreads();
        for (; kc + 2 <= n_chunks; kc += 2) {
          load_a(ra0, rs0, kc + 2 <= last ? kc + 2 : last, NP);
          compute(ns_c, kc, 0, q0, s0);
          load_w(q0, s0, kc + 2 <= last ? kc + 2 : last);
          store_a(ra1, rs1, 1, NP);
          __syncthreads();
          load_a(ra1, rs1, kc + 3 <= last ? kc + 3 : last, NP);
          compute(ns_c, kc + 1, 1, q1, s1);
          load_w(q1, s1, kc + 3 <= last ? kc + 3 : last);
          store_a(ra0, rs0, 0, NP);
          __syncthreads();
        }
      } else {
        uint4 ra[kPieces];
        uint32_t rs = 0;
        load_a(ra, rs, 0, NP);
        load_w(q0, s0, 0);
        load_w(q1, s1, last >= 1 ? 1 : 0);
        store_a(ra, rs, 0, NP);
        __syncthreads();
        for (; kc + 2 <= n_chunks; kc += 2) {
          load_a(ra, rs, kc + 1, NP);
          compute(ns_c, kc, 0, q0, s0);
          load_w(q0, s0, kc + 2 <= last ? kc + 2 : last);
          store_a(ra, rs, 1, NP);
          __syncthreads();
          load_a(ra, rs, kc + 2 <= last ? kc + 2 : last, NP);
          compute(ns_c, kc + 1, 1, q1, s1);
          load_w(q1, s1, kc + 3 <= last ? kc + 3 : last);
          store_a(ra, rs, 0, NP);
          __syncthreads();
        }
      }
      if (kc < n_chunks) compute(ns_c, kc, 0, q0, s0);   // odd chunk count: last chunk in q0
    }
    epilogue(ns_c);
  };
  if constexpr (kMSub == 5) {
    if (msub > 4) {
      run(std::integral_constant<int, 5>{});
    } else if (msub > 3) {
      run(std::integral_constant<int, 4>{});
    } else if (msub > 2) {
      run(std::integral_constant<int, 3>{});
    } else {
      run(std::integral_constant<int, 2>{});
    }
  } else {
    if (msub > kMSub / 2) {
      run(std::integral_constant<int, kMSub>{});
    } else if (msub > kMSub / 4) {
      run(std::integral_constant<int, kMSub / 2>{});
    } else {
      run(std::integral_constant<int, kMSub / 4>{});
    }
  }
}

template <bool kW1, int kMSub, int kFrag, int kWaves, bool kR8, bool kLdsScales, bool kTileAScales>
hipError_t launch_tile_t(const TileArgs& t, hipStream_t stream) {
  // wavefronts per row tile: W1 pairs `half` gate rows with as many up rows, 16 *
  // kFrag/2 of each per wavefront; W2 covers n_rows output rows, 16 * kFrag each
  const int wpt = kW1 ? t.half / (8 * kFrag) : t.n_rows / (16 * kFrag);
  const int bpt = (wpt + kWaves - 1) / kWaves;
  size_t lds = tile_lds_bytes(kMSub, t.K, kWaves, kR8, kLdsScales, kTileAScales);
  // whole tiles per XCD cover row tiles in groups of 8, the column-block/XCD split
  // in pairs: round up to whole groups
  const int64_t blocks = t.whole_tiles               ? (t.tile_bound + 7) / 8 * 8 * bpt
                         : (bpt == 16 || bpt == 8) ? (t.tile_bound + 1) / 2 * 2 * bpt
                                                   : t.tile_bound * bpt;
  gemm_tile_kernel<kW1, kMSub, kFrag, kWaves, kR8, kLdsScales, kTileAScales>
      <<<static_cast<unsigned>(blocks), 64 * kWaves, lds, stream>>>(
      t.act, t.act_bytes, t.asc, t.asc_bytes, t.gather, t.k_top, t.n_slots, t.wq, t.wsc, t.tiles,
      t.n_tiles, t.K, t.n_rows, t.half, wpt, bpt, t.limit, t.clamp, t.out, t.out_sc, t.ld_out,
      t.whole_tiles ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tile(bool w1, int tile_rows, const TileArgs& t, hipStream_t stream) {
  // W1: operand-layout loads; the E8M0 weight scales are staged in LDS while they
  // fit beside the activation buffers (in the CU's 160 KB for 128-row tiles, one
  // workgroup per CU; in half of it for 80-row tiles, two per CU; K <= 4096 either
  // way), otherwise they come with the weights.  W2: the weight transit (for
  // 128-row tiles, on tiles with fewer than eight subtiles).  128-row tiles stage
  // the activations' block scales for all of K when they fit too (K a multiple of
  // 2048 up to 4096: each thread stages whole 16-byte groups); 80-row tiles stage
  // them per chunk.
  if (tile_rows == 128) {
    const bool tile_as = t.K % 2048 == 0 && tile_lds_bytes(8, t.K, 8, !w1, true, true) <= kCuLds;
    if (w1)
      return tile_as ? launch_tile_t<true, 8, 4, 8, false, true, true>(t, stream)
                     : launch_tile_t<true, 8, 4, 8, false, false, false>(t, stream);
    return tile_as ? launch_tile_t<false, 8, 4, 8, true, true, true>(t, stream)
                   : launch_tile_t<false, 8, 4, 8, true, false, false>(t, stream);
  }
  if (!w1) return launch_tile_t<false, 5, 4, 4, true, false, false>(t, stream);
  if (tile_lds_bytes(5, t.K, 4, false, true, false) <= kTileLdsPerWorkgroup)
    return launch_tile_t<true, 5, 4, 4, false, true, false>(t, stream);
  return launch_tile_t<true, 5, 4, 4, false, false, false>(t, stream);
}

}  // namespace moe
