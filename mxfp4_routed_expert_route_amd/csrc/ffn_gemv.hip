// Weight-streaming GEMV for decode batches: one-row tiles.
//
// With fewer rows than experts (T * k < E: a decode or speculative-verify step)
// an expert holds one row, sometimes two, and the FFN is a stream of the touched
// experts' weights past their few activation rows (txtmix.com article, §8:
// decode speed is bandwidth over the bytes read per token).  The matrix cores
// would idle on 16-row tiles that hold one real row, so this kernel multiplies on
// the vector ALUs and spends its effort on the read pattern instead: every load
// instruction of a wavefront reads 1 KB of one weight row, contiguous (lane l:
// bytes 16l .. 16l+15, i.e. K elements 32l .. 32l+31 of a 2048-element slice),
// non-temporal, and a wavefront's weight rows are consecutive, so it reads 8 KB
// runs.  A read-only probe of this pattern streams the verify step's W1 (46
// experts x 4096 rows x 2 KB) at 6.6 TB/s against 5.6-5.7 TB/s for the
// 16-rows-by-64-bytes pattern of the MFMA kernels.
//
// A wavefront streams groups of 8 weight rows of one row tile's expert (W1: 4 gate
// rows and the matching 4 up rows; W2: 8 output rows), all of K for each, K 2048 or
// 4096.  Per 1 KB slice of a row: the lane's 32 E2M1 codes are converted to bf16
// with their E8M0 scale (the gfx950 scaled convert; exact) and multiplied by the
// lane's 32 activations with two-element dot products into fp32.  Each group's 8
// sums are reduced over the 64 lanes with lane exchanges, and W1 applies the
// clamped SwiGLU.  A group's E8M0 scales come as two dwords per lane and slice and
// reach their lanes by lane permutes.  A tile is one row: an expert with several
// rows gets several tiles, whose wavefronts read its weights at about the same time
// on the same XCD (W1 reads such experts with normal loads, so the later reads hit
// the L2); one activation row keeps the registers for two groups of weights in
// flight.  No LDS, no workgroup barrier: every wavefront runs on its own.  In the
// one-call layer, W2 runs with the weighted combine folded in
// (gemv_w2_combine_kernel, one workgroup per token and 32 output columns).
#include <type_traits>

#include "ffn_common.h"

namespace moe {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGemvRows = 8;         // weight rows per wavefront
constexpr int kGemvNt = 2;           // cache-policy operand of a buffer load: non-temporal
constexpr int kGemvSlice = 2048;     // K elements per 1 KB row slice (64 lanes x 32)
// wavefronts per launch, at most: with two resident per SIMD, six rounds of them
// (measured on the verify step's W1 / W2: 2,048 wavefronts 70.6 / 39.0 us, 3,072
// 68.3 / 36.9, 12,288 67.3 / 34.8, 24,576 -- one group each -- 75.3 / 35.6)
constexpr int kGemvMaxWaves = 12288;

__device__ __forceinline__ uint4 load_nt(const uint8_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Lane exchanges of the final reduction: x of lane ^ 16 (a swizzle within 32
// lanes), of lane ^ 8 (DPP row_ror:8), of lane ^ 7 within 8 lanes (row_half_mirror),
// of lane ^ 2 and lane ^ 1 (quad permutations); lane mappings checked on the GPU.
__device__ __forceinline__ float swz_xor16(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x),
                                                               0x401F));
}
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), kCtrl,
                                                            0xF, 0xF, false));
}
constexpr int kDppXor8 = 0x128, kDppMirror8 = 0x141, kDppXor2 = 0x4E, kDppXor1 = 0xB1;

// 32 E2M1 codes (16 bytes, element 2m in the low nibble of byte m) with E8M0 scale
// `scale` -> 16 bf16 pairs, pair m = elements 2m, 2m+1
__device__ __forceinline__ void dequant32(const uint4 q, float scale, bf16x2 (&w)[16]) {
  const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[4 * i + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], scale, 0);
    w[4 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], scale, 1);
    w[4 * i + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], scale, 2);
    w[4 * i + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], scale, 3);
  }
}

// acc + sum over the 32 elements of w * a (a: 32 bf16 as 4 x 16 bytes, pair m in
// dword m), fp32
__device__ __forceinline__ float dot32(const bf16x2 (&w)[16], const uint4 (&a)[4], float acc) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t d[4] = {a[c].x, a[c].y, a[c].z, a[c].w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(w[4 * c + i], __builtin_bit_cast(bf16x2, d[i]), acc,
                                            false);
  }
  return acc;
}

// The E8M0 scale byte of row j (0..7) of a group for this lane (block `lane` of the
// slice), from the dword pair a group's scales are read in: the dword of rows
// 4 (j / 4) + lane / 16 holds blocks 4 (lane % 16) .. +3, so row j's block `lane` is
// byte lane % 4 of lane 16 (j % 4) + lane / 4's dword `sd` (the one for j / 4).
__device__ __forceinline__ uint32_t gemv_scale_byte(uint32_t sd, int j, int lane) {
  const int holder = 16 * (j & 3) + (lane >> 2);
  const uint32_t d =
      static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(4 * holder, static_cast<int>(sd)));
  return (d >> (8 * (lane & 3))) & 0xFFu;
}

// The 8 row sums of a group: v[j] = sum over the lane's elements of row j's
// dequantised weights times the lane's activations, fp32, slice by slice.
// scale(j, i): the E8M0 scale byte of row j, slice i, for this lane.
template <int kSlices, typename Scale>
__device__ __forceinline__ void gemv_dot8(const uint4 (&q)[kGemvRows][kSlices], Scale scale,
                                          const uint4 (&a)[kSlices][4], float (&v)[kGemvRows]) {
#pragma unroll
  for (int j = 0; j < kGemvRows; ++j) {
    v[j] = 0.f;
#pragma unroll
    for (int i = 0; i < kSlices; ++i) {
      bf16x2 w[16];
      dequant32(q[j][i], e8m0_as_f32(scale(j, i)), w);
      v[j] = dot32(w, a[i], v[j]);
      // one row slice's 32 converted weights live at a time (the compiler would
      // otherwise convert every slice of the group first and run out of registers)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Reduce the 8 row sums over the 64 lanes, halving the values a lane holds at each
// exchange: lanes with bit 4 of the lane set keep the upper half of their values,
// the others the lower half, each adding its partner's copy; then the same over
// lane bits 3 and 2 (8 -> 4 -> 2 -> 1 values).  The bit-2 partner is the mirror
// lane (lane ^ 7), which holds the same values.  A lane then holds row
// (lane >> 2) & 7 summed over 8 lanes, and the exchanges with lane ^ 2, lane ^ 1
// and lane ^ 32 complete the sum over all 64 lanes, which every lane holding that
// row returns.
__device__ __forceinline__ float gemv_reduce8(float (&v)[kGemvRows], int lane) {
  const bool up16 = (lane & 16) != 0, up8 = (lane & 8) != 0, up4 = (lane & 4) != 0;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float send = up16 ? v[m] : v[m + 4];
    const float keep = up16 ? v[m + 4] : v[m];
    v[m] = keep + swz_xor16(send);
  }
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const float send = up8 ? v[m] : v[m + 2];
    const float keep = up8 ? v[m + 2] : v[m];
    v[m] = keep + dpp<kDppXor8>(send);
  }
  {
    const float send = up4 ? v[0] : v[1];
    const float keep = up4 ? v[1] : v[0];
    v[0] = keep + dpp<kDppMirror8>(send);
  }
  float sum = v[0];
  sum += dpp<kDppXor2>(sum);
  sum += dpp<kDppXor1>(sum);
  return sum + __shfl_xor(sum, 32, 64);
}

// The lane's activations of a K-row: slice i, elements 2048 i + 32 lane .. +31.
template <int kSlices>
__device__ __forceinline__ void gemv_load_act(const uint16_t* row_base, int lane,
                                              uint4 (&a)[kSlices][4]) {
  const uint4* src = reinterpret_cast<const uint4*>(row_base + 32 * lane);
#pragma unroll
  for (int i = 0; i < kSlices; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) a[i][c] = src[i * (kGemvSlice / 8) + c];
}

// Each row tile (one row) gets `wpt` wavefronts; wavefront w of a tile owns the
// groups of 8 weight rows w, w + wpt, w + 2 wpt, ... (so the tile's wavefronts read
// adjacent rows at the same time) and streams them with one group in flight while
// it computes the previous one.  act: W1 x rows ([T][K] bf16, tile row p -> token
// gather[p] / k_top); W2 h rows ([n_slots][K] bf16, tile row p -> row p).  out: W1
// h ([n_slots][ld_out] bf16, columns = gate rows), W2 y_sorted ([n_slots][ld_out]
// bf16).
template <bool kW1, int kSlices>
__global__ __launch_bounds__(256) void gemv_kernel(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ gather, int k_top, int n_slots,
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ wsc,
    const RowTile* __restrict__ tiles, const int32_t* __restrict__ n_tiles, int n_rows, int half,
    int groups, int wpt, float limit, int clamp, uint16_t* __restrict__ out, int ld_out) {
  constexpr int K = kSlices * kGemvSlice;
  const int lane = threadIdx.x & 63;
  // wavefront-uniform values are made visibly so (scalar registers, scalar branches)
  const int wave = static_cast<int>(blockIdx.x) * 4 +
                   __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int tile_id = wave / wpt;
  const int w_in = wave - tile_id * wpt;
  if (tile_id >= *n_tiles || w_in >= groups) return;   // per wavefront (no barrier here)
  const RowTile rt = tiles[tile_id];
  const int p = __builtin_amdgcn_readfirstlane(rt.p_begin);   // the tile's one row
  const int expert = __builtin_amdgcn_readfirstlane(rt.expert);

  // W1: an expert whose rows span several tiles (two or more rows) is read by
  // several tiles' wavefronts at about the same time, on the same XCD (tile t's
  // wavefront w and tile t + 1's are a multiple of 8 workgroups apart): its loads
  // are normal ones, so that the later reads can hit the L2; all others are
  // non-temporal.
  auto body = [&](auto aux_c) __attribute__((always_inline)) {
    constexpr int kAux = decltype(aux_c)::value;
    // the expert's codes and scales as buffer resources: each load below is a scalar
    // row offset plus the lane's 32-bit offset (no 64-bit address arithmetic per lane)
    const size_t e_rows = static_cast<size_t>(expert) * n_rows;
    const __amdgpu_buffer_rsrc_t wrs =
        make_rsrc(wq + e_rows * (K / 2), static_cast<uint32_t>(n_rows) * (K / 2));
    const __amdgpu_buffer_rsrc_t srs =
        make_rsrc(wsc + e_rows * (K / 32), static_cast<uint32_t>(n_rows) * (K / 32));
    const int lane16 = 16 * lane;
    const int lane_s = (lane >> 4) * (K / 32) + 4 * (lane & 15);
    // weight row j of group g (W1: j < 4 gate rows 4 g + j, j >= 4 the matching up
    // rows; W2: output rows 8 g + j)
    auto wrow = [&](int g, int j) {
      return kW1 ? (j < 4 ? 4 * g + j : half + 4 * g + (j - 4)) : kGemvRows * g + j;
    };
    // A group's codes: one 1 KB load per row and slice, non-temporal.  Its scales: two
    // dwords per lane and slice (rows wrow(g, 4m + lane / 16), blocks 4 (lane % 16) ..
    // +3 of the slice), from which each lane takes its byte (block `lane` of row j)
    // with a lane permute when it is used.
    auto load_group = [&](int g, uint4 (&q)[kGemvRows][kSlices], uint32_t (&sd)[2][kSlices]) {
#pragma unroll
      for (int i = 0; i < kSlices; ++i)
#pragma unroll
        for (int m = 0; m < 2; ++m)
          sd[m][i] = __builtin_amdgcn_raw_buffer_load_b32(
              srs, lane_s + 64 * i, __builtin_amdgcn_readfirstlane(wrow(g, 4 * m) * (K / 32)), 0);
#pragma unroll
      for (int i = 0; i < kSlices; ++i)
#pragma unroll
        for (int j = 0; j < kGemvRows; ++j)
          q[j][i] = __builtin_bit_cast(
              uint4, __builtin_amdgcn_raw_buffer_load_b128(
                         wrs, lane16 + 1024 * i,
                         __builtin_amdgcn_readfirstlane(wrow(g, j) * (K / 2)), kAux));
      // keep the loads where they stand: hoisted into the previous group's products
      // they would hold a third register set
      __builtin_amdgcn_sched_barrier(0);
    };
    uint4 a[kSlices][4];   // the lane's activations (filled below)
    const int idx = (lane >> 2) & 7;   // the row whose sum a lane holds after the reduction
    // group g from q / sd: products, reduction over the lanes, epilogue
    auto finish_group = [&](int g, const uint4 (&q)[kGemvRows][kSlices],
                            const uint32_t (&sd)[2][kSlices]) {
      float v[kGemvRows];
      gemv_dot8<kSlices>(q, [&](int j, int i) { return gemv_scale_byte(sd[j >> 2][i], j, lane); },
                         a, v);
      const float sum = gemv_reduce8(v, lane);
      if (kW1) {
        // gate rows are rows 0..3 (lane bit 4 clear), their up rows 4..7 (lane ^ 16)
        const float up = swz_xor16(sum);
        if ((lane & 0x33) == 0)   // one lane per gate row
          out[static_cast<int64_t>(p) * ld_out + 4 * g + idx] =
              f32_to_bf16_bits(swiglu(sum, up, limit, clamp != 0));
      } else if ((lane & 0x23) == 0) {   // one lane per row
        out[static_cast<int64_t>(p) * ld_out + kGemvRows * g + idx] = f32_to_bf16_bits(sum);
      }
    };

    // Two register sets: the next group's loads are issued before the current group
    // is computed.  The wavefront's groups are w_in + r wpt, r < groups / wpt (an even
    // count), so every load is issued on every path (no load sits under a branch,
    // which would make the compiler's later waits count as if it had not been taken)
    // and each wait counts only older loads.  The first group's loads go out before
    // the activation row's (which wait on the gather index).
    uint4 qa[kGemvRows][kSlices], qb[kGemvRows][kSlices];
    uint32_t sa[2][kSlices], sbb[2][kSlices];
    int g = w_in;
    load_group(g, qa, sa);
    {
      // W1: the tile row's token.  gather comes from moe_expert_offsets; an entry out
      // of range (outside that contract) reads token 0 instead, so that the loads stay
      // in bounds and unconditional (its h row is then unspecified).
      int64_t row = p;
      if (kW1) {
        const int slot = __builtin_amdgcn_readfirstlane(gather[p]);
        row = static_cast<unsigned>(slot) < static_cast<unsigned>(n_slots) ? slot / k_top : 0;
      }
      gemv_load_act<kSlices>(act + row * K, lane, a);
    }
#pragma unroll 1
    for (;;) {
      load_group(g + wpt, qb, sbb);
      finish_group(g, qa, sa);
      if (g + 2 * wpt >= groups) break;
      load_group(g + 2 * wpt, qa, sa);
      finish_group(g + wpt, qb, sbb);
      g += 2 * wpt;
    }
    finish_group(g + wpt, qb, sbb);
  };
  if (kW1 && __builtin_amdgcn_readfirstlane(rt.multi) != 0)
    body(std::integral_constant<int, 0>{});
  else
    body(std::integral_constant<int, kGemvNt>{});
}

// gemv_dot8 with the lane's activations fetched half a slice at a time (act(i, c):
// 16-byte chunk c of slice i): the same products summed in the same order per row,
// with 8 activation and 8 converted-weight registers live instead of 16 and 16.
template <int kSlices, typename Scale, typename Act>
__device__ __forceinline__ void gemv_dot8_halves(const uint4 (&q)[kGemvRows][kSlices], Scale scale,
                                                 Act act, float (&v)[kGemvRows]) {
#pragma unroll
  for (int j = 0; j < kGemvRows; ++j) v[j] = 0.f;
#pragma unroll
  for (int i = 0; i < kSlices; ++i)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint4 ac[2] = {act(i, 2 * hh), act(i, 2 * hh + 1)};
#pragma unroll
      for (int j = 0; j < kGemvRows; ++j) {
        const float sc = e8m0_as_f32(scale(j, i));
        const uint32_t d[2] = {hh ? q[j][i].z : q[j][i].x, hh ? q[j][i].w : q[j][i].y};
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const uint32_t ad[4] = {ac[c].x, ac[c].y, ac[c].z, ac[c].w};
          bf16x2 w[4];
          w[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[c], sc, 0);
          w[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[c], sc, 1);
          w[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[c], sc, 2);
          w[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[c], sc, 3);
#pragma unroll
          for (int m = 0; m < 4; ++m)
            v[j] = __builtin_amdgcn_fdot2_f32_bf16(w[m], __builtin_bit_cast(bf16x2, ad[m]), v[j],
                                                   false);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
}

// W2 with the weighted combine, for the one-call layer on the GEMV path.  A
// workgroup takes one token t and 32 output columns (a wavefront per group of 8),
// and first copies the token's k rows of h (rows scatter[t k + j]) into LDS, where
// its four wavefronts read them.  Each wavefront then runs over the k choices in
// slot order j: for choice j (expert e = ids[t k + j], sorted row p) it computes
// y_sorted[p] on its 8 columns exactly as gemv_kernel<false> does (same products in
// the same order, same reduction) and stores it, and adds w[t k + j] times that
// bf16 value to the column's fp32 sum, in j order, as the combine kernel does; y[t]
// is rounded once at the end.  So y and y_sorted are bit-identical to the separate
// W2 and combine launches, without the combine's launch and its re-read of
// y_sorted.  The next choice's weight loads go out before the current one is
// computed; k is a template argument so that the loop unrolls and every wait
// counts only older loads.  The token's choices sit in lanes 0..k-1 (read once),
// the scale bytes arrive as two dwords per lane and reach their lanes by a lane
// permute, and the products take half a slice of activations at a time: about 110
// VGPRs at K = 2048, four wavefronts per SIMD, so a verify-sized grid (8 tokens x
// 4096 columns: 4096 wavefronts) is resident at once.
template <int kSlices, int kTop>
__global__ __launch_bounds__(256, kSlices == 1 ? 4 : 2) void gemv_w2_combine_kernel(
    const uint16_t* __restrict__ h, const int32_t* __restrict__ ids,
    const float* __restrict__ topw, const int32_t* __restrict__ scatter, int T, int E,
    int n_slots, const uint8_t* __restrict__ wq, const uint8_t* __restrict__ wsc, int n_rows,
    int blocks_per_token, uint16_t* __restrict__ y_sorted, uint16_t* __restrict__ y,
    int ld_out) {
  constexpr int K = kSlices * kGemvSlice;
  constexpr int kRow16 = K / 8;   // 16-byte words per h row
  constexpr int k_top = kTop;
  __shared__ uint4 h_lds[kTop * kRow16];
  const int t = static_cast<int>(blockIdx.x) / blocks_per_token;
  if (t >= T) return;   // whole workgroup (before the barrier)
  const int lane = threadIdx.x & 63;
  const int g = (static_cast<int>(blockIdx.x) - t * blocks_per_token) * 4 +
                __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int idx = (lane >> 2) & 7;   // the column a lane holds after the reduction
  const bool stores = (lane & 0x23) == 0;   // one lane per column

  // the token's k choices, lane j holding choice j: expert, sorted row, weight (an
  // invalid choice, expert or row out of range, contributes nothing)
  int lane_e = -1, lane_p = -1;
  float lane_w = 0.f;
  if (lane < k_top) {
    const int64_t s = static_cast<int64_t>(t) * k_top + lane;
    lane_e = ids[s];
    lane_p = scatter[s];
    lane_w = topw[s];
  }
  const bool lane_ok = static_cast<unsigned>(lane_e) < static_cast<unsigned>(E) &&
                       static_cast<unsigned>(lane_p) < static_cast<unsigned>(n_slots);
  if (!lane_ok) lane_e = -1;
  auto expert_of = [&](int j) { return __builtin_amdgcn_readlane(lane_e, j); };   // -1: none
  auto row_of = [&](int j) { return __builtin_amdgcn_readlane(lane_p, j); };

  // Scales: the group's 8 rows x 64 blocks of a slice are read as two dwords per lane
  // (rows 4m + lane / 16, blocks 4 (lane % 16) .. +3) and each lane's byte (block
  // lane of row r) is fetched from its holder with a lane permute when used.
  auto load_w = [&](int e, uint4 (&q)[kGemvRows][kSlices], uint32_t (&sd)[2][kSlices]) {
    const size_t e_rows = static_cast<size_t>(e >= 0 ? e : 0) * n_rows;
    const uint8_t* wbase = wq + e_rows * (K / 2) + 16 * lane;
    const uint8_t* sbase = wsc + e_rows * (K / 32);
#pragma unroll
    for (int i = 0; i < kSlices; ++i)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const size_t row = static_cast<size_t>(kGemvRows * g + 4 * m + (lane >> 4));
        sd[m][i] = *reinterpret_cast<const uint32_t*>(sbase + row * (K / 32) + 64 * i +
                                                      4 * (lane & 15));
      }
#pragma unroll
    for (int i = 0; i < kSlices; ++i)
#pragma unroll
      for (int jj = 0; jj < kGemvRows; ++jj) {
        const size_t row = static_cast<size_t>(kGemvRows * g + jj);
        q[jj][i] = load_nt(wbase + row * (K / 2) + 1024 * i);
      }
  };
  float acc = 0.f;
  auto finish = [&](int j, const uint4 (&q)[kGemvRows][kSlices], const uint32_t (&sd)[2][kSlices]) {
    const uint4* src = h_lds + j * kRow16 + 4 * lane;
    float v[kGemvRows];
    gemv_dot8_halves<kSlices>(
        q, [&](int r, int i) { return gemv_scale_byte(sd[r >> 2][i], r, lane); },
        [&](int i, int c) { return src[i * (kGemvSlice / 8) + c]; }, v);
    const float sum = gemv_reduce8(v, lane);
    if (expert_of(j) < 0) return;   // uniform over the wavefront
    const uint16_t b = f32_to_bf16_bits(sum);
    const float w = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lane_w), j));
    acc = fmaf(w, bf16_bits_to_f32(b), acc);
    if (stores) y_sorted[static_cast<int64_t>(row_of(j)) * ld_out + kGemvRows * g + idx] = b;
  };

  // the token's k rows of h (zeros for an invalid choice) into LDS, their loads
  // issued ahead of the first two choices' weight loads
  uint4 st[kTop][kRow16 / 256];
#pragma unroll
  for (int j = 0; j < k_top; ++j) {
    const int row = expert_of(j) >= 0 ? row_of(j) : 0;
    const uint4* src = reinterpret_cast<const uint4*>(h + static_cast<int64_t>(row) * K);
#pragma unroll
    for (int c = 0; c < kRow16 / 256; ++c) st[j][c] = src[256 * c + threadIdx.x];
  }
  uint4 qa[kGemvRows][kSlices], qb[kGemvRows][kSlices];
  uint32_t sa[2][kSlices], sbb[2][kSlices];
  load_w(expert_of(0), qa, sa);
  if (k_top > 1) load_w(expert_of(1), qb, sbb);
#pragma unroll
  for (int j = 0; j < k_top; ++j) {
    const bool ok = expert_of(j) >= 0;
#pragma unroll
    for (int c = 0; c < kRow16 / 256; ++c)
      h_lds[j * kRow16 + 256 * c + threadIdx.x] = ok ? st[j][c] : make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  // choice j computed while choice j + 1's loads are in flight (k is a template
  // argument so that the loop unrolls and every wait counts only older loads)
#pragma unroll
  for (int j = 0; j < k_top; ++j) {
    if (j % 2 == 0) {
      finish(j, qa, sa);
      if (j + 2 < k_top) load_w(expert_of(j + 2), qa, sa);
    } else {
      finish(j, qb, sbb);
      if (j + 2 < k_top) load_w(expert_of(j + 2), qb, sbb);
    }
  }
  if (stores)
    y[static_cast<int64_t>(t) * ld_out + kGemvRows * g + idx] = f32_to_bf16_bits(acc);
}

template <bool kW1, int kSlices>
hipError_t launch_gemv_t(unsigned grid, hipStream_t stream, const uint16_t* act,
                         const int32_t* gather, int k_top, int n_slots, const uint8_t* wq,
                         const uint8_t* wsc, const RowTile* tiles, const int32_t* n_tiles,
                         int n_rows, int half, int groups, int wpt, float limit, int clamp,
                         uint16_t* out, int ld_out) {
  gemv_kernel<kW1, kSlices><<<grid, 256, 0, stream>>>(act, gather, k_top, n_slots, wq, wsc, tiles,
                                                      n_tiles, n_rows, half, groups, wpt, limit,
                                                      clamp, out, ld_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(bool w1, int64_t tile_bound, hipStream_t stream, const uint16_t* act,
                       const int32_t* gather, int k_top, int n_slots, const uint8_t* wq,
                       const uint8_t* wsc, const RowTile* tiles, const int32_t* n_tiles, int K,
                       int n_rows, int half, float limit, int clamp, uint16_t* out, int ld_out) {
  // groups of 8 weight rows per tile (W1: 4 gate rows and their up rows; a power of
  // two, 256 to 1024, at the GEMV sizes), and wavefronts per tile: the largest power
  // of two within kGemvMaxWaves over the possible tiles and within half the groups
  // (at least 4: a workgroup's wavefronts share a tile), so that every wavefront
  // gets an even number of groups
  const int groups = w1 ? half / 4 : n_rows / kGemvRows;
  if (groups < 8 || (groups & (groups - 1)) != 0) return hipErrorInvalidValue;
  int64_t wpt_max = kGemvMaxWaves / (tile_bound > 0 ? tile_bound : 1);
  if (wpt_max > groups / 2) wpt_max = groups / 2;   // two groups or more per wavefront
  int64_t wpt = 4;
  while (wpt * 2 <= wpt_max) wpt *= 2;
  const int64_t waves = tile_bound * wpt;
  const unsigned grid = static_cast<unsigned>((waves + 3) / 4);
  if (grid == 0) return hipSuccess;
  const int w = static_cast<int>(wpt);
  const bool two = K == 2 * kGemvSlice;
  if (w1)
    return two ? launch_gemv_t<true, 2>(grid, stream, act, gather, k_top, n_slots, wq, wsc, tiles,
                                        n_tiles, n_rows, half, groups, w, limit, clamp, out, ld_out)
               : launch_gemv_t<true, 1>(grid, stream, act, gather, k_top, n_slots, wq, wsc, tiles,
                                        n_tiles, n_rows, half, groups, w, limit, clamp, out, ld_out);
  return two ? launch_gemv_t<false, 2>(grid, stream, act, gather, k_top, n_slots, wq, wsc, tiles,
                                       n_tiles, n_rows, half, groups, w, limit, clamp, out, ld_out)
             : launch_gemv_t<false, 1>(grid, stream, act, gather, k_top, n_slots, wq, wsc, tiles,
                                       n_tiles, n_rows, half, groups, w, limit, clamp, out, ld_out);
}

namespace {

template <int kSlices, int kTop>
void launch_w2c(unsigned grid, hipStream_t stream, const uint16_t* h, const int32_t* ids,
                const float* topw, const int32_t* scatter, int T, int E, int n_slots,
                const uint8_t* wq, const uint8_t* wsc, int n_rows, int per_token,
                uint16_t* y_sorted, uint16_t* y) {
  gemv_w2_combine_kernel<kSlices, kTop><<<grid, 256, 0, stream>>>(
      h, ids, topw, scatter, T, E, n_slots, wq, wsc, n_rows, per_token, y_sorted, y, n_rows);
}

template <int kSlices>
void launch_w2c_k(int k_top, unsigned grid, hipStream_t stream, const uint16_t* h,
                  const int32_t* ids, const float* topw, const int32_t* scatter, int T, int E,
                  int n_slots, const uint8_t* wq, const uint8_t* wsc, int n_rows, int per_token,
                  uint16_t* y_sorted, uint16_t* y) {
#define MOE_W2C(KT)                                                                          \
  case KT:                                                                                   \
    launch_w2c<kSlices, KT>(grid, stream, h, ids, topw, scatter, T, E, n_slots, wq, wsc,     \
                            n_rows, per_token, y_sorted, y);                                 \
    break;
  switch (k_top) {
    MOE_W2C(1) MOE_W2C(2) MOE_W2C(3) MOE_W2C(4) MOE_W2C(5) MOE_W2C(6) MOE_W2C(7) MOE_W2C(8)
  }
#undef MOE_W2C
}

}  // namespace

hipError_t launch_gemv_w2_combine(int64_t T, int k_top, int E, int n_slots, hipStream_t stream,
                                  const uint16_t* h, const int32_t* ids, const float* topw,
                                  const int32_t* scatter, const uint8_t* wq, const uint8_t* wsc,
                                  int K, int n_rows, uint16_t* y_sorted, uint16_t* y) {
  static_assert(kMaxK == 8, "one instantiation per k");
  if (k_top < 1 || k_top > kMaxK) return hipErrorInvalidValue;
  // four wavefronts (32 columns) per workgroup; the token's k rows of h in LDS
  // (at most 8 rows of 8 KB)
  const int per_token = n_rows / (4 * kGemvRows);
  const unsigned grid = static_cast<unsigned>(T * per_token);
  if (grid == 0) return hipSuccess;
  const int t = static_cast<int>(T);
  if (K == 2 * kGemvSlice)
    launch_w2c_k<2>(k_top, grid, stream, h, ids, topw, scatter, t, E, n_slots, wq, wsc, n_rows,
                    per_token, y_sorted, y);
  else
    launch_w2c_k<1>(k_top, grid, stream, h, ids, topw, scatter, t, E, n_slots, wq, wsc, n_rows,
                    per_token, y_sorted, y);
  return hipGetLastError();
}

}  // namespace moe
