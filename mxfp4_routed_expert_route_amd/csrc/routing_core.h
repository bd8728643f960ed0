// Device routines shared by the routing kernels (separate and fused).
#pragma once
#include "device.h"

namespace moe {

// ---------------------------------------------------------------- top-k of one token
//
// Selection rule (txtmix.com article, §1 and §3: top-6 of 256 experts per token,
// the "fast DeepSeek routing" step): the k largest logits, ordered by logit
// descending then expert index ascending; -0.0 ranks equal to +0.0.  Weights:
// softmax over the k chosen logits.
//
// Each lane holds EPL logits (expert e = i*64 + lane, coalesced loads) as
// order-preserving 32-bit keys.  k rounds of a wave-wide maximum take the
// winners in order, a tie going to the lower index (the first set lane of the
// first non-empty ballot); the winner's key is retired in the lane that holds
// it.  Lane j < k returns slot j's id and weight.

__device__ __forceinline__ uint32_t order_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;   // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_bits_to_f32(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Wave-wide unsigned maximum through DPP (every lane active): prefix maxima
// within each row of 16 lanes by row shifts of 1, 2, 4, 8, then row broadcasts of
// lanes 15 and 31 carry them across rows, so lane 63 holds the maximum, returned as
// a wave-uniform value.  Six VALU steps, against six LDS round trips for a
// butterfly of lane shuffles.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v),
                                                           kCtrl, kRowMask, 0xF, false));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  uint32_t o;
  o = dpp_u32<0x111, 0xF>(v); v = o > v ? o : v;   // row_shr:1
  o = dpp_u32<0x112, 0xF>(v); v = o > v ? o : v;   // row_shr:2
  o = dpp_u32<0x114, 0xF>(v); v = o > v ? o : v;   // row_shr:4
  o = dpp_u32<0x118, 0xF>(v); v = o > v ? o : v;   // row_shr:8
  o = dpp_u32<0x142, 0xA>(v); v = o > v ? o : v;   // row_bcast:15 into rows 1 and 3
  o = dpp_u32<0x143, 0xC>(v); v = o > v ? o : v;   // row_bcast:31 into rows 2 and 3
  return __builtin_amdgcn_readlane(v, 63);
}

template <int EPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k, int lane,
                                            int& my_id, float& my_weight) {
  // key[i]: order-preserving bits of expert i*64 + lane's logit, 0 (below every
  // real key) past E or once taken.  Each round takes the wave-wide maximum key,
  // then the lowest expert index holding it: expert e = i*64 + lane, so that is
  // the first set lane of the first non-empty ballot over i -- the same order as
  // a maximum over (key << 32 | ~e), with one 32-bit reduction instead of two.
  uint32_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = i * 64 + lane;
    key[i] = e < E ? order_bits(row[e]) : 0u;
  }
  my_id = 0;
  float my_logit = 0.f, top = 0.f;
  for (int j = 0; j < k; ++j) {
    uint32_t mine = key[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) mine = key[i] > mine ? key[i] : mine;
    const uint32_t best = wave_max_u32(mine);   // wave-uniform
    int e_best = 0;
#pragma unroll
    for (int i = EPL - 1; i >= 0; --i) {   // the lowest i with a holder wins
      const uint64_t m = __builtin_amdgcn_ballot_w64(key[i] == best);
      if (m != 0ull) e_best = i * 64 + static_cast<int>(__builtin_ctzll(m));
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (i * 64 + lane == e_best) key[i] = 0u;
    const float l = order_bits_to_f32(best);
    if (j == 0) top = l;
    if (lane == j) {
      my_id = e_best;
      my_logit = l;
    }
  }
  // softmax over the selection: fp32 exponentials, fp64 sum in j order
  const float ex = (lane < k) ? expf(my_logit - top) : 0.f;
  double sum = 0.0;
  for (int j = 0; j < k; ++j)   // lane j's exponential, read as a scalar
    sum += static_cast<double>(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j)));
  my_weight = static_cast<float>(static_cast<double>(ex) / sum);
}

// ---------------------------------------------------------------- expert column masks
//
// For a wavefront of 64 consecutive tokens (one per lane): for every expert e, a
// ballot of "my token's bit e is set" is the 64-bit column mask of e over those
// tokens.  Lane (e mod 64) collects that mask, so a group of 64 experts costs
// about five instructions per expert and one 64-bit store per lane.  From the
// masks: count of e = popcount(mask[e]); rank of a token among e's tokens =
// popcount(mask[e] & lanes-below-it), which orders an expert's rows by token.

// The LLVM writelane intrinsic (v_writelane_b32), which this clang does not expose
// as a builtin.  Going through the intrinsic, rather than inline assembly, lets
// the compiler see the instruction and insert the wait state it needs after a
// VALU write of the SGPR it reads (the ballot's compare).
extern "C" __device__ int llvm_amdgcn_writelane(int src, int lane, int old)
    __asm("llvm.amdgcn.writelane.i32");

template <int kLane>
__device__ __forceinline__ uint32_t write_lane(uint32_t v, uint32_t s) {
  return static_cast<uint32_t>(
      llvm_amdgcn_writelane(static_cast<int>(s), kLane, static_cast<int>(v)));
}

template <int kBase, int kBit = 0>
__device__ __forceinline__ void collect_word(uint32_t word, uint32_t& lo, uint32_t& hi) {
  if constexpr (kBit < 32) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(((word >> kBit) & 1u) != 0u);
    lo = write_lane<kBase + kBit>(lo, static_cast<uint32_t>(m));
    hi = write_lane<kBase + kBit>(hi, static_cast<uint32_t>(m >> 32));
    collect_word<kBase, kBit + 1>(word, lo, hi);
  }
}

// masks[e] for the 64 experts of bit-matrix words w0, w0+1 (this lane's token's
// words word0, word1).
__device__ __forceinline__ void column_masks_words(uint32_t word0, uint32_t word1, int E,
                                                   int lane, uint64_t* masks, int w0) {
  uint32_t lo = 0u, hi = 0u;
  collect_word<0>(word0, lo, hi);
  collect_word<32>(word1, lo, hi);
  const int e = w0 * 32 + lane;
  if (e < E) masks[e] = (static_cast<uint64_t>(hi) << 32) | lo;
}

// masks[e] for the 64 experts of bit-matrix words w0, w0+1, for the token of this
// lane (t, valid = t < T).
__device__ __forceinline__ void column_masks_64(const uint32_t* bm, int64_t t, bool valid, int E,
                                                int words, int lane, uint64_t* masks, int w0) {
  const uint32_t word0 = valid ? bm[t * words + w0] : 0u;
  const uint32_t word1 = (valid && w0 + 1 < words) ? bm[t * words + w0 + 1] : 0u;
  column_masks_words(word0, word1, E, lane, masks, w0);
}

// masks[e] <- column mask of expert e over rows[t0 .. t0+63] (rows past T are empty).
// `bm` points at row 0 of a [T][words] bit matrix (global or LDS).
__device__ __forceinline__ void wave_column_masks(const uint32_t* bm, int64_t t0, int64_t T, int E,
                                                  int words, int lane, uint64_t* masks) {
  const int64_t t = t0 + lane;
  const bool valid = t < T;
  if (t0 >= T) {   // no token in this wavefront
    for (int e = lane; e < E; e += 64) masks[e] = 0ull;
    return;
  }
  if (words <= 8) {
    // up to 256 experts: the token's words are loaded together (one memory
    // latency, not one per pair of words)
    uint32_t wd[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) wd[i] = valid && i < words ? bm[t * words + i] : 0u;
#pragma unroll
    for (int w0 = 0; w0 < 8; w0 += 2)
      if (w0 < words) column_masks_words(wd[w0], wd[w0 + 1], E, lane, masks, w0);
    return;
  }
  for (int w0 = 0; w0 < words; w0 += 2) column_masks_64(bm, t, valid, E, words, lane, masks, w0);
}

// Exclusive scan of one value per thread over the workgroup (blockDim.x <= 1024).
__device__ __forceinline__ int block_exclusive_scan(int v, int* __restrict__ wave_tot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) {
    const int tw = wave_tot[w];
    before += w < wave ? tw : 0;
    all += tw;
  }
  *total = all;
  return before + incl - v;
}

}  // namespace moe
