// Activations to the two-part FP8 form read by the tiled FFN's block-scaled MFMAs
// (the format is described at a8_pos in ffn_common.h): the work of one thread, one
// 32-element block of a row.  It reads the block's 64 bytes of bf16, derives the
// block's E8M0 scale from its largest magnitude, and writes the 32 hi and 32 lo
// bytes (two 16-byte runs each, at the block's positions in the chunk's lane
// order) and the scale byte.  Used by act_split_kernel and, in the one-call layer,
// by the extra workgroups of the routing launch.
#pragma once

#include "ffn_common.h"

namespace moe {

__device__ __forceinline__ void act_split_block(const uint16_t* __restrict__ x, int64_t bid,
                                                int K, uint8_t* __restrict__ xq,
                                                uint8_t* __restrict__ xs) {
  const int bpr = K / 32;   // blocks per row
  const int64_t row = bid / bpr;
  const int b = static_cast<int>(bid - row * bpr);
  const uint4* src = reinterpret_cast<const uint4*>(x + row * K + 32 * b);
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 d = src[i];
    w[4 * i + 0] = d.x; w[4 * i + 1] = d.y; w[4 * i + 2] = d.z; w[4 * i + 3] = d.w;
  }
  float v[32];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    const uint32_t a0 = __float_as_uint(v[2 * i]) & 0x7FFFFFFFu;
    const uint32_t a1 = __float_as_uint(v[2 * i + 1]) & 0x7FFFFFFFu;
    m = a0 > m ? a0 : m;   // on magnitudes as integers: NaN bits sort above infinity
    m = a1 > m ? a1 : m;
  }
  const uint32_t s = a8_scale_byte(m);
  const float inv = a8_inv_scale(s);
  uint8_t* dst = xq + row * (2 * static_cast<int64_t>(K)) + (b / 4) * 256;
  const int bb = b % 4;
  // elements 0..15 of the block go to the run at a8_pos(32 bb), 16..31 to a8_pos(32 bb + 16)
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    uint2 h[2], l[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] = v[16 * r + 8 * half + i] * inv;
      a8_split8(t, h[half], l[half]);
    }
    const int pos = a8_pos(32 * bb + 16 * r);
    *reinterpret_cast<uint4*>(dst + pos) = make_uint4(h[0].x, h[0].y, h[1].x, h[1].y);
    *reinterpret_cast<uint4*>(dst + 128 + pos) = make_uint4(l[0].x, l[0].y, l[1].x, l[1].y);
  }
  xs[bid] = static_cast<uint8_t>(s);
}

}  // namespace moe
