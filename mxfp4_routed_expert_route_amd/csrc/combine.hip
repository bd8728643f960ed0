// Weighted combine back to token order:
//   y[t][n] = sum_j w[t][j] * y_sorted[scatter[t*k+j]][n],  fp32 in j order, one bf16 rounding.
// A thread owns 8 consecutive columns (one 16-byte load per expert row); a
// workgroup of 256 threads covers 2048 columns of one token.  When y_sorted is
// larger than the 256 MB last-level cache (MALL) it cannot still be there from
// the W2 kernel, and its rows are read with non-temporal loads (measured on the
// 8,191-token skewed batch, 403 MB: 92.5 -> 79.3 us; on the 2,048-token batch,
// 101 MB, normal loads are faster: 20.8 against 21.6 us).
#include "config.h"
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool kNt>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ ys,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ scatter,
                                                      int64_t T, int H, int k, int chunks,
                                                      uint16_t* __restrict__ y) {
  const int64_t t = blockIdx.x / chunks;
  const int c = blockIdx.x - static_cast<int>(t) * chunks;
  const int col = (c * 256 + threadIdx.x) * 8;
  if (t >= T || col >= H) return;
  const int64_t n_slots = T * k;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  // all k rows' positions and weights, then all k row loads, then the sum in j
  // order: one dependent pair of memory latencies instead of k (k <= kMaxK)
  int64_t p[kMaxK];
  float wj[kMaxK];
  bool ok[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    ok[j] = false;
    if (j < k) {
      p[j] = scatter[t * k + j];
      wj[j] = w[t * k + j];
      ok[j] = p[j] >= 0 && p[j] < n_slots;
    }
  }
  uint4 v[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (ok[j]) {
      const uint16_t* src = ys + p[j] * H + col;
      if constexpr (kNt) {
        const u32x4 d = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
        v[j] = make_uint4(d.x, d.y, d.z, d.w);
      } else {
        v[j] = *reinterpret_cast<const uint4*>(src);
      }
    }
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (!ok[j]) continue;
    const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = fmaf(wj[j], bf16_bits_to_f32(u[i] & 0xFFFFu), acc[2 * i]);
      acc[2 * i + 1] = fmaf(wj[j], bf16_bits_to_f32(u[i] >> 16), acc[2 * i + 1]);
    }
  }
  uint4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(y + t * H + col) = o;
}

}  // namespace

hipError_t launch_combine(const uint16_t* ys, const float* w, const int32_t* scatter, int64_t T,
                          int H, int k, uint16_t* y, hipStream_t stream) {
  const int chunks = (H + 2047) / 2048;
  const dim3 grid(static_cast<unsigned>(T * chunks));
  const int64_t ys_bytes = T * k * static_cast<int64_t>(H) * 2;
  if (ys_bytes > (static_cast<int64_t>(256) << 20))
    combine_kernel<true><<<grid, dim3(256), 0, stream>>>(ys, w, scatter, T, H, k, chunks, y);
  else
    combine_kernel<false><<<grid, dim3(256), 0, stream>>>(ys, w, scatter, T, H, k, chunks, y);
  return hipGetLastError();
}

}  // namespace moe
