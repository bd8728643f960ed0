// Weighted combine back to token order:
//   y[t][n] = sum_j w[t][j] * y_sorted[scatter[t*k+j]][n],  fp32 in j order, one bf16 rounding.
// A thread owns 8 consecutive columns (one 16-byte load per expert row); a
// workgroup of 256 threads covers 2048 columns of one token.
#include "config.h"
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

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
    if (ok[j]) v[j] = *reinterpret_cast<const uint4*>(ys + p[j] * H + col);
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
  combine_kernel<<<dim3(static_cast<unsigned>(T * chunks)), dim3(256), 0, stream>>>(
      ys, w, scatter, T, H, k, chunks, y);
  return hipGetLastError();
}

}  // namespace moe
