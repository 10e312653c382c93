// Top-k weighted combine: out[t, :] = bf16( sum_j w[t, j] * y[t*k + j, :] ).
// TileScale PR #70, review thread on the reduce tail (per-token sum over the
// top-k slots into the BF16 output); FlashInfer PR #5129, Description.
//
// Purely bandwidth bound: each thread owns 8 consecutive columns of one token
// (16-byte loads of every slot row, one 16-byte store), consecutive threads
// own consecutive columns, so each wave reads 1 KB contiguous per slot row.
// The sum runs in fp32 in slot order with one fused multiply-add per slot.
#include "moe_common.cuh"
#include "moe_launch.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const float* __restrict__ w, int64_t T, int k,
                                                      int H, uint16_t* __restrict__ out) {
  const int vpr = H >> 3;  // 8-column vectors per row
  const int64_t total = T * vpr;
  for (int64_t v = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; v < total;
       v += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t t = v / vpr;
    const int c = static_cast<int>(v - t * vpr) << 3;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    const uint16_t* yrow = y + (t * k) * H + c;
    for (int j = 0; j < k; ++j) {
      const float wj = w[t * k + j];
      const uint4 q = *reinterpret_cast<const uint4*>(yrow + static_cast<int64_t>(j) * H);
      const uint32_t p[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __builtin_fmaf(wj, __uint_as_float(p[i] << 16), acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(wj, __uint_as_float(p[i] & 0xFFFF0000u), acc[2 * i + 1]);
      }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(out + t * H + c) = o;
  }
}

}  // namespace

hipError_t launch_combine(const uint16_t* y, const float* w, int64_t T, int k, int H, uint16_t* out,
                          const DeviceInfo& dev, hipStream_t s) {
  const int64_t total = T * (H >> 3);
  int64_t blocks = (total + 255) / 256;
  const int64_t cap = static_cast<int64_t>(dev.num_cus) * 16;
  if (blocks > cap) blocks = cap;
  combine_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(y, w, T, k, H, out);
  return hipGetLastError();
}

}  // namespace moe
