// Top-k weighted combine: out[t, :] = bf16( sum_j w[t, j] * y[t*k + j, :] ).
// TileScale PR #70, review thread on the reduce tail (per-token sum over the
// top-k slots into the BF16 output); FlashInfer PR #5129, Description.
//
// Purely bandwidth bound: each thread owns 8 consecutive columns of one token
// (16-byte loads of every slot row, one 16-byte store), consecutive threads
// own consecutive columns, so each wave reads 1 KB contiguous per slot row.
// The sum runs in fp32 in slot order with one fused multiply-add per slot.
// For k up to 10 the slot count is a template argument and every slot row's
// load is issued before the first is used (k loads in flight per thread,
// instead of one load and its full latency per slot). The y rows are read
// once: non-temporal loads keep them from displacing other lines in the
// caches (Qwen3-30B-A3B shape 54.2 -> 49.3 us, FP8 H 7168 shape 208 -> 177
// us; non-temporal stores of the output measured slower and are not used).
#include "moe_common.cuh"
#include "moe_launch.h"

namespace moe {

namespace {

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// 16 bytes of a y row, read once
__device__ __forceinline__ uint4 load_stream(const uint16_t* p) {
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// KS > 0: k == KS, known at compile time; KS == 0: any k
template <int KS>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const float* __restrict__ w, int64_t T, int k_rt,
                                                      int H, uint16_t* __restrict__ out) {
  const int k = KS > 0 ? KS : k_rt;
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
    auto add = [&](float wj, const uint4& q) {
      const uint32_t p[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __builtin_fmaf(wj, __uint_as_float(p[i] << 16), acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(wj, __uint_as_float(p[i] & 0xFFFF0000u), acc[2 * i + 1]);
      }
    };
    if constexpr (KS > 0) {
      uint4 q[KS];
      float wj[KS];
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        q[j] = load_stream(yrow + static_cast<int64_t>(j) * H);
        wj[j] = w[t * KS + j];
      }
#pragma unroll
      for (int j = 0; j < KS; ++j) add(wj[j], q[j]);
    } else {
      for (int j = 0; j < k; ++j) add(w[t * k + j], load_stream(yrow + static_cast<int64_t>(j) * H));
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(out + t * H + c) = o;
  }
}

template <int KS>
void launch_k(const uint16_t* y, const float* w, int64_t T, int k, int H, uint16_t* out, unsigned blocks,
              hipStream_t s) {
  combine_kernel<KS><<<blocks, 256, 0, s>>>(y, w, T, k, H, out);
}

}  // namespace

hipError_t launch_combine(const uint16_t* y, const float* w, int64_t T, int k, int H, uint16_t* out,
                          const DeviceInfo& dev, hipStream_t s) {
  const int64_t total = T * (H >> 3);
  int64_t blocks = (total + 255) / 256;
  const int64_t cap = static_cast<int64_t>(dev.num_cus) * 16;
  if (blocks > cap) blocks = cap;
  const unsigned g = static_cast<unsigned>(blocks);
  switch (k) {
    case 1: launch_k<1>(y, w, T, k, H, out, g, s); break;
    case 2: launch_k<2>(y, w, T, k, H, out, g, s); break;
    case 3: launch_k<3>(y, w, T, k, H, out, g, s); break;
    case 4: launch_k<4>(y, w, T, k, H, out, g, s); break;
    case 5: launch_k<5>(y, w, T, k, H, out, g, s); break;
    case 6: launch_k<6>(y, w, T, k, H, out, g, s); break;
    case 7: launch_k<7>(y, w, T, k, H, out, g, s); break;
    case 8: launch_k<8>(y, w, T, k, H, out, g, s); break;
    case 9: launch_k<9>(y, w, T, k, H, out, g, s); break;
    case 10: launch_k<10>(y, w, T, k, H, out, g, s); break;
    default: launch_k<0>(y, w, T, k, H, out, g, s); break;
  }
  return hipGetLastError();
}

}  // namespace moe
