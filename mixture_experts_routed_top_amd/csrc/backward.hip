// Elementwise and small steps of the routed-expert MoE backward (BF16 path;
// the pages' follow-up work: Liger-Kernel PR #1463, MoEBenchmark results,
// forward and backward).
//
//   (both per-row kernels cover the rows of the num_tiles tiles only)
//   combine backward: for each sorted row r holding assignment a = (t, j):
//     dY[r, :] = bf16( w[t, j] * dout[t, :] )          (pad rows: 0)
//     dw[t, j] = sum_c dout[t, c] * Y[a, c]             (fp32, one wave per row)
//   routing backward: dlogits[t, e] = w_e (dw_e - sum_j w_j dw_j) for the
//     selected routed experts (softmax over the selected logits), or
//     dw_e w_e (1 - w_e) (sigmoid); 0 for every other expert
//   row gather: x_sorted[r, :] = x[a / k, :] (pad rows: 0), the token operand
//     of the W1 weight gradient in sorted-row order
#include "moe_common.cuh"
#include "moe_launch.h"

namespace moe {

namespace {

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// 16 bytes of a row that is read once: a non-temporal load keeps it from
// displacing lines that are read again (dout, read by all k rows of a token)
__device__ __forceinline__ uint4 load_stream(const uint16_t* p) {
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// one wave per sorted row; each lane handles 8 consecutive columns per pass
__global__ __launch_bounds__(256) void backward_combine_kernel(const uint16_t* __restrict__ dout,
                                                               const float* __restrict__ w,
                                                               const uint16_t* __restrict__ y,
                                                               const int32_t* __restrict__ sorted_ids,
                                                               const int32_t* __restrict__ num_tiles,
                                                               int block_m, int64_t A, int kk, int H,
                                                               uint16_t* __restrict__ dy, float* __restrict__ dw) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= static_cast<int64_t>(*num_tiles) * block_m) return;   // rows no tile covers
  const int a = sorted_ids[r];
  uint16_t* dyr = dy + r * H;
  if (a >= A) {
    for (int c = lane * 8; c < H; c += 512) *reinterpret_cast<uint4*>(dyr + c) = make_uint4(0, 0, 0, 0);
    return;
  }
  const int64_t t = a / kk;
  const float wa = w[a];
  const uint16_t* dr = dout + t * H;
  const uint16_t* yr = y + static_cast<int64_t>(a) * H;
  float dot = 0.0f;
  // unrolled so that several 16-byte loads per lane are in flight
#pragma unroll 4
  for (int c = lane * 8; c < H; c += 512) {
    const uint4 dq = *reinterpret_cast<const uint4*>(dr + c);
    const uint4 yq = load_stream(yr + c);
    const uint32_t dv[4] = {dq.x, dq.y, dq.z, dq.w}, yv[4] = {yq.x, yq.y, yq.z, yq.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float d0 = __uint_as_float(dv[i] << 16), d1 = __uint_as_float(dv[i] & 0xFFFF0000u);
      const float y0 = __uint_as_float(yv[i] << 16), y1 = __uint_as_float(yv[i] & 0xFFFF0000u);
      dot = __builtin_fmaf(d0, y0, dot);
      dot = __builtin_fmaf(d1, y1, dot);
      o[i] = pack_bf16x2(wa * d0, wa * d1);
    }
    *reinterpret_cast<uint4*>(dyr + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off);
  if (lane == 0) dw[a] = dot;
}

// one wave per token: lane j < k holds slot j; the weighted sum over the
// slots is formed once (in slot order, fused multiply-adds, as the per-slot
// formula reads), and each lane writes its experts' entries of the row
// (the gradient of the slot that selected the expert, else 0)
__global__ __launch_bounds__(256) void route_backward_kernel(const float* __restrict__ w,
                                                             const int32_t* __restrict__ ids,
                                                             const float* __restrict__ dw, int64_t T, int E,
                                                             int k, int kk, int score,
                                                             float* __restrict__ dlogits) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;   // whole wave
  const bool slot = lane < k;
  const float wj = slot ? w[t * kk + lane] : 0.0f;
  const float dwj = slot ? dw[t * kk + lane] : 0.0f;
  const int ej = slot ? ids[t * kk + lane] : -1;
  // lane reads (the slot index is wave-uniform)
  auto lane_f = [](float v, int j) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j)); };
  float g = 0.0f;
  if (score == 0) {
    float s = 0.0f;
    for (int q = 0; q < k; ++q) s = __builtin_fmaf(lane_f(wj, q), lane_f(dwj, q), s);
    g = wj * (dwj - s);
  } else {
    g = dwj * wj * (1.0f - wj);
  }
  float* row = dlogits + t * E;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    float v = 0.0f;
    for (int j = 0; j < k; ++j)
      if (__builtin_amdgcn_readlane(ej, j) == e) v = lane_f(g, j);
    if (e < E) row[e] = v;
  }
}

// one wave per sorted row
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ x,
                                                          const int32_t* __restrict__ sorted_ids,
                                                          const int32_t* __restrict__ num_tiles, int block_m,
                                                          int64_t A, int kk, int H, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= static_cast<int64_t>(*num_tiles) * block_m) return;   // rows no tile covers
  const int a = sorted_ids[r];
  uint16_t* o = out + r * H;
  if (a >= A) {
    for (int c = lane * 8; c < H; c += 512) *reinterpret_cast<uint4*>(o + c) = make_uint4(0, 0, 0, 0);
    return;
  }
  const uint16_t* src = x + static_cast<int64_t>(a / kk) * H;
#pragma unroll 4
  for (int c = lane * 8; c < H; c += 512)
    *reinterpret_cast<uint4*>(o + c) = *reinterpret_cast<const uint4*>(src + c);
}

}  // namespace

hipError_t launch_backward_combine(const uint16_t* dout, const float* w, const uint16_t* y,
                                   const int32_t* sorted_ids, const int32_t* num_tiles, int block_m, int64_t A,
                                   int kk, int H, int64_t cap, uint16_t* dy, float* dw, hipStream_t s) {
  backward_combine_kernel<<<static_cast<unsigned>((cap + 3) / 4), 256, 0, s>>>(dout, w, y, sorted_ids, num_tiles,
                                                                               block_m, A, kk, H, dy, dw);
  return hipGetLastError();
}

hipError_t launch_route_backward(const float* w, const int32_t* ids, const float* dw, int64_t T, int E, int k,
                                 int kk, int score, float* dlogits, hipStream_t s) {
  route_backward_kernel<<<static_cast<unsigned>((T + 3) / 4), 256, 0, s>>>(w, ids, dw, T, E, k, kk, score,
                                                                           dlogits);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const uint16_t* x, const int32_t* sorted_ids, const int32_t* num_tiles, int block_m,
                              int64_t A, int kk, int H, int64_t cap, uint16_t* out, hipStream_t s) {
  gather_rows_kernel<<<static_cast<unsigned>((cap + 3) / 4), 256, 0, s>>>(x, sorted_ids, num_tiles, block_m, A, kk,
                                                                          H, out);
  return hipGetLastError();
}

}  // namespace moe
