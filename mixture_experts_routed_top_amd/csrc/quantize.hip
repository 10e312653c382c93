// Quantisers: bf16 -> FP8 E4M3 with fp32 block scales (1x128 activations,
// 128x128 weights; TileScale PR #70, Design), and bf16 -> MXFP8 / MXFP4 with
// one E8M0 scale per 32 elements along a row (FlashInfer PR #6465, Benchmark
// configuration; scale rule of the OCP MX v1.0 specification).
//
// FP8 rule per block: amax = max|v|, s = fp32(amax / 448) correctly rounded
// (s = 1 for an all-zero block), code = E4M3_RN(clamp(fp32(v / s))).
// MX rule per 32-block: X = 2^(floor(log2 amax) - emax) with emax = 8 (E4M3)
// or 2 (E2M1), clamped exponent, byte = exponent + 127 (0 for an all-zero
// block); code = RN_SAT(v / X), the division exact (a power of two).
#include "moe_common.cuh"
#include "moe_launch.h"

namespace moe {

namespace {

__device__ __forceinline__ void unpack8(const uint4& q, float v[8]) {
  const uint32_t p[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(p[i] << 16);
    v[2 * i + 1] = __uint_as_float(p[i] & 0xFFFF0000u);
  }
}

// 1 x 128 blocks: 16 threads per block, 8 elements (16 bytes) each.
__global__ __launch_bounds__(256) void quant_fp8_row_kernel(const uint16_t* __restrict__ in, int64_t rows,
                                                            int64_t cols, uint8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
  const int64_t groups = rows * (cols / 128);
  const int sub = threadIdx.x & 15;
  for (int64_t g = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) >> 4; g < groups;
       g += (static_cast<int64_t>(gridDim.x) * 256) >> 4) {
    const int64_t off = g * 128 + sub * 8;  // row-major: group g covers 128 consecutive elements
    float v[8];
    unpack8(*reinterpret_cast<const uint4*>(in + off), v);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
    amax = group_max<16>(amax);
    const float s = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    uint2 o;
    o.x = pack_e4m3x4(__fdiv_rn(v[0], s), __fdiv_rn(v[1], s), __fdiv_rn(v[2], s), __fdiv_rn(v[3], s));
    o.y = pack_e4m3x4(__fdiv_rn(v[4], s), __fdiv_rn(v[5], s), __fdiv_rn(v[6], s), __fdiv_rn(v[7], s));
    *reinterpret_cast<uint2*>(q + off) = o;
    if (sub == 0) scale[g] = s;
  }
}

// 128 x 128 blocks: one workgroup per block; each thread holds 8 rows x 8 columns.
__global__ __launch_bounds__(256) void quant_fp8_tile_kernel(const uint16_t* __restrict__ in, int64_t rows,
                                                             int64_t cols, uint8_t* __restrict__ q,
                                                             float* __restrict__ scale) {
  __shared__ float red[4];
  const int64_t bc = cols / 128;
  const int64_t br = blockIdx.x / bc, bcol = blockIdx.x % bc;
  const int tid = threadIdx.x;
  const int col = static_cast<int>(bcol * 128) + (tid & 15) * 8;
  float v[8][8];
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int64_t r = br * 128 + (tid >> 4) + 16 * p;
    unpack8(*reinterpret_cast<const uint4*>(in + r * cols + col), v[p]);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[p][i]));
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  const float s = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int64_t r = br * 128 + (tid >> 4) + 16 * p;
    uint2 o;
    o.x = pack_e4m3x4(__fdiv_rn(v[p][0], s), __fdiv_rn(v[p][1], s), __fdiv_rn(v[p][2], s),
                      __fdiv_rn(v[p][3], s));
    o.y = pack_e4m3x4(__fdiv_rn(v[p][4], s), __fdiv_rn(v[p][5], s), __fdiv_rn(v[p][6], s),
                      __fdiv_rn(v[p][7], s));
    *reinterpret_cast<uint2*>(q + r * cols + col) = o;
  }
  if (tid == 0) scale[blockIdx.x] = s;
}

// 1 x 32 MX blocks: 4 threads per block, 8 elements each.
template <bool FP4>
__global__ __launch_bounds__(256) void quant_mx_kernel(const uint16_t* __restrict__ in, int64_t rows,
                                                       int64_t cols, uint8_t* __restrict__ q,
                                                       uint8_t* __restrict__ e8m0) {
  const int64_t groups = rows * (cols / 32);
  const int sub = threadIdx.x & 3;
  for (int64_t g = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) >> 2; g < groups;
       g += (static_cast<int64_t>(gridDim.x) * 256) >> 2) {
    const int64_t off = g * 32 + sub * 8;
    float v[8];
    unpack8(*reinterpret_cast<const uint4*>(in + off), v);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
    amax = group_max<4>(amax);
    const int x = mx_scale_exponent(amax, FP4 ? 2 : 8);
    const float inv = mx_inv_scale(x);
    if (FP4) {
      uint32_t o = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) o |= e2m1_code(v[i] * inv) << (4 * i);
      *reinterpret_cast<uint32_t*>(q + off / 2) = o;
    } else {
      uint2 o;
      o.x = pack_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
      o.y = pack_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
      *reinterpret_cast<uint2*>(q + off) = o;
    }
    if (sub == 0) e8m0[g] = static_cast<uint8_t>(x + 127);
  }
}

unsigned grid_for(int64_t threads) {
  int64_t b = (threads + 255) / 256;
  if (b > 65536) b = 65536;
  return static_cast<unsigned>(b < 1 ? 1 : b);
}

}  // namespace

hipError_t launch_quantize_fp8(const uint16_t* in, int64_t rows, int64_t cols, int block_rows, uint8_t* q,
                               float* scale, hipStream_t s) {
  if (block_rows == 1) {
    quant_fp8_row_kernel<<<grid_for(rows * (cols / 128) * 16), 256, 0, s>>>(in, rows, cols, q, scale);
  } else {
    const int64_t blocks = (rows / 128) * (cols / 128);
    quant_fp8_tile_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(in, rows, cols, q, scale);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_mx(const uint16_t* in, int64_t rows, int64_t cols, bool fp4, uint8_t* q,
                              uint8_t* e8m0, hipStream_t s) {
  const unsigned grid = grid_for(rows * (cols / 32) * 4);
  if (fp4) quant_mx_kernel<true><<<grid, 256, 0, s>>>(in, rows, cols, q, e8m0);
  else quant_mx_kernel<false><<<grid, 256, 0, s>>>(in, rows, cols, q, e8m0);
  return hipGetLastError();
}

}  // namespace moe
