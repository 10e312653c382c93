// Measurement probe of the gfx950 matrix cores the grouped GEMMs use:
//
//   rate   the issue rate of each MFMA form, every CU busy (two workgroups of
//          four waves per CU, eight independent accumulators per wave), in
//          TFLOP/s: v_mfma_f32_32x32x16_bf16 and the scaled
//          v_mfma_scale_f32_32x32x64_f8f6f4 with FP8 x FP8, FP4 x FP8 and
//          FP4 x FP4 operands. This is what the roofline of the MXFP4-weight
//          GEMMs is priced against: FP4 on one operand only issues at the
//          FP8 rate, so those GEMMs are reported against the FP8 peak.
//   lds    the BF16 GEMMs' inner loop without its operand loads: a
//          workgroup of 8 waves, each wave a 64 x 128 tile (the forward
//          GEMMs' per-wave tile), reads its MFMA fragments (16 bytes a lane)
//          from 128-byte LDS rows, the next 16-K substep's fragments while
//          the current substep's MFMAs run, one barrier per 64-K step; with
//          the 16-byte chunk XOR-swizzled by row & 7 and by (row >> 1) & 7.
//          Also the plain LDS read bandwidth of 16-byte reads. This is the
//          compute side's own ceiling, with operand loads taken out.
//   accum  the accumulation precision of one MFMA: one output is a sum of
//          two large products (equal, or cancelling) and many small ones of
//          magnitude 2^e, C = 0; the result is printed beside the exact sum.
//          Within an aligned group of 8 K elements the hardware adds the
//          products after aligning them to the group's largest, so bits far
//          below it are lost; this sets the rounding bound the parity tests
//          allow each FP8 / MX dot product beyond plain fp32 accumulation.
//
// One JSON line per measurement on stdout. Every kernel touches only its own
// registers and writes one output buffer inside its bounds.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;

#define CK(x)                                                                  \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(1);                                                                 \
    }                                                                          \
  } while (0)

// ------------------------------------------------------------------ issue rate
enum Kind { kBf16 = 0, kFp8Fp8 = 1, kFp4Fp8 = 2, kFp4Fp4 = 3 };
constexpr int kAcc = 8;

template <int KIND>
__global__ __launch_bounds__(256, 2) void rate_kernel(float* out, int iters) {
  f32x16 acc[kAcc];
#pragma unroll
  for (int i = 0; i < kAcc; ++i) acc[i] = f32x16{};
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  i32x8 fa, fb;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(0.001f * (lane + i));
    b[i] = static_cast<__bf16>(0.002f * (lane - i));
    fa[i] = 0x38383838 + lane;
    fb[i] = 0x30303030 + i;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kAcc; ++i) {
      if (KIND == kBf16) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
      if (KIND == kFp8Fp8) acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, acc[i], 0, 0, 0, 127, 0, 127);
      if (KIND == kFp4Fp8) acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, acc[i], 4, 0, 0, 127, 0, 127);
      if (KIND == kFp4Fp4) acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, acc[i], 4, 4, 0, 127, 0, 127);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kAcc; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[i][v];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

template <int KIND>
double rate(int cus, float* out, double flop_per_mfma, double peak, const char* name) {
  const int grid = cus * 2, iters = 4000;
  hipEvent_t a, b;
  CK(hipEventCreate(&a));
  CK(hipEventCreate(&b));
  rate_kernel<KIND><<<grid, 256>>>(out, iters);
  CK(hipDeviceSynchronize());
  float best = 1e30f;
  for (int r = 0; r < 5; ++r) {
    CK(hipEventRecord(a));
    rate_kernel<KIND><<<grid, 256>>>(out, iters);
    CK(hipEventRecord(b));
    CK(hipEventSynchronize(b));
    float ms;
    CK(hipEventElapsedTime(&ms, a, b));
    if (ms < best) best = ms;
  }
  const double tf = grid * 4.0 * iters * kAcc * flop_per_mfma / (best * 1e-3) / 1e12;
  printf("{\"probe\": \"rate\", \"mfma\": \"%s\", \"tflops\": %.1f, \"published_dense_peak_tflops\": %.1f, "
         "\"frac_of_peak\": %.3f}\n", name, tf, peak, tf / peak);
  return tf;
}

// ------------------------------------------------------------------ MFMA + LDS
// Offset of 16-byte chunk c of LDS row `row` (128-byte rows).
template <int SWZ>
__device__ __forceinline__ uint32_t lds_off(int row, int c) {
  const int s = SWZ == 0 ? (row & 7) : ((row >> 1) & 7);
  return static_cast<uint32_t>(row * 128 + ((c ^ s) << 4));
}

// WM x WN waves, each FM x FN 32 x 32 output blocks; LDS holds BM token rows
// and BN weight rows of 64 bf16 (one 64-K step), filled once.
template <int WM, int WN, int FM, int FN, int SWZ>
__global__ __launch_bounds__(64 * WM * WN, 1) void mfma_lds_kernel(float* out, int iters) {
  constexpr int TM = FM * 32, TN = FN * 32, BM = WM * TM, BN = WN * TN;
  constexpr int BYTES = (BM + BN) * 128;
  static_assert(BYTES <= 160 * 1024, "one k-step of both operands fits in LDS");
  __shared__ __attribute__((aligned(1024))) char lds[BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  for (int i = tid; i < BYTES / 4; i += 64 * WM * WN) reinterpret_cast<float*>(lds)[i] = 0.001f * (i & 255);
  __syncthreads();
  const char* tok = lds;
  const char* wgt = lds + BM * 128;
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
    __builtin_amdgcn_s_barrier();
    bf16x8 xf[2][FM], wf[2][FN];
    auto frags = [&](int kk, int buf) {
      const int ch = kk * 2 + (lane >> 5);   // rows < BM / BN, chunk < 8: inside the array
#pragma unroll
      for (int i = 0; i < FM; ++i)
        xf[buf][i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                                    tok + lds_off<SWZ>(wm * TM + i * 32 + (lane & 31), ch)));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        wf[buf][j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                                    wgt + lds_off<SWZ>(wn * TN + j * 32 + (lane & 31), ch)));
    };
    frags(0, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < 4) frags(kk + 1, cur ^ 1);
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cur][j], xf[cur][i], acc[i][j], 0, 0, 0);
    }
    // the next substep's reads interleaved with the current substep's MFMAs
    constexpr int READS = FM + FN, MFMAS = FM * FN, PAIRS = READS < MFMAS ? READS : MFMAS;
    __builtin_amdgcn_sched_group_barrier(0x100, READS, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk + 1 < 4) {
#pragma unroll
        for (int q = 0; q < PAIRS; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if (MFMAS > PAIRS) __builtin_amdgcn_sched_group_barrier(0x008, MFMAS - PAIRS, 0);
        if (READS > PAIRS) __builtin_amdgcn_sched_group_barrier(0x100, READS - PAIRS, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, MFMAS, 0);
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += acc[i][j][v];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// 4 waves, each reading 16 bytes a lane from 32 consecutive 128-byte rows, 8 reads an iteration.
template <int SWZ>
__global__ __launch_bounds__(256, 1) void lds_read_kernel(float* out, int iters) {
  __shared__ __attribute__((aligned(1024))) char lds[512 * 128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 512 * 128 / 4; i += 256) reinterpret_cast<float*>(lds)[i] = 0.001f * (i & 255);
  __syncthreads();
  uint4 s = {0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = (wave * 8 + r) * 32 % 512 + (lane & 31);   // < 512
      const uint4 v = *reinterpret_cast<const uint4*>(lds + lds_off<SWZ>(row, (it & 3) * 2 + (lane >> 5)));
      s.x ^= v.x;
      s.y += v.y;
      s.z ^= v.z;
      s.w += v.w;
    }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = static_cast<float>(s.x + s.y + s.z + s.w);
}

template <class K>
float best_ms(K kernel, int grid, int block, int iters, float* out) {
  hipEvent_t a, b;
  CK(hipEventCreate(&a));
  CK(hipEventCreate(&b));
  kernel<<<grid, block>>>(out, iters);
  CK(hipDeviceSynchronize());
  float best = 1e30f;
  for (int r = 0; r < 5; ++r) {
    CK(hipEventRecord(a));
    kernel<<<grid, block>>>(out, iters);
    CK(hipEventRecord(b));
    CK(hipEventSynchronize(b));
    float ms;
    CK(hipEventElapsedTime(&ms, a, b));
    if (ms < best) best = ms;
  }
  return best;
}

void mfma_lds(int cus, float* out) {
  const int iters = 2000;
  const double flop = 8.0 * 4 * 8 * 32768.0 * iters;   // 8 waves x 4 substeps x 8 MFMAs x 32x32x16x2
  const float m7 = best_ms(mfma_lds_kernel<4, 2, 2, 4, 0>, cus, 512, iters, out);
  const float m1 = best_ms(mfma_lds_kernel<4, 2, 2, 4, 1>, cus, 512, iters, out);
  const char* sw[2] = {"row & 7", "(row >> 1) & 7"};
  const float ms[2] = {m7, m1};
  for (int i = 0; i < 2; ++i) {
    const double tf = cus * flop / (ms[i] * 1e-3) / 1e12;
    printf("{\"probe\": \"mfma_lds\", \"tile\": \"8 waves x 64x128\", \"swizzle\": \"%s\", \"tflops\": %.1f, "
           "\"frac_of_bf16_peak\": %.3f}\n", sw[i], tf, tf / 2516.6);
  }
  const int riters = 20000;
  const float r7 = best_ms(lds_read_kernel<0>, cus, 256, riters, out);
  const float r1 = best_ms(lds_read_kernel<1>, cus, 256, riters, out);
  const float rs[2] = {r7, r1};
  for (int i = 0; i < 2; ++i) {
    const double bytes = cus * 4.0 * 8 * 64 * 16 * riters;
    printf("{\"probe\": \"lds_read_b128\", \"swizzle\": \"%s\", \"tb_s\": %.2f, "
           "\"bytes_per_clock_per_cu_at_2.4GHz\": %.1f}\n", sw[i], bytes / (rs[i] * 1e-3) / 1e12,
           bytes / (rs[i] * 1e-3) / cus / 2.4e9);
  }
}

// ------------------------------------------------------------------ accumulation
// One MFMA, C = 0. Output row 0 (A row 0) sums: big0 and big1 at K = 0, 1 and
// 62 products of the small value at the other K; row 1 sums 64 small products.
// mode 0: FP8 x FP8, A carries the values, B = 1.0 (E4M3 0x38).
// mode 1: FP4 x FP8, A (E2M1) = 6, -6 at K = 0, 1 and 0.5 elsewhere;
//         B (E4M3) = big at K = 0, 1 (so the large products are +-6 big) and
//         the small value elsewhere (products 0.5 small).
// mode 2: BF16 32x32x16 (16 K), A carries the values, B = 1.0: row 0 sums
//         big0, big1 and 14 small.
__global__ void accum_kernel(int mode, uint32_t big0, uint32_t big1, uint32_t small, float* out) {
  const int lane = threadIdx.x;
  f32x16 acc = {};
  if (mode == 2) {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(small));
      b[i] = static_cast<__bf16>(1.0f);
    }
    if (lane == 0) {
      a[0] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(big0));
      a[1] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(big1));
    }
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  } else {
    uint8_t ab[32], bb[32];
    for (int i = 0; i < 32; ++i) {
      ab[i] = mode == 0 ? static_cast<uint8_t>(small) : 0x11;      // E2M1 0.5 in both nibbles
      bb[i] = mode == 0 ? 0x38 : static_cast<uint8_t>(small);
    }
    if (mode == 0 && lane == 0) {
      ab[0] = static_cast<uint8_t>(big0);
      ab[1] = static_cast<uint8_t>(big1);
    }
    if (mode == 1) {
      if (lane == 0) ab[0] = 0xF7;                                 // K0 = 6, K1 = -6
      if (lane < 32) {                                             // K = 0, 1 of every B column
        bb[0] = static_cast<uint8_t>(big0);
        bb[1] = static_cast<uint8_t>(big0);
      }
    }
    i32x8 fa, fb;
    for (int i = 0; i < 8; ++i) {
      fa[i] = ab[4 * i] | (ab[4 * i + 1] << 8) | (ab[4 * i + 2] << 16) | (ab[4 * i + 3] << 24);
      fb[i] = bb[4 * i] | (bb[4 * i + 1] << 8) | (bb[4 * i + 2] << 16) | (bb[4 * i + 3] << 24);
    }
    if (mode == 0) acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, acc, 0, 0, 0, 127, 0, 127);
    else acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, acc, 4, 0, 0, 127, 0, 127);
  }
  // lane 0, registers 0 and 1: rows 0 and 1 of output column 0
  if (lane == 0) {
    out[0] = acc[0];
    out[1] = acc[1];
  }
}

double e4m3(uint32_t c) {
  const int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
  const double v = e == 0 ? m * ldexp(1.0, -9) : (1 + m / 8.0) * ldexp(1.0, e - 7);
  return s ? -v : v;
}

uint32_t e4m3_pow2(int e) { return e < -6 ? (1u << (e + 9)) : static_cast<uint32_t>((e + 7) << 3); }

double bf16v(uint32_t bits) {
  const uint32_t u = bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

void accum(int mode, uint32_t big0, uint32_t big1, uint32_t small, float* dout) {
  accum_kernel<<<1, 64>>>(mode, big0, big1, small, dout);
  CK(hipDeviceSynchronize());
  float h[2];
  CK(hipMemcpy(h, dout, sizeof(h), hipMemcpyDeviceToHost));
  double b0, b1, sm, e0, e1;
  const char* name;
  if (mode == 2) {
    b0 = bf16v(big0), b1 = bf16v(big1), sm = bf16v(small);
    e0 = b0 + b1 + 14 * sm, e1 = 16 * sm, name = "bf16";
  } else if (mode == 0) {
    b0 = e4m3(big0), b1 = e4m3(big1), sm = e4m3(small);
    e0 = b0 + b1 + 62 * sm, e1 = 64 * sm, name = "fp8xfp8";
  } else {
    b0 = 6 * e4m3(big0), b1 = -6 * e4m3(big0), sm = 0.5 * e4m3(small);
    e0 = 62 * sm, e1 = 0.5 * 2 * e4m3(big0) + 62 * sm, name = "fp4xfp8";
  }
  printf("{\"probe\": \"accum\", \"mfma\": \"%s\", \"large_products\": [%g, %g], \"small_product\": %g, "
         "\"row0\": %.10g, \"row0_exact\": %.10g, \"row1\": %.10g, \"row1_exact\": %.10g}\n",
         name, b0, b1, sm, h[0], e0, h[1], e1);
}

int main(int argc, char** argv) {
  hipDeviceProp_t prop;
  CK(hipGetDeviceProperties(&prop, 0));
  printf("{\"device\": \"%s\", \"cus\": %d, \"clock_khz\": %d}\n", prop.gcnArchName, prop.multiProcessorCount,
         prop.clockRate);
  float* out;
  CK(hipMalloc(&out, static_cast<size_t>(prop.multiProcessorCount) * 2 * 256 * sizeof(float)));
  rate<kBf16>(prop.multiProcessorCount, out, 32.0 * 32 * 16 * 2, 2516.6, "32x32x16_bf16");
  rate<kFp8Fp8>(prop.multiProcessorCount, out, 32.0 * 32 * 64 * 2, 5033.2, "scale_32x32x64_fp8xfp8");
  rate<kFp4Fp8>(prop.multiProcessorCount, out, 32.0 * 32 * 64 * 2, 5033.2, "scale_32x32x64_fp4xfp8");
  rate<kFp4Fp4>(prop.multiProcessorCount, out, 32.0 * 32 * 64 * 2, 10066.3, "scale_32x32x64_fp4xfp4");
  mfma_lds(prop.multiProcessorCount, out);
  // FP8: large products 448 (+448 or -448), small 2^e
  for (int e = -9; e <= -2; ++e) {
    accum(0, 0x7E, 0x00, e4m3_pow2(e), out);
    accum(0, 0x7E, 0xFE, e4m3_pow2(e), out);
  }
  // FP4 x FP8: large products +-6 * 448, small 0.5 * 2^e
  for (int e = -9; e <= 0; ++e) accum(1, 0x7E, 0, e4m3_pow2(e), out);
  // BF16: large products 2^20 (+2^20 or -2^20), small 2^e
  for (int e = -12; e <= -2; ++e) {
    const uint32_t sm = static_cast<uint32_t>(127 + e) << 7;
    accum(2, 0x4980, 0x0000, sm, out);
    accum(2, 0x4980, 0xC980, sm, out);
  }
  CK(hipFree(out));
  return 0;
}
