// Device helpers shared by the gfx950 kernels: vector types, bf16 / E4M3 /
// E2M1 / E8M0 conversions, wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;

constexpr int kWave = 64;

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even of a finite fp32 value to bf16 (bit pattern).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// ------------------------------------------------------------------ E4M3 (OCP E4M3FN)
// Hardware conversion of two fp32 values to E4M3 (round to nearest even) into
// the low (WORD_HI = false) or high 16 bits of `old`. Inputs are clamped to
// [-448, 448] first, which is the saturating conversion: every magnitude
// above 448 would round to 448 or to the (absent) 480.
template <bool WORD_HI>
__device__ __forceinline__ uint32_t cvt_e4m3x2(float a, float b, uint32_t old) {
  a = __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f);
  b = __builtin_fminf(__builtin_fmaxf(b, -448.0f), 448.0f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, static_cast<int>(old), WORD_HI));
}

__device__ __forceinline__ uint32_t pack_e4m3x4(float v0, float v1, float v2, float v3) {
  const uint32_t r = cvt_e4m3x2<false>(v0, v1, 0u);
  return cvt_e4m3x2<true>(v2, v3, r);
}

// ------------------------------------------------------------------ E2M1
// Round-to-nearest-even of a finite fp32 value to a 4-bit E2M1 code
// (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), saturating at 6. Decision
// thresholds are the midpoints of the grid; at a midpoint the code with an
// even mantissa bit wins (0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2,
// 3.5->4, 5->4).
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = __builtin_fabsf(v);
  uint32_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  return c | ((__float_as_uint(v) >> 28) & 0x8u);
}

// ------------------------------------------------------------------ E8M0 (OCP MX shared scale)
// floor(log2(a)) of a finite a > 0 (normal or subnormal fp32), exactly.
__device__ __forceinline__ int floor_log2(float a) {
  const uint32_t u = __float_as_uint(a);
  const int ex = static_cast<int>((u >> 23) & 0xFF);
  if (ex != 0) return ex - 127;
  return (31 - static_cast<int>(__builtin_clz(u & 0x7FFFFFu))) - 149;  // subnormal: m * 2^-149
}

// E8M0 byte of a block with maximum magnitude amax for an element format whose
// largest power of two is 2^emax (E4M3: 8, E2M1: 2). Byte 0 when amax == 0.
__device__ __forceinline__ int mx_scale_exponent(float amax, int emax) {
  if (!(amax > 0.0f)) return -127;
  int x = floor_log2(amax) - emax;
  return x < -127 ? -127 : (x > 127 ? 127 : x);
}

// 2^-x as fp32 for x in [-127, 127] (the reciprocal of the MX scale); v * it
// is exact whenever the product is a normal fp32 number.
__device__ __forceinline__ float mx_inv_scale(int x) { return __builtin_ldexpf(1.0f, -x); }

// Split a finite scale s >= 0 into s = m * 2^(b - 127) with b an E8M0 byte
// (b in [0, 254]): for a normal s, b is its biased exponent and m in [1, 2);
// for a subnormal s (or 0), b = 0 and m = s * 2^127, exact and below 1.
__device__ __forceinline__ float split_e8m0(float s, int& b) {
  const uint32_t u = __float_as_uint(s);
  b = static_cast<int>((u >> 23) & 0xFF);
  return b ? __uint_as_float((u & 0x007FFFFFu) | 0x3F800000u) : s * 0x1p127f;
}

// ------------------------------------------------------------------ wave reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o));
  return v;
}

template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, WIDTH));
  return v;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }


// ------------------------------------------------------------------ LDS pipelines
// Wait until at most N of this wave's vector memory operations are outstanding
// (loads complete in issue order, so: all but the N most recent loads have
// landed, in LDS for the direct-to-LDS form) and every LDS read it issued has
// returned, so that a stage it read may be refilled after the next barrier.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// Workgroup barrier that orders the compiler's memory accesses around it (the
// clobber) without the release/acquire fences of __syncthreads, whose wait for
// every outstanding load would also wait for the later pipeline stages.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// ------------------------------------------------------------------ grouped task order
// Task order of the grouped GEMMs over the expert-sorted m-tiles (the BF16
// kernels always, the FP8 / MX kernels when one m-tile's walk over the
// n-tiles reads more weight bytes than an XCD's L2 holds): the m-tiles of one
// expert (groups of up to GROUP, from the expert's first tile) go side by
// side along n, m fastest, so the tasks that read the same weight slice run
// together and share it in L2. A group of c m-tiles
// owns the c * ntn tasks from its first tile times ntn, so tile task / ntn
// lies in the task's group; one 64-lane load around that tile (lane 0 at it,
// lanes 1..31 behind, lanes 32..63 after) finds the expert's first and last
// tile, and longer runs continue 64 tiles at a time. Tiles are in expert
// order (tile_expert is non-decreasing over [0, num_tiles)). Called by whole
// waves with wave-uniform arguments; returns the task's n-tile, m-tile and
// expert. The 64-lane load is grouped_probe, issued ahead (a task loads the
// next task's probe, so that its latency hides behind the k-loop) and passed
// in as v.
__device__ __forceinline__ int grouped_probe(int64_t task, int ntn, int num_tiles, const int32_t* tile_expert,
                                             int lane) {
  const int q = static_cast<int>(task / ntn);
  const int i = lane < 32 ? q - lane : q + lane - 31;
  return tile_expert[i < 0 ? 0 : (i < num_tiles ? i : q)];
}

template <int GROUP>
__device__ __forceinline__ void grouped_task(int64_t task, int ntn, int num_tiles, const int32_t* tile_expert,
                                             int lane, int v, int& nt, int& mt, int& e) {
  const int q = static_cast<int>(task / ntn);
  const int i = lane < 32 ? q - lane : q + lane - 31;
  e = __builtin_amdgcn_readfirstlane(v);
  const uint64_t m = __ballot(i >= 0 && i < num_tiles && v == e);
  const uint32_t mb = static_cast<uint32_t>(m), ma = static_cast<uint32_t>(m >> 32);
  const int rb = ~mb == 0 ? 32 : __builtin_ctz(~mb);      // tiles q, q-1, .. of expert e
  const int ra = ~ma == 0 ? 32 : __builtin_ctz(~ma);      // tiles q+1, q+2, .. of expert e
  int f = q + 1 - rb, l = q + 1 + ra;
  if (rb == 32) {
    for (;;) {
      const int j = f - 1 - lane;
      const uint64_t mm = __ballot(j >= 0 && tile_expert[j >= 0 ? j : 0] == e);
      const int run = ~mm == 0 ? 64 : __builtin_ctzll(~mm);
      f -= run;
      if (run < 64) break;
    }
  }
  if (ra == 32) {
    for (;;) {
      const int j = l + lane;
      const uint64_t mm = __ballot(j < num_tiles && tile_expert[j < num_tiles ? j : 0] == e);
      const int run = ~mm == 0 ? 64 : __builtin_ctzll(~mm);
      l += run;
      if (run < 64) break;
    }
  }
  const int gs = f + (q - f) / GROUP * GROUP;
  const int gc = l - gs < GROUP ? l - gs : GROUP;
  const int r = static_cast<int>(task - static_cast<int64_t>(gs) * ntn);
  nt = r / gc;
  mt = gs + r % gc;
}

}  // namespace moe
