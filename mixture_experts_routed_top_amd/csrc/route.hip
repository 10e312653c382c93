// Top-k routing: one wavefront per token.
//
// Selection is a radix select on order-preserving integer keys of the fp32
// logits: 32 ballot rounds find the k-th largest key (no cross-lane data
// movement), the k winners are the keys above it plus the lowest-index keys
// equal to it, and one compaction through LDS puts them in slot order (logit
// descending, equal logits -> lower expert index). The gate weights are the
// softmax over the selected logits, summed in slot order, or the sigmoid of
// each selected logit (TileScale PR #70, Design: routing precedes the expert
// GEMMs; the renormalised top-k softmax equals a softmax over the k selected
// logits).
#include "moe_common.cuh"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kWavesPerBlock = 4;

// Order-preserving key of an fp32 value: larger value <-> larger key; -0 and
// +0 map to the same key, as they compare equal.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// (ka, ea) ranks before (kb, eb): larger key, or equal key and lower id.
__device__ __forceinline__ bool before(uint32_t ka, int ea, uint32_t kb, int eb) {
  return ka > kb || (ka == kb && ea < eb);
}

__device__ __forceinline__ int popc(uint64_t m) { return __popcll(m); }

template <int PER_LANE>
__global__ __launch_bounds__(64 * kWavesPerBlock) void route_kernel(const float* __restrict__ logits, int64_t T,
                                                                    int E, int k, int score, int n_shared,
                                                                    int32_t* __restrict__ ids,
                                                                    float* __restrict__ w) {
  __shared__ uint32_t s_key[kWavesPerBlock][32];
  __shared__ int s_e[kWavesPerBlock][32];
  __shared__ float s_v[kWavesPerBlock][32];
  const int lane = threadIdx.x & 63, wib = threadIdx.x >> 6;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wib;
  if (t >= T) return;  // whole wave leaves together; no workgroup barrier below
  const float* row = logits + t * E;
  const uint64_t lt_mask = (1ull << lane) - 1;   // lanes below this one

  uint32_t key[PER_LANE];
  float val[PER_LANE];
  bool ok[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int e = lane + 64 * i;
    ok[i] = e < E;
    val[i] = ok[i] ? row[e] : 0.0f;
    key[i] = order_key(val[i]);
  }

  // the k-th largest key: the largest tau with #{key >= tau} >= k
  uint32_t tau = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = tau | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) cnt += popc(__ballot(ok[i] && key[i] >= cand));
    if (cnt >= k) tau = cand;
  }
  // winners: every key above tau, then the lowest-index keys equal to tau
  int n_gt = 0;
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) n_gt += popc(__ballot(ok[i] && key[i] > tau));
  const int n_eq_take = k - n_gt;
  int eq_before = 0, sel_before = 0;
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const uint64_t eq = __ballot(ok[i] && key[i] == tau);
    const bool take_eq = ((eq >> lane) & 1ull) && eq_before + popc(eq & lt_mask) < n_eq_take;
    eq_before += popc(eq);
    const bool sel = (ok[i] && key[i] > tau) || take_eq;
    const uint64_t sm = __ballot(sel);
    if (sel) {
      // compact in expert order: position among the winners
      const int pos = sel_before + popc(sm & lt_mask);
      s_key[wib][pos] = key[i];
      s_e[wib][pos] = lane + 64 * i;
      s_v[wib][pos] = val[i];
    }
    sel_before += popc(sm);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // slot of winner j = number of winners ranked before it
  uint32_t my_key = 0;
  int my_e = 0, slot = 0;
  float my_v = 0.0f;
  if (lane < k) {
    my_key = s_key[wib][lane];
    my_e = s_e[wib][lane];
    my_v = s_v[wib][lane];
    for (int j = 0; j < k; ++j) slot += before(s_key[wib][j], s_e[wib][j], my_key, my_e) ? 1 : 0;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < k) {
    s_e[wib][slot] = my_e;
    s_v[wib][slot] = my_v;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // lane j now takes slot j
  if (lane < k) {
    my_e = s_e[wib][lane];
    my_v = s_v[wib][lane];
  }

  float wj;
  if (score == 0) {
    const float l0 = __shfl(my_v, 0);
    const float z = lane < k ? expf(my_v - l0) : 0.0f;
    float sum = 0.0f;
    for (int j = 0; j < k; ++j) sum += __shfl(z, j);
    wj = __fdiv_rn(z, sum);
  } else {
    wj = __fdiv_rn(1.0f, 1.0f + expf(-my_v));
  }
  // slots k .. k + n_shared - 1: the shared experts E .. E + n_shared - 1, weight 1
  const int kk = k + n_shared;
  if (lane < k) {
    ids[t * kk + lane] = my_e;
    w[t * kk + lane] = wj;
  } else if (lane < kk) {
    ids[t * kk + lane] = E + (lane - k);
    w[t * kk + lane] = 1.0f;
  }
}

}  // namespace

hipError_t launch_route(const float* logits, int64_t T, int E, int k, int score, int n_shared, int32_t* ids,
                        float* w, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((T + kWavesPerBlock - 1) / kWavesPerBlock)), block(64 * kWavesPerBlock);
  if (E <= 64) route_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, score, n_shared, ids, w);
  else if (E <= 128) route_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, score, n_shared, ids, w);
  else if (E <= 256) route_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, score, n_shared, ids, w);
  else if (E <= 512) route_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, score, n_shared, ids, w);
  else route_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k, score, n_shared, ids, w);
  return hipGetLastError();
}

}  // namespace moe
