// Top-k routing: one wavefront per token.
//
// The k largest logits are taken in k rounds of a wave-wide arg-max over
// (logit, expert) pairs ordered by logit descending, then expert ascending,
// so equal logits go to the lower expert index. Lane j keeps the j-th winner;
// the gate weights are then the softmax over the selected logits, summed in
// slot order, or the sigmoid of each selected logit (TileScale PR #70, Design:
// routing precedes the expert GEMMs; the renormalised top-k softmax equals a
// softmax over the k selected logits).
#include <climits>

#include "moe_common.cuh"
#include "moe_launch.h"

namespace moe {

namespace {

__device__ __forceinline__ bool better(float v, int e, float bv, int be) {
  // (v, e) ranks before (bv, be): larger logit, or equal logit and lower id.
  // be == INT_MAX marks "nothing yet".
  if (e == INT_MAX) return false;
  if (be == INT_MAX) return true;
  return v > bv || (v == bv && e < be);
}

template <int PER_LANE>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                    int k, int score, int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave leaves together
  const float* row = logits + t * E;

  float v[PER_LANE];
  uint32_t avail = 0;
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : 0.0f;
    if (e < E) avail |= 1u << i;
  }

  float my_v = 0.0f;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int be = INT_MAX;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      const int e = lane + 64 * i;
      if (((avail >> i) & 1u) && better(v[i], e, bv, be)) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oe = __shfl_xor(be, o);
      if (better(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    // every lane now holds the same winner
    if ((be & 63) == lane) avail &= ~(1u << (be >> 6));
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
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
  if (lane < k) {
    ids[t * k + lane] = my_e;
    w[t * k + lane] = wj;
  }
}

}  // namespace

hipError_t launch_route(const float* logits, int64_t T, int E, int k, int score, int32_t* ids,
                        float* w, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((T + 3) / 4)), block(256);
  if (E <= 64) route_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, score, ids, w);
  else if (E <= 128) route_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, score, ids, w);
  else if (E <= 256) route_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, score, ids, w);
  else if (E <= 512) route_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, score, ids, w);
  else route_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k, score, ids, w);
  return hipGetLastError();
}

}  // namespace moe
