// Top-k routing: one wavefront per token.
//
// Selection is a radix select on order-preserving integer keys of the fp32
// logits: 32 counting rounds find the k-th largest key, the k winners are the keys above it plus the lowest-index keys
// equal to it, and one compaction through LDS puts them in slot order (logit
// descending, equal logits -> lower expert index). With more than 128
// experts the select runs on a few candidates instead of every key: the k-th
// largest of the 64 lanes' maxima is a lower bound of the k-th largest key
// (k lanes hold a key at least that large), so every winner is among the
// keys at or above it; when those are at most 64 (about k + 1 for random
// logits) they are gathered in expert order, one a lane, and selected there. The gate weights are the
// softmax over the selected logits, summed in slot order, or the sigmoid of
// each selected logit, both in double precision and rounded once to fp32 (TileScale PR #70, Design: routing precedes the expert
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

// DPP lane patterns: within each row of 16 lanes, swap neighbours, swap
// pairs, mirror each half row, mirror the row; across rows, lane 15 of each
// row to the next row, lane 31 to rows 2 and 3 (the row masks below pick
// which rows take them).
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_add(int v) {
  // rows outside ROW_MASK keep v (the moved value is not added there)
  return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

// Number of the wave's keys >= c (wave-uniform). Padding keys are 0, below
// every c >= 1. With one or two keys a lane, one ballot and one scalar
// popcount per key. With more, a lane counts its own keys and the counts
// are added across lanes by DPP moves (quad swaps, then the half-row and row
// mirrors leave each row's sum in all its lanes; two row broadcasts then
// leave the wave's sum in lane 63), read once: one ballot per key would make
// the CU's single scalar unit the bottleneck (8 keys a lane, 64 waves a CU,
// up to 32 rounds).
template <int PER_LANE>
__device__ __forceinline__ int count_ge(const uint32_t (&key)[PER_LANE], uint32_t c) {
  if constexpr (PER_LANE <= 2) {
    int n = 0;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) n += popc(__ballot(key[i] >= c));
    return n;
  } else {
    int n = 0;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) n += key[i] >= c ? 1 : 0;
    n = dpp_add<kDppXor1>(n);
    n = dpp_add<kDppXor2>(n);
    n = dpp_add<kDppHalfMirror>(n);
    n = dpp_add<kDppMirror>(n);             // every lane: its row's sum
    n = dpp_add<kDppBcast15, 0xA>(n);       // rows 1, 3: rows 0 + 1, rows 2 + 3
    n = dpp_add<kDppBcast31, 0xC>(n);       // rows 2, 3: + rows 0 + 1 (row 3: all four)
    return __builtin_amdgcn_readlane(n, 63);
  }
}

template <int PER_LANE>
__global__ __launch_bounds__(64 * kWavesPerBlock) void route_kernel(const float* __restrict__ logits, int64_t T,
                                                                    int E, int k, int score, int n_shared,
                                                                    int32_t* __restrict__ ids,
                                                                    float* __restrict__ w) {
  __shared__ uint32_t s_key[kWavesPerBlock][32];
  __shared__ int s_e[kWavesPerBlock][32];
  __shared__ float s_v[kWavesPerBlock][32];
  __shared__ uint32_t s_ck[kWavesPerBlock][64];   // candidates (more than 128 experts)
  __shared__ int s_ce[kWavesPerBlock][64];
  __shared__ float s_cv[kWavesPerBlock][64];
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
    key[i] = ok[i] ? order_key(val[i]) : 0u;   // padding: below every candidate tau | bit
  }

  // the k winners go to s_key / s_e / s_v (any order)
  bool done = false;
  if constexpr (PER_LANE >= 4) {
    // lower bound: the k-th largest lane maximum (every lane holds a real
    // key, and padding keys are 0, so a lane's maximum is one of its real
    // keys and at least k real keys lie at or above the bound)
    uint32_t lm = key[0];
#pragma unroll
    for (int i = 1; i < PER_LANE; ++i) lm = key[i] > lm ? key[i] : lm;
    uint32_t t0 = 0;
    for (int b = 31; b >= 0; --b) {
      const uint32_t cand = t0 | (1u << b);
      const int n = popc(__ballot(lm >= cand));
      if (n >= k) t0 = cand;
      if (n == k) break;
    }
    uint64_t m[PER_LANE];
    int total = 0;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      m[i] = __ballot(ok[i] && key[i] >= t0);
      total += popc(m[i]);
    }
    if (total <= 64) {
      // gather the candidates in expert order (slot-major: expert lane + 64 i)
      int before = 0;
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i) {
        if ((m[i] >> lane) & 1ull) {
          const int pos = before + popc(m[i] & lt_mask);
          s_ck[wib][pos] = key[i];
          s_ce[wib][pos] = lane + 64 * i;
          s_cv[wib][pos] = val[i];
        }
        before += popc(m[i]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const bool has = lane < total;
      const uint32_t ck = has ? s_ck[wib][lane] : 0u;
      const int ce = has ? s_ce[wib][lane] : 0;
      const float cv = has ? s_cv[wib][lane] : 0.0f;
      uint32_t tau = 0;
      for (int b = 31; b >= 0; --b) {
        const uint32_t cand = tau | (1u << b);
        const int n = popc(__ballot(ck >= cand));
        if (n >= k) tau = cand;
        if (n == k) break;
      }
      // winners: every candidate above tau, then the first (lowest-expert) ones equal to it
      const int n_gt = popc(__ballot(has && ck > tau));
      const uint64_t eq = __ballot(has && ck == tau);
      const bool take_eq = ((eq >> lane) & 1ull) && popc(eq & lt_mask) < k - n_gt;
      const bool sel = (has && ck > tau) || take_eq;
      const uint64_t sm = __ballot(sel);
      if (sel) {
        const int pos = popc(sm & lt_mask);
        s_key[wib][pos] = ck;
        s_e[wib][pos] = ce;
        s_v[wib][pos] = cv;
      }
      done = true;
    }
  }
  if (!done) {
    // the k-th largest key: the largest tau with #{key >= tau} >= k. Once a
    // candidate has exactly k keys at or above it, those keys are the winners
    // and the lower bits cannot change the selection below (every key equal to
    // tau is then taken), so the search stops there: after about 15 of the 32
    // rounds for distinct random logits.
    uint32_t tau = 0;
    for (int b = 31; b >= 0; --b) {
      const uint32_t cand = tau | (1u << b);
      const int n = count_ge<PER_LANE>(key, cand);
      if (n >= k) tau = cand;
      if (n == k) break;
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

  // The weights are evaluated in double precision and rounded once to fp32:
  // the difference of two fp32 logits is exact in double, and the double
  // exp / sum / division err by a few units in 2^-53, so the fp32 result is
  // the correctly rounded weight except within that distance of a rounding
  // midpoint. (k exponentials per token; the kernel is bound by its logit
  // reads, not by this arithmetic.)
  float wj;
  if (score == 0) {
    const double l0 = static_cast<double>(__shfl(my_v, 0));
    const double z = lane < k ? exp(static_cast<double>(my_v) - l0) : 0.0;
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += __shfl(z, j);
    wj = static_cast<float>(z / sum);
  } else {
    wj = static_cast<float>(1.0 / (1.0 + exp(-static_cast<double>(my_v))));
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
