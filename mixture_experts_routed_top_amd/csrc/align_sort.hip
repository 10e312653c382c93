// Expert-sorted, tile-padded permutation of the assignments and the flat tile
// queue (FlashInfer PR #5129, Description: padded expert-sorted rows;
// TileScale PR #70, first commit note: a flat m-task list instead of a
// per-tile rescan of experts; Liger-Kernel PR #1463, Summary: empty experts
// own no work).
//
// A deterministic counting sort in two launches (one workgroup for at most
// 2048 assignments: one_block_kernel, the same steps in LDS):
//   1. count_rank: each 1024-assignment chunk is split over 4 wavefronts; a
//      wave ranks its 64 assignments at a time by matching equal expert ids
//      with one ballot per id bit (a wave-wide "match any"), so each
//      assignment gets its rank among the earlier, equal-expert assignments
//      of its chunk; per-chunk expert counts go to the workspace.
//   2. scan and scatter: every block reads all the chunk counts and forms
//      each expert's total and the base of its own chunk inside each expert,
//      pads the totals to block_m and scans them over the experts (offsets),
//      then puts every assignment of its rows at offsets[e] + chunk base +
//      rank, fills pad rows with the sentinel A and writes the tile queue
//      (tile -> expert, -1 past the last tile). Small problems (E * chunks
//      <= 2048) use blocks of 256 rows (scan_scatter_kernel), larger ones
//      one block of 1024 threads per chunk (scan_scatter_wide_kernel).
// Nothing depends on the order of atomic operations, so the output is the
// stable order by (expert, assignment) on every run.
#include <mutex>

#include "moe_common.cuh"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kMaxE = 1024;

__device__ __forceinline__ int rank_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
}

__global__ __launch_bounds__(256) void count_rank_kernel(const int32_t* __restrict__ ids, int64_t A,
                                                         int E, int nbits,
                                                         int32_t* __restrict__ chunk_counts,
                                                         int32_t* __restrict__ local_rank) {
  __shared__ int32_t wcnt[4][kMaxE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int e = tid; e < E; e += 256) {
    wcnt[0][e] = 0;
    wcnt[1][e] = 0;
    wcnt[2][e] = 0;
    wcnt[3][e] = 0;
  }
  __syncthreads();

  const int64_t base = static_cast<int64_t>(blockIdx.x) * kAlignChunk + wave * 256;
  int r[4], ex[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int64_t a = base + g * 64 + lane;
    const bool valid = a < A;
    const int e = valid ? ids[a] : 0;
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    const int rk = rank_below(m);
    const int cnt = __popcll(m);
    const int b0 = valid ? wcnt[wave][e] : 0;
    r[g] = b0 + rk;
    ex[g] = e;
    if (valid && rk == 0) wcnt[wave][e] = b0 + cnt;  // one writer per distinct expert
  }
  __syncthreads();

  for (int e = tid; e < E; e += 256) {
    const int c0 = wcnt[0][e], c1 = wcnt[1][e], c2 = wcnt[2][e], c3 = wcnt[3][e];
    wcnt[0][e] = 0;
    wcnt[1][e] = c0;
    wcnt[2][e] = c0 + c1;
    wcnt[3][e] = c0 + c1 + c2;
    chunk_counts[static_cast<int64_t>(blockIdx.x) * E + e] = c0 + c1 + c2 + c3;
  }
  __syncthreads();

#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int64_t a = base + g * 64 + lane;
    if (a < A) local_rank[a] = wcnt[wave][ex[g]] + r[g];
  }
}

// Largest e in [0, E) with off[e] <= r (off non-decreasing, off[0] = 0 <= r).
__device__ __forceinline__ int find_expert(const int32_t* off, int E, int r) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Steps 2-4 in one launch, for small problems (E * nchunks <= kFusedScan,
// where a launch costs more than the work): every block of 256 assignments
// reads all the chunk counts (coalesced) and adds them into per-expert
// totals and per-expert prefixes before its own chunk with LDS atomics
// (integer sums: the order does not matter), scans the padded offsets, then
// scatters its rows. Block 0 writes counts, offsets, num_tiles.
constexpr int kFusedScan = 2048;

__global__ __launch_bounds__(256) void scan_scatter_kernel(const int32_t* __restrict__ ids,
                                                           const int32_t* __restrict__ local_rank,
                                                           const int32_t* __restrict__ chunk_counts, int nchunks,
                                                           int64_t A, int E, int block_m, int64_t cap,
                                                           int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ num_tiles,
                                                           int32_t* __restrict__ sorted_ids,
                                                           int32_t* __restrict__ tile_expert) {
  __shared__ int32_t tot[kMaxE];
  __shared__ int32_t pre[kMaxE];
  __shared__ int32_t off[kMaxE + 1];
  __shared__ int sh[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * 256;
  const int cb = i0 < A ? static_cast<int>(i0 / kAlignChunk) : nchunks;   // this block's chunk (256 | 1024)
  for (int e = tid; e < E; e += 256) {
    tot[e] = 0;
    pre[e] = 0;
  }
  __syncthreads();
  const int n = E * nchunks;
  for (int idx = tid; idx < n; idx += 256) {
    const int c = idx / E, e = idx - c * E;
    const int v = chunk_counts[idx];
    if (v) {
      atomicAdd(&tot[e], v);
      if (c < cb) atomicAdd(&pre[e], v);
    }
  }
  __syncthreads();
  // exclusive scan of the padded counts over the experts, 4 a thread
  int loc[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    loc[q] = e < E ? (tot[e] + block_m - 1) / block_m * block_m : 0;
    sum += loc[q];
  }
  int inc = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(inc, o);
    if (lane >= o) inc += u;
  }
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  int wbase = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) wbase += sh[w];
    all += sh[w];
  }
  int run = wbase + inc - sum;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    if (e < E) off[e] = run;
    run += loc[q];
  }
  if (tid == 0) off[E] = all;
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int e = tid; e <= E; e += 256) {
      offsets[e] = off[e];
      if (e < E) counts[e] = tot[e];
    }
    if (tid == 0) *num_tiles = all / block_m;
  }
  const int64_t i = i0 + tid;
  if (i < A) {
    const int e = ids[i];
    sorted_ids[off[e] + pre[e] + local_rank[i]] = static_cast<int32_t>(i);
  }
  if (i < cap) {
    const int r = static_cast<int>(i);
    bool pad = r >= all;
    if (!pad) {
      const int e = find_expert(off, E, r);
      pad = r - off[e] >= tot[e];
    }
    if (pad) sorted_ids[r] = static_cast<int32_t>(A);
  }
  if (i < cap / block_m) {
    const int r = static_cast<int>(i) * block_m;
    tile_expert[i] = r < all ? find_expert(off, E, r) : -1;
  }
}

// Steps 2-4 in one launch for the larger problems (E * nchunks > kFusedScan),
// one block of 1024 threads per 1024 rows, so that block b scatters exactly
// chunk b's assignments. Every block reads the whole chunk-count matrix (at
// most a few hundred KB, from L2): thread (s, e), s < S = 1024 / E, adds
// expert e's counts over the chunks s, s + S, s + 2S, ... in registers, 16
// loads in flight, both in full (the expert's total) and over the chunks
// before the block's own (its base inside the expert); the S slices are then
// added in LDS. The padded scan over the experts and the scatter follow as in
// scan_scatter_kernel. Integer sums: the result is the same stable order.
// (It replaced three launches, a column scan per expert, the offsets and the
// scatter, each a few us of launch and dependency time for almost no work:
// 65536 assignments over 128 experts 12.5 -> 10.2 us, 64 experts 12.9 -> 9.2
// us, 163840 over 512 experts 16.6 -> 15.0 us, back-to-back calls.)
constexpr int kWideLoads = 16;
static_assert(kAlignChunk == 1024, "one 1024-thread block per chunk");

__global__ __launch_bounds__(1024) void scan_scatter_wide_kernel(const int32_t* __restrict__ ids,
                                                                 const int32_t* __restrict__ local_rank,
                                                                 const int32_t* __restrict__ chunk_counts,
                                                                 int nchunks, int64_t A, int E, int block_m,
                                                                 int64_t cap, int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ num_tiles,
                                                                 int32_t* __restrict__ sorted_ids,
                                                                 int32_t* __restrict__ tile_expert) {
  __shared__ int32_t ptot[1024];   // per (slice, expert): partial total
  __shared__ int32_t ppre[1024];   // ... and partial sum over the chunks before this block's
  __shared__ int32_t tot[kMaxE];
  __shared__ int32_t pre[kMaxE];
  __shared__ int32_t off[kMaxE + 1];
  __shared__ int sh[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * kAlignChunk;
  const int cb = i0 < A ? static_cast<int>(i0 / kAlignChunk) : nchunks;   // this block's chunk
  const int S = 1024 / E;                                                  // E <= kMaxE = 1024
  const int sl = tid / E, e = tid - sl * E;
  int t_acc = 0, p_acc = 0;
  if (sl < S) {
    int c = sl;
    for (; c + (kWideLoads - 1) * S < nchunks; c += kWideLoads * S) {
      int v[kWideLoads];
#pragma unroll
      for (int u = 0; u < kWideLoads; ++u) v[u] = chunk_counts[static_cast<int64_t>(c + u * S) * E + e];
#pragma unroll
      for (int u = 0; u < kWideLoads; ++u) {
        t_acc += v[u];
        p_acc += c + u * S < cb ? v[u] : 0;
      }
    }
    for (; c < nchunks; c += S) {
      const int v = chunk_counts[static_cast<int64_t>(c) * E + e];
      t_acc += v;
      p_acc += c < cb ? v : 0;
    }
  }
  ptot[tid] = t_acc;
  ppre[tid] = p_acc;
  __syncthreads();
  if (tid < E) {
    int a = 0, b = 0;
    for (int q = 0; q < S; ++q) {
      a += ptot[q * E + tid];
      b += ppre[q * E + tid];
    }
    tot[tid] = a;
    pre[tid] = b;
  }
  __syncthreads();
  // padded offsets: exclusive scan over the experts, one a thread
  const int p = tid < E ? (tot[tid] + block_m - 1) / block_m * block_m : 0;
  int inc = p;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(inc, o);
    if (lane >= o) inc += u;
  }
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  int wbase = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    if (w < wave) wbase += sh[w];
    all += sh[w];
  }
  if (tid < E) off[tid] = wbase + inc - p;
  if (tid == 0) off[E] = all;
  __syncthreads();
  if (blockIdx.x == 0) {
    if (tid < E) {
      offsets[tid] = off[tid];
      counts[tid] = tot[tid];
    }
    if (tid == 0) {
      offsets[E] = all;   // E may be 1024, one past the last thread
      *num_tiles = all / block_m;
    }
  }
  const int64_t i = i0 + tid;
  if (i < A) {
    const int x = ids[i];
    sorted_ids[off[x] + pre[x] + local_rank[i]] = static_cast<int32_t>(i);
  }
  if (i < cap) {
    const int r = static_cast<int>(i);
    bool pad = r >= all;
    if (!pad) {
      const int x = find_expert(off, E, r);
      pad = r - off[x] >= tot[x];
    }
    if (pad) sorted_ids[r] = static_cast<int32_t>(A);
  }
  if (i < cap / block_m) {
    const int r = static_cast<int>(i) * block_m;
    tile_expert[i] = r < all ? find_expert(off, E, r) : -1;
  }
}

// The whole sort in one workgroup, for at most kOneBlockMaxA assignments
// (2048: one launch instead of two pays only while one CU finishes the work
// quickly; the MXFP4 512-expert shape at T = 128, 1280 assignments, took
// 11.5 against 14.5 us, but at 8192 and 10240 assignments it was 1.7-3 us
// slower than the two launches):
// each of the 16 waves ranks a contiguous share (up to 16 groups of 64, the
// same ballot match as count_rank_kernel) and keeps ranks and experts in
// registers; the per-wave counts are scanned over the waves (each wave's
// base inside its expert) and the padded totals over the experts, all in
// LDS; then every wave scatters its share, each expert's thread writes its
// tiles of the tile queue, the pad rows are spread over all threads, and the
// rows and tiles past the last tile are filled. The result is the same
// stable order.
constexpr int kOneBlockWaves = 16, kOneBlockGroups = 2;
constexpr int64_t kOneBlockMaxA = int64_t{kOneBlockWaves} * kOneBlockGroups * 64;

__global__ __launch_bounds__(1024) void one_block_kernel(const int32_t* __restrict__ ids, int A, int E, int nbits,
                                                         int block_m, int cap, int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ num_tiles,
                                                         int32_t* __restrict__ sorted_ids,
                                                         int32_t* __restrict__ tile_expert) {
  __shared__ int32_t wcnt[kOneBlockWaves][kMaxE];   // per-wave counts, then per-wave bases
  __shared__ int32_t off[kMaxE + 1];
  __shared__ int32_t tot[kMaxE];
  __shared__ int sh[kOneBlockWaves];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int e = tid; e < E; e += 1024)
#pragma unroll
    for (int w = 0; w < kOneBlockWaves; ++w) wcnt[w][e] = 0;
  __syncthreads();

  // this wave's share: [lo, hi), a multiple of 64 long
  const int per = ((A + kOneBlockWaves - 1) / kOneBlockWaves + 63) / 64 * 64;
  const int lo = wave * per, hi = lo + per < A ? lo + per : A;
  int r[kOneBlockGroups], ex[kOneBlockGroups];
  // every id of the share is loaded before the first is used: one load
  // latency for the wave, not one per group
#pragma unroll
  for (int g = 0; g < kOneBlockGroups; ++g) {
    const int a = lo + g * 64 + lane;
    ex[g] = g * 64 < per && a < hi ? ids[a] : 0;
  }
#pragma unroll
  for (int g = 0; g < kOneBlockGroups; ++g) {
    r[g] = 0;
    if (g * 64 < per) {
      const int a = lo + g * 64 + lane;
      const bool valid = a < hi;
      const int e = ex[g];
      uint64_t m = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
      }
      const int rk = rank_below(m);
      const int b0 = valid ? wcnt[wave][e] : 0;
      r[g] = b0 + rk;
      if (valid && rk == 0) wcnt[wave][e] = b0 + __popcll(m);  // one writer per distinct expert
    }
  }
  __syncthreads();
  // each expert: exclusive prefix over the waves, and its total
  for (int e = tid; e < E; e += 1024) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kOneBlockWaves; ++w) {
      const int c = wcnt[w][e];
      wcnt[w][e] = run;
      run += c;
    }
    tot[e] = run;
  }
  __syncthreads();
  // padded offsets: exclusive scan over the experts (E <= 1024, one a thread)
  const int p = tid < E ? (tot[tid] + block_m - 1) / block_m * block_m : 0;
  int inc = p;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(inc, o);
    if (lane >= o) inc += u;
  }
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  int wbase = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kOneBlockWaves; ++w) {
    if (w < wave) wbase += sh[w];
    all += sh[w];
  }
  if (tid < E) off[tid] = wbase + inc - p;
  if (tid == 0) off[E] = all;
  __syncthreads();

#pragma unroll
  for (int g = 0; g < kOneBlockGroups; ++g) {
    const int a = lo + g * 64 + lane;
    if (g * 64 < per && a < hi) sorted_ids[off[ex[g]] + wcnt[wave][ex[g]] + r[g]] = a;
  }
  for (int e = tid; e < E; e += 1024) {
    counts[e] = tot[e];
    offsets[e] = off[e];
    for (int t = off[e] / block_m; t < off[e + 1] / block_m; ++t) tile_expert[t] = e;
  }
  // pad rows: slot j of expert e (j < block_m - 1) is row off[e] + tot[e] + j
  // if that is below off[e + 1]; spread over all threads
  for (int i = tid; i < E * (block_m - 1); i += 1024) {
    const int e = i / (block_m - 1), row = off[e] + tot[e] + (i - e * (block_m - 1));
    if (row < off[e + 1]) sorted_ids[row] = A;
  }
  for (int row = all + tid; row < cap; row += 1024) sorted_ids[row] = A;
  for (int t = all / block_m + tid; t < cap / block_m; t += 1024) tile_expert[t] = -1;
  if (tid == 0) {
    offsets[E] = all;
    *num_tiles = all / block_m;
  }
}

int bits_for(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

constexpr int64_t kNoAllocWords = (kNoAllocMaxA + kAlignChunk - 1) / kAlignChunk * kMaxE + kNoAllocMaxA;

}  // namespace

// Fixed scratch for callers that cannot allocate (moe_align_sort_noalloc):
// the workspace of up to kNoAllocMaxA assignments over kMaxE experts, in a
// file-scope device array. Each GPU the library runs on holds its own copy
// (2 MiB) until the process ends; every call on that GPU shares it. Its
// contents need no clearing: the counting pass writes every word a call
// reads before the later passes read it.
static __device__ __align__(256) int32_t scratch[kNoAllocWords];

size_t align_sort_scratch_bytes() { return static_cast<size_t>(kNoAllocWords) * sizeof(int32_t); }

// Device address of this GPU's scratch array. In host code `scratch` is only a
// host-side handle of the symbol, not a device address: the address is looked
// up once per device, with that device current, and kept.
hipError_t align_sort_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static void* addr[kMaxDevices];
  static hipError_t err[kMaxDevices];
  int d = -1;
  if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[d], [d] { err[d] = hipGetSymbolAddress(&addr[d], HIP_SYMBOL(scratch)); });
  if (err[d] != hipSuccess) return err[d];
  *ptr = addr[d];
  return hipSuccess;
}

size_t align_sort_ws_bytes(int64_t T, int k, int E) {
  const int64_t A = T * k;
  if (A <= 0) return 0;
  const int64_t nchunks = (A + kAlignChunk - 1) / kAlignChunk;
  return static_cast<size_t>(nchunks * E + A) * sizeof(int32_t);
}

hipError_t launch_align_sort(const int32_t* ids, int64_t T, int k, int E, int block_m, int32_t* counts,
                             int32_t* offsets, int32_t* sorted_ids, int32_t* tile_expert,
                             int32_t* num_tiles, int64_t cap, void* ws, hipStream_t s) {
  const int64_t A = T * k;
  if (A <= kOneBlockMaxA) {
    one_block_kernel<<<1, 1024, 0, s>>>(ids, static_cast<int>(A), E, bits_for(E), block_m, static_cast<int>(cap),
                                        counts, offsets, num_tiles, sorted_ids, tile_expert);
    return hipGetLastError();
  }
  const int nchunks = static_cast<int>((A + kAlignChunk - 1) / kAlignChunk);
  int32_t* chunk_counts = static_cast<int32_t*>(ws);
  int32_t* local_rank = chunk_counts + static_cast<int64_t>(nchunks) * E;
  count_rank_kernel<<<nchunks, 256, 0, s>>>(ids, A, E, bits_for(E), chunk_counts, local_rank);
  const int64_t n = cap > A ? cap : A;
  const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
  if (static_cast<int64_t>(E) * nchunks <= kFusedScan) {
    scan_scatter_kernel<<<blocks, 256, 0, s>>>(ids, local_rank, chunk_counts, nchunks, A, E, block_m, cap, counts,
                                               offsets, num_tiles, sorted_ids, tile_expert);
  } else {
    const unsigned wide = static_cast<unsigned>((n + kAlignChunk - 1) / kAlignChunk);
    scan_scatter_wide_kernel<<<wide, 1024, 0, s>>>(ids, local_rank, chunk_counts, nchunks, A, E, block_m, cap,
                                                   counts, offsets, num_tiles, sorted_ids, tile_expert);
  }
  return hipGetLastError();
}

}  // namespace moe
