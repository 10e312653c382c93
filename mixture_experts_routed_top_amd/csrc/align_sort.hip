// Expert-sorted, tile-padded permutation of the assignments and the flat tile
// queue (FlashInfer PR #5129, Description: padded expert-sorted rows;
// TileScale PR #70, first commit note: a flat m-task list instead of a
// per-tile rescan of experts; Liger-Kernel PR #1463, Summary: empty experts
// own no work).
//
// A deterministic counting sort in four launches:
//   1. count_rank: each 1024-assignment chunk is split over 4 wavefronts; a
//      wave ranks its 64 assignments at a time by matching equal expert ids
//      with one ballot per id bit (a wave-wide "match any"), so each
//      assignment gets its rank among the earlier, equal-expert assignments
//      of its chunk; per-chunk expert counts go to the workspace.
//   2. scan_chunks: one block per expert turns its column of chunk counts
//      into exclusive prefixes (the chunk's base inside the expert) and the
//      expert's total.
//   3. offsets: one block pads each count to block_m and scans over experts.
//   4. scatter: every assignment lands at offsets[e] + chunk base + rank;
//      the same grid fills pad rows with the sentinel A and writes the tile
//      queue (tile -> expert, -1 past the last tile).
// Nothing depends on the order of atomic operations, so the output is the
// stable order by (expert, assignment) on every run.
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

// Exclusive scan of a block of 256 values; returns this thread's prefix and
// writes the block total to *total (all threads).
__device__ __forceinline__ int block_exclusive_scan(int v, int* total, int* sh /*[4]*/) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(inc, o);
    if (lane >= o) inc += u;
  }
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  int wbase = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int s = sh[w];
    if (w < wave) wbase += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return wbase + inc - v;
}

__global__ __launch_bounds__(256) void scan_chunks_kernel(int32_t* __restrict__ chunk_counts, int nchunks,
                                                          int E, int32_t* __restrict__ counts) {
  __shared__ int sh[4];
  const int e = blockIdx.x;
  int carry = 0;
  for (int c0 = 0; c0 < nchunks; c0 += 256) {
    const int c = c0 + threadIdx.x;
    const int v = c < nchunks ? chunk_counts[static_cast<int64_t>(c) * E + e] : 0;
    int tot;
    const int ex = block_exclusive_scan(v, &tot, sh);
    if (c < nchunks) chunk_counts[static_cast<int64_t>(c) * E + e] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) counts[e] = carry;
}

__global__ __launch_bounds__(1024) void offsets_kernel(const int32_t* __restrict__ counts, int E, int block_m,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ num_tiles) {
  __shared__ int sh[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid < E ? counts[tid] : 0;
  const int p = (c + block_m - 1) / block_m * block_m;
  int inc = p;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(inc, o);
    if (lane >= o) inc += u;
  }
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  int wbase = 0, tot = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) wbase += sh[w];
    tot += sh[w];
  }
  if (tid < E) offsets[tid] = wbase + inc - p;
  if (tid == 0) {
    offsets[E] = tot;
    *num_tiles = tot / block_m;
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

__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ ids,
                                                      const int32_t* __restrict__ local_rank,
                                                      const int32_t* __restrict__ chunk_base,
                                                      const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ offsets, int64_t A,
                                                      int E, int block_m, int64_t cap,
                                                      int32_t* __restrict__ sorted_ids,
                                                      int32_t* __restrict__ tile_expert) {
  __shared__ int32_t off[kMaxE + 1];
  __shared__ int32_t cnt[kMaxE];
  for (int e = threadIdx.x; e <= E; e += 256) {
    off[e] = offsets[e];
    if (e < E) cnt[e] = counts[e];
  }
  __syncthreads();
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int total = off[E];
  if (i < A) {
    const int e = ids[i];
    const int64_t c = i / kAlignChunk;
    const int pos = off[e] + chunk_base[c * E + e] + local_rank[i];
    sorted_ids[pos] = static_cast<int32_t>(i);
  }
  if (i < cap) {
    const int r = static_cast<int>(i);
    bool pad = r >= total;
    if (!pad) {
      const int e = find_expert(off, E, r);
      pad = r - off[e] >= cnt[e];
    }
    if (pad) sorted_ids[r] = static_cast<int32_t>(A);
  }
  if (i < cap / block_m) {
    const int r = static_cast<int>(i) * block_m;
    tile_expert[i] = r < total ? find_expert(off, E, r) : -1;
  }
}

int bits_for(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

}  // namespace

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
  const int nchunks = static_cast<int>((A + kAlignChunk - 1) / kAlignChunk);
  int32_t* chunk_counts = static_cast<int32_t*>(ws);
  int32_t* local_rank = chunk_counts + static_cast<int64_t>(nchunks) * E;
  count_rank_kernel<<<nchunks, 256, 0, s>>>(ids, A, E, bits_for(E), chunk_counts, local_rank);
  scan_chunks_kernel<<<E, 256, 0, s>>>(chunk_counts, nchunks, E, counts);
  offsets_kernel<<<1, 1024, 0, s>>>(counts, E, block_m, offsets, num_tiles);
  const int64_t n = cap > A ? cap : A;
  scatter_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
      ids, local_rank, chunk_counts, counts, offsets, A, E, block_m, cap, sorted_ids, tile_expert);
  return hipGetLastError();
}

}  // namespace moe
