// BF16 grouped GEMMs over the expert-sorted rows (FlashInfer PR #5129,
// Description: GEMM1 writes padded expert-sorted rows, GEMM2 reads them
// contiguously and scatters back to assignment order; TileScale PR #70,
// Design: GEMM1 + SwiGLU in one kernel, fp32 accumulation).
//
// Design for gfx950:
//   * persistent workgroups walk one flat task list: task = (m-tile of the
//     sorted rows, n-tile of the output columns); the m-tile count is read
//     from device memory, so the host never waits for the router. The list is
//     cut into one contiguous slice per XCD (workgroup b runs on XCD b % 8), so
//     the workgroups that run together on one XCD work on neighbouring tasks of
//     the same expert and share its weight slices in that XCD's L2; within the
//     list an expert's m-tiles go side by side along n (grouped_task);
//   * MFMA v_mfma_f32_32x32x16_bf16 with the weight rows as the MFMA "A"
//     operand and the token rows as "B" (output transposed in registers: each
//     lane ends up with four consecutive output columns of one token, which
//     become one 8-byte store);
//   * 8 waves per workgroup (two per SIMD, so one wave's MFMAs cover the other's
//     waits; 4 for 32-row tiles); every tile stages 256 weight rows (128 gate
//     + 128 up in GEMM1) against 256, 128, 64 or 32 sorted rows, the row-tile
//     size moe_pick_block_m chooses from the mean rows per expert; a wave holds
//     up to 128 accumulator registers, the most the register file leaves room
//     for;
//   * operands reach LDS by direct-to-LDS buffer loads (16 bytes a lane, 1 KB
//     a wave instruction), each k-step's LDS stage split: token rows in one
//     of two buffers, weight rows in one of three (the 256-row tiles take
//     exactly the 160 KB of LDS), so the weight rows, most of the L2 misses,
//     stream two k-steps ahead; every wave issues the same number of each
//     kind of load, and one exact wait count per step lets the newest weight
//     loads stay in flight across the barrier that starts the step;
//   * inside a k-step the MFMA fragments of the next 16-K substep are read
//     from LDS while the current substep's MFMAs run (order pinned with
//     scheduling-group barriers);
//   * LDS rows of BK bf16 with the 16-byte chunk index XOR-swizzled by row, so
//     the fragment reads of 8 consecutive rows fall on distinct chunks;
//   * GEMM1 keeps the gate rows n and up rows I + n of the same output column
//     in one workgroup, so SwiGLU runs in registers in the epilogue;
//   * what bounds it: on the Qwen3-30B-A3B shape the operand loads alone and
//     the MFMAs with their LDS fragment reads alone each take most of the
//     kernel time, and they overlap only partly; no single bandwidth is
//     saturated (a third of the loads miss L2; HBM runs at half of what a
//     pure stream reaches); the loads are bound by how far ahead they are
//     issued (a step waits on its slowest requests).
#include "moe_common.cuh"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kXcds = kSplitXcds;
constexpr int kGroup = 4;       // m-tiles of one expert that walk the n-tiles side by side
constexpr int kMinSplitSteps = 8;   // the last round is split along K only from 8 k-steps (K >= 512)
constexpr int kActSwiglu = 0;   // h = silu(gate) * up
constexpr int kActRelu2 = 1;    // h = max(g, 0)^2, one projection

template <int BM, int BN, int WM, int WN, bool GEMM1, int ACT>
struct Cfg {
  static constexpr int BK = 64;                       // bf16 per k-step: 128-byte LDS rows
  static constexpr int HALVES = GEMM1 && ACT == kActSwiglu ? 2 : 1;   // gate + up, or one projection
  static constexpr int B_ROWS = HALVES * BN;          // weight rows staged per k-step
  static constexpr int TM = BM / WM;                  // token rows per wave
  static constexpr int TN = BN / WN;                  // output columns per wave
  static constexpr int FM = TM / 32;
  static constexpr int FN = TN / 32;
  static constexpr int WAVES = WM * WN;
  static constexpr int THREADS = 64 * WAVES;
  // Split pipeline: the token rows of a k-step in one of two LDS buffers and
  // its weight rows in one of three, so the weight rows (most of the L2
  // misses) stream two k-steps ahead and the token rows one. Every wave
  // issues the same number of token and of weight loads per step (1 KB
  // direct-to-LDS loads, 8 rows each), which makes one wait count exact.
  static constexpr int T_BYTES = BM * 128, W_BYTES = B_ROWS * 128;
  static constexpr int T_GROUPS = BM / 8, W_GROUPS = B_ROWS / 8;
  static constexpr int GPW_T = T_GROUPS / WAVES;       // token loads per wave per k-step
  static constexpr int GPW_W = W_GROUPS / WAVES;       // weight loads per wave per k-step
  static constexpr int GPW = GPW_T + GPW_W;            // loads per wave per k-step
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile is a multiple of 32");
  static_assert(BM % 8 == 0 && T_GROUPS % WAVES == 0 && W_GROUPS % WAVES == 0, "uniform loads per wave");
  static_assert(2 * T_BYTES + 3 * W_BYTES <= 160 * 1024, "the split stages fit in LDS");
  static_assert(BN % (GPW_W * 8) == 0, "a wave's weight rows lie in one half (gate or up)");
};

// The XOR swizzle of the 16-byte chunks of LDS row `row`: row & 7, which
// spreads 8 consecutive rows over distinct chunks. gfx950's LDS has 64
// four-byte banks and a 16-byte read serves 16 lanes (16 rows) per sweep, so
// rows r and r + 8 still meet (two-way conflicts, half of the LDS-active
// cycles); the conflict-free (row >> 1) & 7 measured 1-2% slower on these
// kernels (same-process medians, Qwen3-30B-A3B and Nemotron shapes) and is
// used by the FP8 / MX and backward kernels, where it is neutral.
__device__ __forceinline__ int swz(int row) { return row & 7; }

// Byte offset of 16-byte chunk c of LDS row `row`.
__device__ __forceinline__ uint32_t lds_off(int row, int c) {
  return static_cast<uint32_t>(row * 128 + ((c ^ swz(row)) << 4));
}

__device__ __forceinline__ bf16x8 lds_frag(const char* base, int row, int chunk) {
  const uint4 v = *reinterpret_cast<const uint4*>(base + lds_off(row, chunk));
  return __builtin_bit_cast(bf16x8, v);
}

// Raw buffer accesses: a 32-bit byte offset against a descriptor whose range
// is one operand (or one expert's weights). An offset at or beyond the range
// reads as zeros, which is how pad rows, rows past N and the K tail become
// zeros without branches.
constexpr uint32_t kOob = 0x7FFFFFF0u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

// Cache policy of a buffer access with device-scope coherence (sc1), the
// policy the compiler gives device-scope atomic loads and stores.
constexpr int kDeviceScope = 16;

// The fused combine's y rows: written through with device-scope stores (the
// counts then only wait for the stores), or stored normally and made visible
// by a device-scope release fence (which writes back the XCD's whole L2).
constexpr bool kFuseWriteThrough = true;

struct Params {
  const uint16_t* a;       // GEMM1: x [T, H]; GEMM2: h [cap, I]
  const uint16_t* w;       // GEMM1: W1 [E, 2I, H] (SwiGLU) or [E, I, H] (ReLU2); GEMM2: W2 [E, H, I]
  const int32_t* sorted_ids;
  const int32_t* tile_expert;
  const int32_t* num_tiles;
  uint16_t* out;           // GEMM1: h [cap, I]; GEMM2: y [A, H]
  uint16_t* gu;            // GEMM1 (SwiGLU), optional: saved pre-activations [cap, 2I] (gate, up)
  float* h32;              // GEMM1, optional: the fp32 h before its bf16 rounding [cap, I]
  const float* topk_w;     // GEMM2 with the fused combine: gate weights [A]
  uint16_t* comb;          //   combined output [T, H]
  int32_t* counters;       //   [T, ceil(H / BN)] finished slots per (token, column tile); zero between calls
  int32_t* split_cnt;      // optional K-split of the last round: halves finished per slot; zero between calls
  float* split_part;       //   fp32 partial tiles, two per slot
  int32_t* queue;          // optional per-XCD item queues (claimed, finished); zero between calls
  int64_t A;
  uint32_t a_bytes;        // bytes of the token operand (below 2^31)
  int H, I, k;
  int n_begin, n_end;      // the launch covers output columns [n_begin, n_end) (multiples of 8)
};

// The weighted top-k combine fused into GEMM2 (TileScale PR #70, Design:
// "Kernel 2" runs L2, the scatter to (token, slot) rows and the reduce).
// Called by the whole workgroup after it has stored the y rows of its tile
// (sorted rows row0.., output columns [n0, n0 + BN)). Every real row bumps
// the counter of its (token, column tile); the workgroup that brings a
// counter to k stored the last of that token's k rows for these columns, so
// all k rows are complete: it sums them in fp32 in slot order (the same
// arithmetic as the separate combine, so the result is identical) and resets
// the counter to zero for the next call. The release fence before the count
// makes this workgroup's y rows visible to whichever workgroup finishes the
// token; the acquire fence after it makes the other workgroups' rows visible
// here. `last_tok` is LDS scratch of BM ints.
template <int BM, int BN, int THREADS>
__device__ __forceinline__ void fused_combine(const Params& p, int64_t row0, int nt, int ntn, int N,
                                              int32_t* last_tok) {
  constexpr int WAVES = THREADS / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = p.n_begin + nt * BN;
  const __amdgpu_buffer_rsrc_t yrs = make_rsrc(p.out, static_cast<uint32_t>(p.A * N * 2));
  if (kFuseWriteThrough) {
    wait_vmcnt<0>();   // this wave's y rows went out with device-scope stores: they are now visible
  } else {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  }
  __syncthreads();
  for (int r = tid; r < BM; r += THREADS) {
    const int sid = p.sorted_ids[row0 + r];
    int t = -1;
    if (sid < p.A) {
      const int tt = sid / p.k;
      int32_t* c = p.counters + static_cast<int64_t>(tt) * ntn + nt;
      if (__hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == p.k - 1) {
        t = tt;
        __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    last_tok[r] = t;
  }
  __syncthreads();
  // the other workgroups' rows are read with device-scope loads (past any
  // stale line in this XCD's L2), so no acquire fence invalidates the L2
  for (int r = wave; r < BM; r += WAVES) {
    const int t = last_tok[r];                 // the same for every lane of the wave
    if (t < 0) continue;
    const int64_t a0 = static_cast<int64_t>(t) * p.k;
    for (int c = lane * 8; c < BN; c += 512) {
      const int n = n0 + c;
      if (n >= N) break;
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
      for (int j = 0; j < p.k; ++j) {
        const float wj = p.topk_w[a0 + j];
        const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(yrs, static_cast<uint32_t>(((a0 + j) * N + n) * 2), 0,
                                                              kDeviceScope);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = __builtin_fmaf(wj, __uint_as_float(q[i] << 16), acc[2 * i]);
          acc[2 * i + 1] = __builtin_fmaf(wj, __uint_as_float(q[i] & 0xFFFF0000u), acc[2 * i + 1]);
        }
      }
      uint4 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      o.z = pack_bf16x2(acc[4], acc[5]);
      o.w = pack_bf16x2(acc[6], acc[7]);
      *reinterpret_cast<uint4*>(p.comb + static_cast<int64_t>(t) * N + n) = o;
    }
  }
  __syncthreads();   // last_tok is read before the next task's loads reuse the LDS
}

template <int BM, int BN, int WM, int WN, bool GEMM1, int ACT, bool FUSE = false>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_bf16_kernel(Params p) {
  using C = Cfg<BM, BN, WM, WN, GEMM1, ACT>;
  static_assert(!FUSE || !GEMM1, "the combine fuses into GEMM2");
  constexpr int BK = C::BK;
  // separate LDS arrays, so the compiler can tell the buffer being filled by
  // the direct-to-LDS loads from the one being read: two token buffers and
  // three weight buffers
  __shared__ __attribute__((aligned(1024))) char stage0[C::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char stage1[C::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char wst0[C::W_BYTES];
  __shared__ __attribute__((aligned(1024))) char wst1[C::W_BYTES];
  __shared__ __attribute__((aligned(1024))) char wst2[C::W_BYTES];

  // the wave index is uniform across the wave: keep it in a scalar register so
  // that the LDS destinations and descriptors of the loads are scalar too
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  // LDS byte offsets of this lane's MFMA fragments in substep kk of a k-step:
  // row wm * TM + lane % 32 (token) or wn * TN + lane % 32 (weight) at chunk
  // 2 kk + lane / 32. Fragment rows start at multiples of 32, so every
  // fragment row of a lane has the swizzle lane & 7 and the other fragments
  // of the substep sit at compile-time offsets (32-row steps) from these.
  uint32_t xo_t[Cfg<BM, BN, WM, WN, GEMM1, ACT>::BK / 16], xo_w[Cfg<BM, BN, WM, WN, GEMM1, ACT>::BK / 16];
#pragma unroll
  for (int kk = 0; kk < Cfg<BM, BN, WM, WN, GEMM1, ACT>::BK / 16; ++kk) {
    const uint32_t cb = static_cast<uint32_t>(((kk * 2 + (lane >> 5)) ^ (lane & 7)) << 4);
    xo_t[kk] = static_cast<uint32_t>((wm * Cfg<BM, BN, WM, WN, GEMM1, ACT>::TM + (lane & 31)) * 128) + cb;
    xo_w[kk] = static_cast<uint32_t>((wn * Cfg<BM, BN, WM, WN, GEMM1, ACT>::TN + (lane & 31)) * 128) + cb;
  }
  const int N = GEMM1 ? p.I : p.H;      // output columns
  const int K = GEMM1 ? p.H : p.I;      // reduction length
  const int ntn = (p.n_end - p.n_begin + BN - 1) / BN;
  const int num_tiles = *p.num_tiles;
  const int total = num_tiles * ntn;
  const int nk = (K + BK - 1) / BK;
  // this lane's place in a direct-to-LDS load: the load writes 64 x 16 bytes
  // contiguously, i.e. 8 LDS rows; lane l fills physical chunk l % 8 of row l / 8
  const int g_row = lane >> 3, g_pc = lane & 7;

  // XCD-aware slice of the flat task list
  const int G = gridDim.x;
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const int per_xcd = (G + kXcds - 1 - xcd) / kXcds;        // workgroups on this XCD
  // contiguous slice [t0, t1) of the task list for this XCD, proportional to its workgroups
  const int64_t t0 = static_cast<int64_t>(total) * (xcd * (G / kXcds) + (xcd < G % kXcds ? xcd : G % kXcds)) / G;
  const int64_t t1 = static_cast<int64_t>(total) *
                     ((xcd + 1) * (G / kXcds) + (xcd + 1 < G % kXcds ? xcd + 1 : G % kXcds)) / G;

  // The m-tiles of one expert walk the n-tiles side by side (groups of up to
  // kGroup, m fastest), so that the m-tiles that read the same weight slice
  // run together and share it in L2. (Token tiles are shared along n either
  // way.) Walking one m-tile's n-tiles in a row instead, so that the next
  // m-tile finds the slices still in L2, loses even when the walk is smaller
  // than an XCD's 4 MB L2: on the Qwen3-30B-A3B shape GEMM2's 3.1 MB walk ran
  // 322 us that way against 309 us grouped.
  //
  // Work balance: the slice's tasks go round robin over the XCD's
  // workgroups, so when the last round holds at most half as many tasks as
  // there are workgroups, most of them would idle through it. Given the split
  // workspace, each task of that round is then cut in two along K (items
  // 2j and 2j + 1 of the split range, k-steps [0, nk/2) and [nk/2, nk)), and
  // the workgroup that finishes second adds the two fp32 partial tiles and
  // runs the epilogue. Items are wave-uniform.
  //
  // With the workspace the items are also handed out dynamically: a
  // workgroup's first item is `local`, every further one is claimed from its
  // XCD's queue (an atomic counter) when the current item starts, so the
  // claim's latency hides behind the k-loop and workgroups that run faster
  // take more items, in the same order. Wave 0 makes the claim; the other
  // waves read it from LDS after the k-loop. The last workgroup of an XCD to
  // finish resets the XCD's counters for the next call; nothing waits.
  const bool dyn = p.queue != nullptr;
  int32_t* const qclaim = dyn ? p.queue + xcd * kQueueStride : nullptr;
  int32_t* const qdone = dyn ? qclaim + kQueueStride / 2 : nullptr;
  const int64_t nslice = t1 - t0;
  const int64_t rounds = nslice / per_xcd, left = nslice - rounds * per_xcd;
  const bool split = p.split_cnt != nullptr && left > 0 && 2 * left <= per_xcd && nk >= kMinSplitSteps;
  const int64_t nfull = split ? rounds * per_xcd : nslice;       // items below nfull are whole tasks
  const int64_t nitems = split ? nfull + 2 * left : nslice;
  auto task_of = [&](int64_t it) { return t0 + (it < nfull ? it : nfull + (it - nfull) / 2); };
  int probe = local < nitems ? grouped_probe(task_of(local), ntn, num_tiles, p.tile_expert, lane) : 0;
  int64_t it_next = 0;
  for (int64_t it = local; it < nitems; it = it_next) {
    const int64_t task = task_of(it);
    int32_t claimed = 0;   // wave 0, lane 0: the next item, per_xcd + the queue's count
    if (dyn && tid == 0) claimed = __hip_atomic_fetch_add(qclaim, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool part = it >= nfull;                  // half of a split task
    const int khalf = part ? static_cast<int>((it - nfull) & 1) : 0;
    const int kb = khalf ? nk / 2 : 0;              // k-steps [kb, ke) of this item
    const int ke = part && khalf == 0 ? nk / 2 : nk;
    int nt, mt, e;
    grouped_task<kGroup>(task, ntn, num_tiles, p.tile_expert, lane, probe, nt, mt, e);
    if (!dyn && it + per_xcd < nitems)
      probe = grouped_probe(task_of(it + per_xcd), ntn, num_tiles, p.tile_expert, lane);
    const int64_t row0 = static_cast<int64_t>(mt) * BM;
    // GEMM2: the destination rows of this lane's stores, loaded with the
    // task's first operand loads, so that the epilogue does not start with a
    // round trip (GEMM2 1-2% faster on the Qwen3, Scout and Nemotron shapes)
    int out_sid[C::FM];
#pragma unroll
    for (int i = 0; i < C::FM; ++i) out_sid[i] = GEMM1 ? 0 : p.sorted_ids[row0 + wm * C::TM + i * 32 + (lane & 31)];
    const int n0 = p.n_begin + nt * BN;

    // source of every LDS row this lane fills: a byte offset into the token
    // operand (rows < BM) or into expert e's weights (kOob: zeros)
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(p.a, p.a_bytes);
    const int wrows = GEMM1 ? C::HALVES * p.I : p.H;   // weight rows of one expert
    const __amdgpu_buffer_rsrc_t b_rsrc =
        make_rsrc(p.w + static_cast<int64_t>(e) * wrows * K, static_cast<uint32_t>(wrows) * K * 2);
    // This lane's place in every direct-to-LDS load: a load fills 8 LDS rows
    // (1 KB), lane l physical chunk l % 8 of row l / 8 of the group, and the
    // swizzle is row & 7, so every row this lane fills holds the same logical
    // chunk lc: one K column for all of the lane's loads. Keeping the per-load
    // bookkeeping to one offset per gathered token row (and none per weight
    // row) is what keeps the large tiles free of register spills.
    const int lc = g_pc ^ g_row;
    const int kcol = lc * 8;
    // token rows: GEMM1 gathers them by sorted id (every id this lane needs is
    // loaded before any is used, so the loads overlap), GEMM2 reads the sorted
    // rows in place; toff = byte offset of this lane's chunk of each token row
    // it fills (kOob for pad rows)
    uint32_t toff[C::GPW_T];
    {
      int sid[C::GPW_T];
#pragma unroll
      for (int q = 0; q < C::GPW_T; ++q)
        sid[q] = GEMM1 ? p.sorted_ids[row0 + (wave * C::GPW_T + q) * 8 + g_row] : 0;
#pragma unroll
      for (int q = 0; q < C::GPW_T; ++q) {
        int64_t src = -1;
        if (GEMM1) {
          if (sid[q] < p.A) src = sid[q] / p.k;
        } else {
          src = row0 + (wave * C::GPW_T + q) * 8 + g_row;
        }
        toff[q] = src < 0 ? kOob : static_cast<uint32_t>(src * K * 2 + lc * 16);
      }
    }
    // weight rows: a wave's groups are consecutive rows of one half (gate or
    // up; BN is a multiple of the rows one wave loads), 8 rows apart; rows at
    // or past column N read as zeros
    const int br0 = wave * C::GPW_W * 8;                       // the wave's first weight row (uniform)
    const int half = C::HALVES == 2 && br0 >= BN ? 1 : 0;
    const int nfirst = n0 + br0 - half * BN + g_row;           // output column of the lane's first row
    uint32_t woff[C::GPW_W];
#pragma unroll
    for (int q = 0; q < C::GPW_W; ++q)
      woff[q] = nfirst + q * 8 < N ? static_cast<uint32_t>(half * p.I + nfirst + q * 8) * K * 2 + lc * 16 : kOob;
    // split pipeline: the token loads of k-step kt into `tb`, the weight loads into `wb`
    auto load_t = [&](char* tb, int kt) {
      const uint32_t soff = static_cast<uint32_t>(kt) * BK * 2;
      // past K every chunk reads zeros: every offset here is below kOob (the
      // operands stay under 2 GiB), so max() with kOob is the out-of-range
      // offset (a plain max: the compiler branches around the loads on a select)
      const uint32_t klim = kt * BK + kcol < K ? 0u : kOob;
#pragma unroll
      for (int q = 0; q < C::GPW_T; ++q) {
        const uint32_t o = __builtin_elementwise_max(toff[q], klim);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr_t)(tb + (wave * C::GPW_T + q) * 1024), 16, o, soff,
                                                 0, 0);
      }
    };
    auto load_w = [&](char* wb, int kt) {
      const uint32_t soff = static_cast<uint32_t>(kt) * BK * 2;
      const uint32_t klim = kt * BK + kcol < K ? 0u : kOob;
#pragma unroll
      for (int q = 0; q < C::GPW_W; ++q) {
        const uint32_t o = __builtin_elementwise_max(woff[q], klim);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lds_ptr_t)(wb + (wave * C::GPW_W + q) * 1024), 16, o, soff,
                                                 0, 0);
      }
    };

    f32x16 acc[C::HALVES][C::FM][C::FN];
#pragma unroll
    for (int h = 0; h < C::HALVES; ++h)
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[h][i][j] = f32x16{};

    // the fragments of 16-K substep kk + 1 are read from LDS into the other
    // register set while the MFMAs of substep kk run, so the LDS latency
    // hides behind MFMA work instead of stalling the matrix pipe
    // `tbase`: the k-step's token rows; `wbase`: its weight rows
    auto compute = [&](const char* tbase, const char* wbase) {
      bf16x8 xf[2][C::FM], wf[2][C::HALVES][C::FN];
      // fragment row (32 i + lane % 32 of the wave's rows) at its substep's
      // chunk: the per-lane part xo_t / xo_w[kk] plus a compile-time offset
      auto read_frags = [&](int kk, int buf) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
          xf[buf][i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(tbase + xo_t[kk] + i * 32 * 128));
#pragma unroll
        for (int h = 0; h < C::HALVES; ++h)
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
            wf[buf][h][j] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const uint4*>(wbase + xo_w[kk] + (h * BN + j * 32) * 128));
      };
      read_frags(0, 0);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int cur = kk & 1;
        if (kk + 1 < BK / 16) read_frags(kk + 1, cur ^ 1);
#pragma unroll
        for (int h = 0; h < C::HALVES; ++h)
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
              acc[h][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cur][h][j], xf[cur][i], acc[h][i][j], 0, 0, 0);
      }
      // pin the interleave: the reads of substep 0, then per substep one
      // fragment read of the next substep after each MFMA
      constexpr int READS = C::FM + C::HALVES * C::FN, MFMAS = C::HALVES * C::FN * C::FM;
      constexpr int PAIRS = READS < MFMAS ? READS : MFMAS;
      __builtin_amdgcn_sched_group_barrier(0x100, READS, 0);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        if (kk + 1 < BK / 16) {
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
    };

    // k-step s reads tokens from buffer s % 2 and weights from buffer s % 3.
    // Issue order per step: tokens of s + 1, then weights of s + 2; so when
    // step s starts, everything but the newest GPW - GPW_T loads (the
    // weights of s + 1) has landed, tokens and weights of s included. The
    // barrier after that wait also means every wave has finished step
    // s - 1, whose buffers step s refills; the loads are issued ahead of the
    // MFMAs (the scheduling barrier keeps them there). Six steps repeat the
    // buffer pattern; the k-steps past the item's end are loaded (zeros past
    // K) but not computed.
    auto step = [&](char* tb, char* wb, char* tb_next, char* wb_next2, int s) {
      wait_vmcnt<C::GPW - C::GPW_T>();
      barrier_no_fence();
      load_t(tb_next, s + 1);
      load_w(wb_next2, s + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(tb, wb);
    };
    load_t(stage0, kb);
    load_w(wst0, kb);
    load_w(wst1, kb + 1);
    for (int kt = kb;; kt += 6) {
      step(stage0, wst0, stage1, wst2, kt);
      if (kt + 1 >= ke) break;
      step(stage1, wst1, stage0, wst0, kt + 1);
      if (kt + 2 >= ke) break;
      step(stage0, wst2, stage1, wst1, kt + 2);
      if (kt + 3 >= ke) break;
      step(stage1, wst0, stage0, wst2, kt + 3);
      if (kt + 4 >= ke) break;
      step(stage0, wst1, stage1, wst0, kt + 4);
      if (kt + 5 >= ke) break;
      step(stage1, wst2, stage0, wst1, kt + 5);
      if (kt + 6 >= ke) break;
    }
    // the loads issued past the end have landed and every wave is done
    // with LDS before the next task refills it
    wait_vmcnt<0>();
    barrier_no_fence();
    if (dyn) {
      // the claimed item, through wst2: the next item's first loads go to
      // stage0, wst0 and wst1, and wst2 is refilled only after its first
      // barrier, which every wave reaches after reading this
      int32_t* const slot_next = reinterpret_cast<int32_t*>(wst2);
      if (tid == 0) *slot_next = claimed;
      __syncthreads();
      const int32_t c = *slot_next;
      it_next = c >= 0 ? per_xcd + static_cast<int64_t>(c) : nitems;   // (a counter never zeroed: stop)
      if (it_next < nitems) probe = grouped_probe(task_of(it_next), ntn, num_tiles, p.tile_expert, lane);
    } else {
      it_next = it + per_xcd;
    }

    if (part) {
      // Both halves store their partial tile (lane-major f32x4 rows: whole
      // 1 KB wave rows) and count; the second to count adds the other half's
      // tile to its own (fp32 addition commutes, so the sum does not depend
      // on which half finishes first) and resets the counter for the next
      // call. The task's slot: items 2j, 2j + 1 of this XCD's split range.
      // The tiles move with the cache policy of device-scope atomics (sc1:
      // stores write through, loads bypass the non-coherent cache levels),
      // so the store waits (vmcnt 0) before the count are all the ordering
      // the exchange needs. Release / acquire fences at device scope would
      // instead write back and invalidate the whole L2 of the XCD, whose
      // other workgroups are still streaming their operands through it
      // (measured: a split GEMM1 slower than none).
      constexpr int NV = C::HALVES * C::FM * C::FN * 4;        // f32x4 per lane
      const int64_t slot = static_cast<int64_t>(xcd) * split_slots_per_xcd(G) + (it - nfull) / 2;
      const __amdgpu_buffer_rsrc_t prs =
          make_rsrc(p.split_part + slot * 2 * NV * C::THREADS * 4, static_cast<uint32_t>(2 * NV * C::THREADS * 16));
      const uint32_t mine = static_cast<uint32_t>((khalf * NV * C::THREADS + tid) * 16);
      const uint32_t other = static_cast<uint32_t>(((khalf ^ 1) * NV * C::THREADS + tid) * 16);
#pragma unroll
      for (int h = 0; h < C::HALVES; ++h)
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x4 v = {acc[h][i][j][4 * q], acc[h][i][j][4 * q + 1], acc[h][i][j][4 * q + 2],
                               acc[h][i][j][4 * q + 3]};
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), prs,
                                                     mine + (((h * C::FM + i) * C::FN + j) * 4 + q) * C::THREADS * 16,
                                                     0, kDeviceScope);
            }
      wait_vmcnt<0>();
      __syncthreads();
      int32_t* flag = reinterpret_cast<int32_t*>(stage0);        // LDS is free until the next task
      if (tid == 0) {
        const int32_t was = __hip_atomic_fetch_add(p.split_cnt + slot, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (was == 1) __hip_atomic_store(p.split_cnt + slot, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = was;
      }
      __syncthreads();
      if (*flag == 0) continue;   // the other half finishes the task (this was the workgroup's last item)
      // the other half's tile, 16 loads in flight at a time (one at a time,
      // each waited for, the 32 round trips took 15 us)
      constexpr int G16 = NV < 16 ? NV : 16;
      static_assert(NV % G16 == 0, "whole groups of loads");
#pragma unroll
      for (int c = 0; c < NV; c += G16) {
        f32x4 o[G16];
#pragma unroll
        for (int u = 0; u < G16; ++u)
          o[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               prs, other + (c + u) * C::THREADS * 16, 0, kDeviceScope));
#pragma unroll
        for (int u = 0; u < G16; ++u) {
          const int v = c + u, q = v % 4, j = v / 4 % C::FN, i = v / (4 * C::FN) % C::FM, h = v / (4 * C::FN * C::FM);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[h][i][j][4 * q + r] += o[u][r];
        }
      }
    }


    // epilogue: lane holds output columns 8*(v/4) + 4*(lane/32) + v%4 of token lane%32
    // (GEMM1: h = the activation, stored as bf16; GEMM2: Y rows scattered to
    // assignment order)
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      const int m = wm * C::TM + i * 32 + (lane & 31);
      int64_t dst_row;
      bool row_ok;
      if (GEMM1) {
        dst_row = row0 + m;
        row_ok = true;
      } else {
        const int sid = out_sid[i];
        row_ok = sid < p.A;
        dst_row = sid;
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        if constexpr (!GEMM1) {
          // Y: lanes r and r + 32 hold columns 8g .. 8g + 3 and 8g + 4 .. 8g + 7
          // of the same row. One lane swap per word (v_permlane32_swap trades
          // the upper lanes' first operand for the lower lanes' second) gives
          // lane r groups 0 and 1 whole and lane r + 32 groups 2 and 3, stored
          // 16 bytes at a time: half the store instructions of 8-byte pieces.
          uint32_t u[4][2], from_lo[2][2], from_hi[2][2];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            u[g][0] = pack_bf16x2(acc[0][i][j][4 * g], acc[0][i][j][4 * g + 1]);
            u[g][1] = pack_bf16x2(acc[0][i][j][4 * g + 2], acc[0][i][j][4 * g + 3]);
          }
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int w = 0; w < 2; ++w) {
              const auto r = __builtin_amdgcn_permlane32_swap(u[q][w], u[q + 2][w], false, false);
              from_lo[q][w] = r[0];   // upper lanes: the lower lane's u[q + 2][w]
              from_hi[q][w] = r[1];   // lower lanes: the upper lane's u[q][w]
            }
          const bool upper = lane >= 32;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int n = n0 + wn * C::TN + j * 32 + (upper ? q + 2 : q) * 8;
            const uint4 st = upper ? make_uint4(from_lo[q][0], from_lo[q][1], u[q + 2][0], u[q + 2][1])
                                   : make_uint4(u[q][0], u[q][1], from_hi[q][0], from_hi[q][1]);
            if (row_ok && n < N) {   // N % 8 == 0
              if (FUSE && kFuseWriteThrough)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, st),
                                                       make_rsrc(p.out, static_cast<uint32_t>(p.A * N * 2)),
                                                       static_cast<uint32_t>((dst_row * N + n) * 2), 0, kDeviceScope);
              else
                *reinterpret_cast<uint4*>(p.out + dst_row * N + n) = st;
            }
          }
        } else {
          // h: the activation of the four column groups, then the same lane
          // swap as Y above, so h is stored 16 bytes at a time
          float hv[4][4];
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float gv = acc[0][i][j][g * 4 + r];
              if (ACT == kActSwiglu) {
                const float uv = acc[C::HALVES - 1][i][j][g * 4 + r];
                hv[g][r] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
              } else {
                hv[g][r] = gv > 0.0f ? gv * gv : 0.0f;
              }
            }
          uint32_t u[4][2], from_lo[2][2], from_hi[2][2];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            u[g][0] = pack_bf16x2(hv[g][0], hv[g][1]);
            u[g][1] = pack_bf16x2(hv[g][2], hv[g][3]);
          }
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int w = 0; w < 2; ++w) {
              const auto r = __builtin_amdgcn_permlane32_swap(u[q][w], u[q + 2][w], false, false);
              from_lo[q][w] = r[0];
              from_hi[q][w] = r[1];
            }
          const bool upper = lane >= 32;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int n = n0 + wn * C::TN + j * 32 + (upper ? q + 2 : q) * 8;
            const uint4 st = upper ? make_uint4(from_lo[q][0], from_lo[q][1], u[q + 2][0], u[q + 2][1])
                                   : make_uint4(u[q][0], u[q][1], from_hi[q][0], from_hi[q][1]);
            if (n < N) *reinterpret_cast<uint4*>(p.out + dst_row * N + n) = st;   // N % 8 == 0
          }
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = n0 + wn * C::TN + j * 32 + g * 8 + (lane >> 5) * 4;
            if (n >= N) continue;
            if (p.h32 != nullptr)   // the values rounded to bf16 above, for checking that rounding
              *reinterpret_cast<f32x4*>(p.h32 + dst_row * N + n) = f32x4{hv[g][0], hv[g][1], hv[g][2], hv[g][3]};
            if (ACT == kActSwiglu && p.gu != nullptr) {
              // training forward: the gate and up pre-activations for the backward
              uint16_t* gr = p.gu + dst_row * 2 * N + n;
              *reinterpret_cast<uint2*>(gr) = make_uint2(pack_bf16x2(acc[0][i][j][g * 4], acc[0][i][j][g * 4 + 1]),
                                                         pack_bf16x2(acc[0][i][j][g * 4 + 2], acc[0][i][j][g * 4 + 3]));
              *reinterpret_cast<uint2*>(gr + N) =
                  make_uint2(pack_bf16x2(acc[C::HALVES - 1][i][j][g * 4], acc[C::HALVES - 1][i][j][g * 4 + 1]),
                             pack_bf16x2(acc[C::HALVES - 1][i][j][g * 4 + 2], acc[C::HALVES - 1][i][j][g * 4 + 3]));
            }
          }
        }
        // finish this block's accumulators before the next block's are read:
        // with the accumulators in AGPRs (four-wave tiles), reading them all
        // at once would need every VGPR and spill the task's load offsets
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (FUSE) fused_combine<BM, BN, C::THREADS>(p, row0, nt, ntn, N, reinterpret_cast<int32_t*>(stage1));
  }
  // the last workgroup of the XCD to get here (every one has made its final,
  // failing claim by then) resets the XCD's queue for the next call
  if (dyn && tid == 0 &&
      __hip_atomic_fetch_add(qdone, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == per_xcd - 1) {
    __hip_atomic_store(qclaim, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(qdone, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int BM, int BN, int WM, int WN, bool GEMM1, int ACT = kActSwiglu, bool FUSE = false>
hipError_t launch(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s, const CombineArgs* cmb = nullptr,
                  int n_begin = 0, int n_end = -1) {
  using C = Cfg<BM, BN, WM, WN, GEMM1, ACT>;
  Params p;
  p.topk_w = cmb ? cmb->topk_w : nullptr;
  p.comb = cmb ? cmb->out : nullptr;
  p.counters = cmb ? cmb->counters : nullptr;
  p.a = static_cast<const uint16_t*>(g.a);
  p.w = static_cast<const uint16_t*>(g.w);
  p.sorted_ids = g.sorted_ids;
  p.tile_expert = g.tile_expert;
  p.num_tiles = g.num_tiles;
  p.out = static_cast<uint16_t*>(g.out);
  p.gu = static_cast<uint16_t*>(g.out_scale);   // BF16 SwiGLU GEMM1: the optional saved pre-activations
  p.h32 = GEMM1 ? static_cast<float*>(g.h32) : nullptr;
  // the fused combine keeps whole tasks (its counters follow every tile's stores)
  static_assert(BM * C::HALVES * BN <= kSplitTileFloats, "a partial tile fits its workspace slot");
  p.split_cnt = !FUSE && g.split_ws ? static_cast<int32_t*>(g.split_ws) : nullptr;
  p.queue = !FUSE && g.split_ws ? reinterpret_cast<int32_t*>(static_cast<char*>(g.split_ws) + kQueueOffset) : nullptr;
  p.split_part = !FUSE && g.split_ws ? reinterpret_cast<float*>(static_cast<char*>(g.split_ws) + kWsCounterBytes)
                                     : nullptr;
  p.A = g.T * g.k;
  p.a_bytes = static_cast<uint32_t>((GEMM1 ? g.T * g.H : g.cap * g.I) * 2);
  p.H = g.H;
  p.I = g.I;
  p.k = g.k;
  const int N = GEMM1 ? g.I : g.H;
  p.n_begin = n_begin;
  p.n_end = n_end < 0 ? N : n_end;
  const int64_t max_tasks = (g.cap / BM) * ((p.n_end - n_begin + BN - 1) / BN);
  int64_t grid = dev.num_cus;
  if (grid > max_tasks) grid = max_tasks;
  if (grid < 1) grid = 1;
  gemm_bf16_kernel<BM, BN, WM, WN, GEMM1, ACT, FUSE><<<static_cast<unsigned>(grid), C::THREADS, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

bool gemm_bf16_supports(int block_m) { return block_m == 32 || block_m == 64 || block_m == 128 || block_m == 256; }

// A 256-row launch whose last column tile would be at most half full runs
// the whole tiles first and the rest with tiles half as wide. Used for the
// squared-ReLU GEMM1: at the Nemotron shape (I = 1856 = 7 x 256 + 64, T =
// 8192) it took 591 us against 614 for one launch (same-process medians).
// GEMM2 at H = 2688 = 10 x 256 + 128 was slower split (608 us against 597):
// its last tile is half full, not a quarter, and the second launch's own
// ramp-up and tail cost more than that saves.
template <int BN, class Wide, class Narrow>
hipError_t two_widths(int N, Wide wide, Narrow narrow) {
  const int rem = N % BN;
  if (N < BN || rem == 0 || rem > BN / 2) return wide(0, -1);
  const hipError_t e = wide(0, N - rem);
  return e != hipSuccess ? e : narrow(N - rem, N);
}

// Tiles: 256 rows x 128 output columns (128 gate + 128 up weight rows) for
// the largest row tile; 128- and 64-row tiles keep 256 weight rows a
// task too, so that their stages split (tokens double, weights triple
// buffered): wider tiles (512 weight rows, two whole stages) staged fewer
// bytes per MFMA but ran 3-18% slower (Qwen3-30B-A3B and Scout shapes at
// T = 1024 .. 4096). 32-row tiles run four waves (a token stage of 32 rows
// is four 1 KB loads, one a wave), which lets them split too (2-17% faster
// at T = 256 .. 512 than eight waves over 512 weight rows).
hipError_t launch_gemm1_bf16(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
  switch (g.block_m) {
    case 256: return launch<256, 128, 4, 2, true>(g, dev, s);
    case 128: return launch<128, 128, 2, 4, true>(g, dev, s);
    case 64: return launch<64, 128, 2, 4, true>(g, dev, s);
    case 32: return launch<32, 128, 1, 4, true>(g, dev, s);
    default: return hipErrorInvalidValue;
  }
}

// ReLU2: one projection per output column, so the tiles of GEMM2's shape
hipError_t launch_gemm1_relu2_bf16(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
  switch (g.block_m) {
    case 256:
      return two_widths<256>(
          g.I, [&](int a, int b) { return launch<256, 256, 4, 2, true, kActRelu2>(g, dev, s, nullptr, a, b); },
          [&](int a, int b) { return launch<256, 128, 4, 2, true, kActRelu2>(g, dev, s, nullptr, a, b); });
    case 128: return launch<128, 256, 2, 4, true, kActRelu2>(g, dev, s);
    case 64: return launch<64, 256, 2, 4, true, kActRelu2>(g, dev, s);
    case 32: return launch<32, 256, 1, 4, true, kActRelu2>(g, dev, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm2_bf16(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
  switch (g.block_m) {
    case 256: return launch<256, 256, 4, 2, false>(g, dev, s);
    case 128: return launch<128, 256, 2, 4, false>(g, dev, s);
    case 64: return launch<64, 256, 2, 4, false>(g, dev, s);
    case 32: return launch<32, 256, 1, 4, false>(g, dev, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm2_combine_bf16(const GemmArgs& g, const CombineArgs& c, const DeviceInfo& dev, hipStream_t s) {
  switch (g.block_m) {
    case 256: return launch<256, 256, 4, 2, false, kActSwiglu, true>(g, dev, s, &c);
    case 128: return launch<128, 256, 2, 4, false, kActSwiglu, true>(g, dev, s, &c);
    case 64: return launch<64, 256, 2, 4, false, kActSwiglu, true>(g, dev, s, &c);
    case 32: return launch<32, 256, 1, 4, false, kActSwiglu, true>(g, dev, s, &c);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
