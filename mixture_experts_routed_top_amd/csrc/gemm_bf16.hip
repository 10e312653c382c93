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

constexpr int kXcds = 8;
constexpr int kGroup = 4;       // m-tiles of one expert that walk the n-tiles side by side
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
  static constexpr int GPW = GPW_T + W_GROUPS / WAVES;  // loads per wave per k-step
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile is a multiple of 32");
  static_assert(BM % 8 == 0 && T_GROUPS % WAVES == 0 && W_GROUPS % WAVES == 0, "uniform loads per wave");
  static_assert(2 * T_BYTES + 3 * W_BYTES <= 160 * 1024, "the split stages fit in LDS");
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

struct Params {
  const uint16_t* a;       // GEMM1: x [T, H]; GEMM2: h [cap, I]
  const uint16_t* w;       // GEMM1: W1 [E, 2I, H] (SwiGLU) or [E, I, H] (ReLU2); GEMM2: W2 [E, H, I]
  const int32_t* sorted_ids;
  const int32_t* tile_expert;
  const int32_t* num_tiles;
  uint16_t* out;           // GEMM1: h [cap, I]; GEMM2: y [A, H]
  uint16_t* gu;            // GEMM1 (SwiGLU), optional: saved pre-activations [cap, 2I] (gate, up)
  const float* topk_w;     // GEMM2 with the fused combine: gate weights [A]
  uint16_t* comb;          //   combined output [T, H]
  int32_t* counters;       //   [T, ceil(H / BN)] finished slots per (token, column tile); zero between calls
  int64_t A;
  uint32_t a_bytes;        // bytes of the token operand (below 2^31)
  int H, I, k;
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
  const int n0 = nt * BN;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
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
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
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
        const uint4 q = *reinterpret_cast<const uint4*>(p.out + (a0 + j) * N + n);
        const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = __builtin_fmaf(wj, __uint_as_float(w4[i] << 16), acc[2 * i]);
          acc[2 * i + 1] = __builtin_fmaf(wj, __uint_as_float(w4[i] & 0xFFFF0000u), acc[2 * i + 1]);
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
  const int N = GEMM1 ? p.I : p.H;      // output columns
  const int K = GEMM1 ? p.H : p.I;      // reduction length
  const int ntn = (N + BN - 1) / BN;
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
  int probe = t0 + local < t1 ? grouped_probe(t0 + local, ntn, num_tiles, p.tile_expert, lane) : 0;
  for (int64_t task = t0 + local; task < t1; task += per_xcd) {
    int nt, mt, e;
    grouped_task<kGroup>(task, ntn, num_tiles, p.tile_expert, lane, probe, nt, mt, e);
    if (task + per_xcd < t1) probe = grouped_probe(task + per_xcd, ntn, num_tiles, p.tile_expert, lane);
    const int64_t row0 = static_cast<int64_t>(mt) * BM;
    const int n0 = nt * BN;

    // source of every LDS row this lane fills: a byte offset into the token
    // operand (rows < BM) or into expert e's weights (kOob: zeros)
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(p.a, p.a_bytes);
    const int wrows = GEMM1 ? C::HALVES * p.I : p.H;   // weight rows of one expert
    const __amdgpu_buffer_rsrc_t b_rsrc =
        make_rsrc(p.w + static_cast<int64_t>(e) * wrows * K, static_cast<uint32_t>(wrows) * K * 2);
    // byte offset of the start of LDS row `row`'s source row: a token row
    // (gathered by sorted id in GEMM1) or a weight row of expert e; kOob for
    // pad rows, rows past N and rows past the tile
    // (`sid`: the sorted id of a GEMM1 token row, loaded beforehand)
    auto row_src = [&](int row, int sid) -> uint32_t {
      if (row >= BM + C::B_ROWS) return kOob;
      if (row < BM) {
        int64_t src_row = -1;
        if (GEMM1) {
          if (sid < p.A) src_row = sid / p.k;
        } else {
          src_row = row0 + row;
        }
        return src_row < 0 ? kOob : static_cast<uint32_t>(src_row * K * 2);
      }
      const int br = row - BM;
      int n, wrow;
      if (GEMM1) {
        const int half = br >= BN ? 1 : 0;
        n = n0 + br - half * BN;
        wrow = half * p.I + n;
      } else {
        n = n0 + br;
        wrow = n;
      }
      return n < N ? static_cast<uint32_t>(wrow) * K * 2 : kOob;
    };
    uint32_t off[C::GPW];
    int kcol[C::GPW];                                   // first K column of this lane's chunk
    // load q of this wave fills the 8 LDS rows of group grp_of(q): in the
    // split pipeline the first GPW_T are token groups, the rest weight groups
    // (numbered from the first weight row)
    auto grp_of = [&](int q) -> int {
      return q < C::GPW_T ? wave * C::GPW_T + q : wave * (C::GPW - C::GPW_T) + (q - C::GPW_T);
    };
    auto row_of = [&](int q) -> int { return grp_of(q) * 8 + g_row + (q >= C::GPW_T ? BM : 0); };
    // GEMM1 gathers its token rows by sorted id: every id this lane needs is
    // loaded before any is used, so the loads overlap instead of each one
    // waiting for the last (a weight row loads a harmless id too)
    int sid[C::GPW];
#pragma unroll
    for (int q = 0; q < C::GPW; ++q) {
      const int row = row_of(q);
      sid[q] = GEMM1 ? p.sorted_ids[row0 + (row < BM ? row : 0)] : 0;
    }
#pragma unroll
    for (int q = 0; q < C::GPW; ++q) {
      const int row = row_of(q);
      const int lc = g_pc ^ swz(row);                   // logical chunk stored at this place
      kcol[q] = lc * 8;
      const uint32_t base = row_src(row, sid[q]);
      off[q] = base == kOob ? kOob : base + lc * 16;
    }
    // split pipeline: the token loads of k-step kt into `tb`, the weight loads into `wb`
    auto load_t = [&](char* tb, int kt) {
      const uint32_t soff = static_cast<uint32_t>(kt) * BK * 2;
#pragma unroll
      for (int q = 0; q < C::GPW_T; ++q) {
        const uint32_t o = kt * BK + kcol[q] < K ? off[q] : kOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr_t)(tb + grp_of(q) * 1024), 16, o, soff, 0, 0);
      }
    };
    auto load_w = [&](char* wb, int kt) {
      const uint32_t soff = static_cast<uint32_t>(kt) * BK * 2;
#pragma unroll
      for (int q = C::GPW_T; q < C::GPW; ++q) {
        const uint32_t o = kt * BK + kcol[q] < K ? off[q] : kOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lds_ptr_t)(wb + grp_of(q) * 1024), 16, o, soff, 0, 0);
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
      auto read_frags = [&](int kk, int buf) {
        const int ch = kk * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < C::FM; ++i) xf[buf][i] = lds_frag(tbase, wm * C::TM + i * 32 + (lane & 31), ch);
#pragma unroll
        for (int h = 0; h < C::HALVES; ++h)
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
            wf[buf][h][j] = lds_frag(wbase, h * BN + wn * C::TN + j * 32 + (lane & 31), ch);
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
    // buffer pattern; the k-steps past the end load zeros and are not computed.
    auto step = [&](char* tb, char* wb, char* tb_next, char* wb_next2, int s) {
      wait_vmcnt<C::GPW - C::GPW_T>();
      barrier_no_fence();
      load_t(tb_next, s + 1);
      load_w(wb_next2, s + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(tb, wb);
    };
    load_t(stage0, 0);
    load_w(wst0, 0);
    load_w(wst1, 1);
    for (int kt = 0;; kt += 6) {
      step(stage0, wst0, stage1, wst2, kt);
      if (kt + 1 >= nk) break;
      step(stage1, wst1, stage0, wst0, kt + 1);
      if (kt + 2 >= nk) break;
      step(stage0, wst2, stage1, wst1, kt + 2);
      if (kt + 3 >= nk) break;
      step(stage1, wst0, stage0, wst2, kt + 3);
      if (kt + 4 >= nk) break;
      step(stage0, wst1, stage1, wst0, kt + 4);
      if (kt + 5 >= nk) break;
      step(stage1, wst2, stage0, wst1, kt + 5);
      if (kt + 6 >= nk) break;
    }
    // the loads issued past the end have landed and every wave is done
    // with LDS before the next task refills it
    wait_vmcnt<0>();
    barrier_no_fence();


    // epilogue: lane holds output columns 8*(v/4) + 4*(lane/32) + v%4 of token lane%32
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      const int m = wm * C::TM + i * 32 + (lane & 31);
      int64_t dst_row;
      bool row_ok;
      if (GEMM1) {
        dst_row = row0 + m;
        row_ok = true;
      } else {
        const int sid = p.sorted_ids[row0 + m];
        row_ok = sid < p.A;
        dst_row = sid;
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * C::TN + j * 32 + g * 8 + (lane >> 5) * 4;
          float o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float gv = acc[0][i][j][g * 4 + r];
            if (GEMM1 && ACT == kActSwiglu) {
              const float uv = acc[C::HALVES - 1][i][j][g * 4 + r];
              o[r] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
            } else if (GEMM1) {
              o[r] = gv > 0.0f ? gv * gv : 0.0f;
            } else {
              o[r] = gv;
            }
          }
          if (row_ok && n < N) {
            uint2 st;
            st.x = pack_bf16x2(o[0], o[1]);
            st.y = pack_bf16x2(o[2], o[3]);
            *reinterpret_cast<uint2*>(p.out + dst_row * N + n) = st;
            if (GEMM1 && ACT == kActSwiglu && p.gu != nullptr) {
              // training forward: the gate and up pre-activations for the backward
              const float gv[4] = {acc[0][i][j][g * 4], acc[0][i][j][g * 4 + 1], acc[0][i][j][g * 4 + 2],
                                   acc[0][i][j][g * 4 + 3]};
              const float uv[4] = {acc[C::HALVES - 1][i][j][g * 4], acc[C::HALVES - 1][i][j][g * 4 + 1],
                                   acc[C::HALVES - 1][i][j][g * 4 + 2], acc[C::HALVES - 1][i][j][g * 4 + 3]};
              uint16_t* gr = p.gu + dst_row * 2 * N + n;
              *reinterpret_cast<uint2*>(gr) = make_uint2(pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3]));
              *reinterpret_cast<uint2*>(gr + N) = make_uint2(pack_bf16x2(uv[0], uv[1]), pack_bf16x2(uv[2], uv[3]));
            }
          }
        }
      }
    }
    if constexpr (FUSE) fused_combine<BM, BN, C::THREADS>(p, row0, nt, ntn, N, reinterpret_cast<int32_t*>(stage1));
  }
}

template <int BM, int BN, int WM, int WN, bool GEMM1, int ACT = kActSwiglu, bool FUSE = false>
hipError_t launch(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s, const CombineArgs* cmb = nullptr) {
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
  p.A = g.T * g.k;
  p.a_bytes = static_cast<uint32_t>((GEMM1 ? g.T * g.H : g.cap * g.I) * 2);
  p.H = g.H;
  p.I = g.I;
  p.k = g.k;
  const int N = GEMM1 ? g.I : g.H;
  const int64_t max_tasks = (g.cap / BM) * ((N + BN - 1) / BN);
  int64_t grid = dev.num_cus;
  if (grid > max_tasks) grid = max_tasks;
  if (grid < 1) grid = 1;
  gemm_bf16_kernel<BM, BN, WM, WN, GEMM1, ACT, FUSE><<<static_cast<unsigned>(grid), C::THREADS, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

bool gemm_bf16_supports(int block_m) { return block_m == 32 || block_m == 64 || block_m == 128 || block_m == 256; }

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
    case 256: return launch<256, 256, 4, 2, true, kActRelu2>(g, dev, s);
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
