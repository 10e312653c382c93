// BF16 grouped GEMMs of the routed-expert MoE backward (the training pass of
// the forward in gemm_bf16.hip; the pages' follow-up work: Liger-Kernel PR
// #1463, MoEBenchmark results, forward and backward).
//
//   dH  (kDh):    dh[r, i]    = sum_c dY[r, c] W2[e, c, i], then the SwiGLU
//                 backward with the saved pre-activations (g, u) of row r:
//                 dGU[r, i] = dh u silu'(g), dGU[r, I + i] = dh silu(g)
//   dX  (kDx):    dx_row[a, c] = sum_n dGU[r, n] W1[e, n, c], written to the
//                 row of assignment a = sorted_ids[r] (pad rows dropped)
//   dW  (kWgrad): dW[e, n, m]  = sum over expert e's sorted rows r of
//                 P[r, m] Q[r, n] (dW2: P = h, Q = dY; dW1: P = x gathered into
//                 sorted rows, Q = dGU), fp32 output
//
// Every operand sits in memory with the reduction index K as its slow index
// for at least one side: the weights W[e] are [K, M] (M contiguous) in the
// dgrad GEMMs, and both sorted-row operands are [K = row, M or N] in the
// weight gradients. Such a tile is staged into LDS as it is in memory, rows
// of K, and the MFMA fragments (8 consecutive K per lane) are read from it
// with the gfx950 transposing LDS read ds_read_b64_tr_b16: within each group
// of 16 lanes, lane j addresses 4 consecutive columns of row kb + j/4
// (columns m0 + 4 (j % 4) ...), and lane i receives column m0 + i of rows
// kb .. kb + 3. The operand whose K is contiguous (the sorted rows of dY or
// dGU in the dgrad GEMMs) is staged and read as in the forward kernels.
//
// Pipeline, XCD-aware persistent task slices, zero-filled out-of-range
// buffer loads and the 8-wave 256 x 256 workgroup tile follow the forward
// BF16 kernels.
#include "moe_common.cuh"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kXcds = 8;
constexpr int kDh = 0;
constexpr int kDx = 1;
constexpr int kWgrad = 2;
constexpr uint32_t kOob = 0x7FFFFFF0u;
constexpr int kWgradGroupN = 8;   // weight gradients: n-tiles walked side by side (see the task order)
constexpr int kDgradGroup = 4;    // dgrad: row tiles of one expert walked side by side (see the task order)
constexpr int BK = 64;            // K per pipeline step
constexpr int BO = 256;           // output tile: M (and N) extent per workgroup
constexpr int WM = 4, WN = 2;     // waves along M and N
constexpr int WAVES = WM * WN;
constexpr int THREADS = 64 * WAVES;
constexpr int TM = BO / WM, TN = BO / WN;
constexpr int FM = TM / 32, FN = TN / 32;
constexpr int T_TILE = BK * BO * 2;      // a transposed tile: BK rows of K x BO columns
constexpr int N_TILE = BO * BK * 2;      // a K-contiguous tile: BO rows x BK
constexpr int STAGE = T_TILE + N_TILE;   // both tiles have the same size
constexpr int GROUPS = STAGE / 1024;     // 1 KB direct-to-LDS loads per step
constexpr int GPW = GROUPS / WAVES;
static_assert(T_TILE == N_TILE && GROUPS % WAVES == 0, "uniform loads per wave");
static_assert(2 * STAGE <= 160 * 1024 && 3 * T_TILE + 2 * N_TILE <= 160 * 1024 && GPW % 2 == 0,
              "two whole stages, or the split stages, fit in LDS");

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short v4s __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

// Transposed tile: row k of the tile (one K index), 16-byte chunk c of its
// BO columns; the chunk index is XOR-swizzled by 4 (k & 3) so that the four
// rows one 16-lane group reads land on distinct banks.
__device__ __forceinline__ uint32_t t_off(int k, int c) {
  return static_cast<uint32_t>(k * (BO * 2) + ((c ^ ((k & 3) << 2)) << 4));
}
// K-contiguous tile: row r (one output column of the N side), 16-byte chunk c
// of its BK elements, swizzled by (r / 2) % 8 as in the forward kernels: the
// 16 consecutive rows of one fragment read fill the 64 banks once.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ uint32_t n_off(int r, int c) {
  return static_cast<uint32_t>(r * (BK * 2) + ((c ^ swz(r)) << 4));
}

// Fragment of 8 consecutive K (k0 + 8 (lane / 32) ...) for column m_base +
// lane % 32 of a transposed tile, by two transposing reads of 4 K each.
__device__ __forceinline__ bf16x8 t_frag(const char* tile, int lane, int m_base, int k0) {
  const int g16 = lane >> 4, j = lane & 15;
  const int m0 = m_base + 16 * (g16 & 1) + 4 * (j & 3);
  const int kb = k0 + 8 * (g16 >> 1) + (j >> 2);
  const int c = m0 >> 3, half = (m0 & 7) * 2;            // 16-byte chunk and byte within it
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4s_ptr)(tile + t_off(kb, c) + half));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4s_ptr)(tile + t_off(kb + 4, c) + half));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ bf16x8 n_frag(const char* tile, int row, int chunk) {
  const uint4 v = *reinterpret_cast<const uint4*>(tile + n_off(row, chunk));
  return __builtin_bit_cast(bf16x8, v);
}

struct Params {
  const uint16_t* a;        // transposed operand: dgrad W [E, K, M]; wgrad P [cap, M]
  const uint16_t* b;        // dgrad: sorted rows [cap, K]; wgrad: Q [cap, N] (transposed)
  const uint16_t* gu;       // kDh: saved pre-activations [cap, 2M] (g in [0, M), u in [M, 2M))
  const int32_t* sorted_ids;
  const int32_t* tile_expert;
  const int32_t* num_tiles;
  const int32_t* offsets;   // kWgrad: padded expert offsets [E + 1]
  void* out;                // kDh: dGU [cap, 2M] bf16; kDx: dx rows [A, M] bf16; kWgrad: fp32 [E, N, M]
  int64_t A;
  int M, N, K, E, block_m;
  uint32_t a_bytes, b_bytes;  // bytes of the operands (below 2^31)
  uint32_t gu_bytes;          // kDh: bytes of gu and of dGU (below 2^31)
};

template <int MODE>
__global__ __launch_bounds__(THREADS, 1) void gemm_bwd_kernel(Params p) {
  constexpr bool WGRAD = MODE == kWgrad;
  // Weight gradients: the A tile of a step in one of three LDS buffers, the
  // B tile in one of two (160 KB), so A (the P rows the m-tiles walk, most of
  // the L2 misses) streams two steps ahead and B one. The dgrad kernels keep
  // two whole stages (A and B buffers 0 and 1): at 252-255 registers they
  // spill with the split pipeline's extra LDS addresses and ran 5-10% slower.
  // Separate arrays, so the compiler can tell the buffers being filled from
  // the ones being read.
  // (two stages: abuf0 / abuf1 hold a whole stage each, the A tile then the
  // B tile)
  constexpr bool SPLIT = WGRAD;
  __shared__ __attribute__((aligned(1024))) char abuf0[SPLIT ? T_TILE : STAGE];
  __shared__ __attribute__((aligned(1024))) char abuf1[SPLIT ? T_TILE : STAGE];
  __shared__ __attribute__((aligned(1024))) char abuf2[SPLIT ? T_TILE : 16];
  __shared__ __attribute__((aligned(1024))) char bbuf0[SPLIT ? N_TILE : 16];
  __shared__ __attribute__((aligned(1024))) char bbuf1[SPLIT ? N_TILE : 16];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int ntm = (p.M + BO - 1) / BO;
  // dgrad: tasks (row tile, m tile); wgrad: (expert, n tile, m tile)
  const int ntn_w = (p.N + BO - 1) / BO;
  const int64_t total = WGRAD ? static_cast<int64_t>(p.E) * ntn_w * ntm : static_cast<int64_t>(*p.num_tiles) * ntm;

  const int G = gridDim.x;
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const int per_xcd = (G + kXcds - 1 - xcd) / kXcds;
  const int64_t t0 = total * (xcd * (G / kXcds) + (xcd < G % kXcds ? xcd : G % kXcds)) / G;
  const int64_t t1 = total * ((xcd + 1) * (G / kXcds) + (xcd + 1 < G % kXcds ? xcd + 1 : G % kXcds)) / G;

  // dgrad task order: the row tiles of one expert (groups of up to
  // kDgradGroup) walk the weight slices side by side, so that the tasks that
  // read the same slice run together and share it in L2 (m fastest per row
  // tile read every slice once per row tile: twice the weight bytes on the
  // Scout shape); the tile-list probe is loaded one task ahead in the dx
  // kernel and when the task starts in the dGU kernel (carried across the
  // k-loop it needs one register more than that kernel has)
  const int num_rt = WGRAD ? 0 : *p.num_tiles;
  int probe = MODE == kDx && t0 + local < t1 ? grouped_probe(t0 + local, ntm, num_rt, p.tile_expert, lane) : 0;
  for (int64_t task = t0 + local; task < t1; task += per_xcd) {
    int e, m0, n0, nk;
    int64_t row0 = 0;          // dgrad: first sorted row of the row tile; wgrad: first row of expert e
    if (WGRAD) {
      // Within an expert the n-tiles go in groups of G, n fastest: the tasks
      // that run together share each P tile (m) and the group's Q tiles (n,
      // 2 MB for 512 rows) stay in L2 while the m-tiles pass; G = 1 is m
      // fastest, where every n-tile reads all of the expert's P rows again
      // (several MB, from beyond L2: 12x the algorithmic bytes on the Scout
      // shape) but the tasks that run together write whole rows of dW. Groups
      // of 8 paid where the M side has at least as many tiles as the N side
      // (Scout dW2, 32 x 20 tiles: 1490 -> 1370 us; Qwen3-30B-A3B dW1, 8 x 6:
      // 767 -> 726 us) and cost where it has fewer (Scout dW1, 20 x 64: 2552
      // -> 2793 us; Qwen3 dW2, 3 x 8, level), same-process medians.
      const int G = ntm >= ntn_w ? kWgradGroupN : 1;
      e = static_cast<int>(task / (static_cast<int64_t>(ntn_w) * ntm));
      const int rem = static_cast<int>(task - static_cast<int64_t>(e) * ntn_w * ntm);
      const int ng = rem / (G * ntm);
      const int gn = ntn_w - ng * G < G ? ntn_w - ng * G : G;
      const int loc = rem - ng * G * ntm;
      m0 = (loc / gn) * BO;
      n0 = (ng * G + loc % gn) * BO;
      row0 = p.offsets[e];
      nk = (p.offsets[e + 1] - p.offsets[e] + BK - 1) / BK;
    } else {
      int mt, rt;
      if (MODE == kDh) probe = grouped_probe(task, ntm, num_rt, p.tile_expert, lane);
      grouped_task<kDgradGroup>(task, ntm, num_rt, p.tile_expert, lane, probe, mt, rt, e);
      if (MODE == kDx && task + per_xcd < t1) probe = grouped_probe(task + per_xcd, ntm, num_rt, p.tile_expert, lane);
      m0 = mt * BO;
      row0 = static_cast<int64_t>(rt) * p.block_m;
      n0 = 0;
      nk = (p.K + BK - 1) / BK;
    }
    const int rows_e = WGRAD ? p.offsets[e + 1] - p.offsets[e] : 0;

    // A (transposed): dgrad W[e] rows of K; wgrad P rows of expert e
    const __amdgpu_buffer_rsrc_t a_rsrc =
        WGRAD ? make_rsrc(p.a, p.a_bytes)
              : make_rsrc(p.a + static_cast<int64_t>(e) * p.K * p.M, static_cast<uint32_t>(p.K) * p.M * 2);
    const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(p.b, p.b_bytes);

    // per-lane source of each 1 KB group: groups [0, GROUPS/2) fill the A
    // tile, the rest the B tile; every wave loads GPW/2 of each (load q < GPW/2
    // is an A group). A transposed tile row is BO * 2 = 512 bytes, so a group
    // covers 2 rows; a K-contiguous row is 128 bytes, 8 per group.
    // (two-stage pipeline: waves 0 .. WAVES/2 - 1 load A, the others B)
    auto grp_of = [&](int q) -> int {
      if (!SPLIT) return wave * GPW + q;
      return q < GPW / 2 ? wave * (GPW / 2) + q : GROUPS / 2 + wave * (GPW / 2) + (q - GPW / 2);
    };
    uint32_t off[GPW];
    int krow[GPW];                 // K row (transposed tiles) or K column of the chunk (K-contiguous tile)
#pragma unroll
    for (int q = 0; q < GPW; ++q) {
      const int grp = grp_of(q);
      off[q] = kOob;
      krow[q] = 0;
      const bool in_a = grp < GROUPS / 2;
      const int gl = in_a ? grp : grp - GROUPS / 2;
      if (in_a || WGRAD) {
        // transposed tile: row k = 2 gl + lane / 32, physical chunk lane % 32
        const int k = 2 * gl + (lane >> 5), pc = lane & 31;
        const int lc = pc ^ ((k & 3) << 2);
        const int col = (in_a ? m0 : n0) + lc * 8;
        const int width = in_a ? p.M : p.N;
        krow[q] = k;
        if (col < width) {
          if (WGRAD)
            off[q] = static_cast<uint32_t>((row0 + k) * width + col) * 2;
          else
            off[q] = static_cast<uint32_t>(k * width + col) * 2;
        }
      } else {
        // K-contiguous rows of the sorted operand: row r = 8 gl + lane / 8
        const int r = 8 * gl + (lane >> 3), pc = lane & 7;
        const int lc = pc ^ swz(r);
        krow[q] = lc * 8;
        off[q] = static_cast<uint32_t>((row0 + r) * p.K + lc * 8) * 2;
      }
    }
    // issue the loads of step kt: with the split pipeline the A loads
    // (q < GPW/2, a_side) or the B loads into `buf`; with two stages every
    // load of the wave, A groups into `buf`, B groups into `bbuf`. Rows /
    // columns past the end (and steps past the end) read zeros.
    auto load = [&](char* buf, int kt, bool a_side, char* bbuf = nullptr) {
#pragma unroll
      for (int q = SPLIT ? (a_side ? 0 : GPW / 2) : 0; q < (SPLIT ? (a_side ? GPW / 2 : GPW) : GPW); ++q) {
        const int grp = grp_of(q);
        const bool in_a = grp < GROUPS / 2;
        uint32_t o, soff;
        if (in_a || WGRAD) {
          const int width = in_a ? p.M : p.N;
          const int k = kt * BK + krow[q];
          const bool live = WGRAD ? k < rows_e : k < p.K;
          o = live ? off[q] : kOob;
          soff = static_cast<uint32_t>(kt) * BK * width * 2;
        } else {
          o = kt * BK + krow[q] < p.K ? off[q] : kOob;
          soff = static_cast<uint32_t>(kt) * BK * 2;
        }
        const __amdgpu_buffer_rsrc_t rsrc = in_a ? a_rsrc : b_rsrc;
        char* const dst = (in_a || SPLIT ? buf : bbuf) + (in_a ? grp : grp - GROUPS / 2) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)dst, 16, o, soff, 0, 0);
      }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    auto compute = [&](const char* ta, const char* tb) {
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        bf16x8 af[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = t_frag(ta, lane, wm * TM + i * 32, kk * 16);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const bf16x8 bf = WGRAD ? t_frag(tb, lane, wn * TN + j * 32, kk * 16)
                                  : n_frag(tb, wn * TN + j * 32 + (lane & 31), kk * 2 + (lane >> 5));
          // the weight gradient takes its N side as the MFMA A operand, so
          // that each lane holds one M index (contiguous in dW) of 16 N rows
#pragma unroll
          for (int i = 0; i < FM; ++i)
            acc[i][j] = WGRAD ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf, af[i], acc[i][j], 0, 0, 0)
                              : __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf, acc[i][j], 0, 0, 0);
        }
      }
    };

    // Step s reads A from buffer s % 3 and B from buffer s % 2. Issue order
    // per step: B of s + 1, then A of s + 2; so when step s starts, all but
    // the newest GPW/2 loads (A of s + 1) have landed, A and B of s
    // included, and after the barrier every wave is done with step s - 1,
    // whose buffers step s refills. Six steps repeat the buffer pattern; the
    // steps past the end load zeros and are not computed.
    auto step = [&](char* a, char* b, char* b_next, char* a_next2, int st) {
      wait_vmcnt<GPW / 2>();
      barrier_no_fence();
      load(b_next, st + 1, false);
      load(a_next2, st + 2, true);
      __builtin_amdgcn_sched_barrier(0);
      compute(a, b);
    };
    if constexpr (SPLIT) {
    load(bbuf0, 0, false);
    load(abuf0, 0, true);
    load(abuf1, 1, true);
    for (int kt = 0;; kt += 6) {
      step(abuf0, bbuf0, bbuf1, abuf2, kt);
      if (kt + 1 >= nk) break;
      step(abuf1, bbuf1, bbuf0, abuf0, kt + 1);
      if (kt + 2 >= nk) break;
      step(abuf2, bbuf0, bbuf1, abuf1, kt + 2);
      if (kt + 3 >= nk) break;
      step(abuf0, bbuf1, bbuf0, abuf2, kt + 3);
      if (kt + 4 >= nk) break;
      step(abuf1, bbuf0, bbuf1, abuf0, kt + 4);
      if (kt + 5 >= nk) break;
      step(abuf2, bbuf1, bbuf0, abuf1, kt + 5);
      if (kt + 6 >= nk) break;
    }
    // the loads issued past the end have landed and every wave is done with
    // LDS before the next task refills it
    wait_vmcnt<0>();
    barrier_no_fence();
    } else {
      // two stages: step s+1 streams into one while the MFMAs read the other
      load(abuf0, 0, true, abuf0 + T_TILE);
      __syncthreads();
      for (int kt = 0; kt < nk; kt += 2) {
        load(abuf1, kt + 1, true, abuf1 + T_TILE);
        __builtin_amdgcn_sched_barrier(0);
        compute(abuf0, abuf0 + T_TILE);
        __syncthreads();
        load(abuf0, kt + 2, true, abuf0 + T_TILE);
        __builtin_amdgcn_sched_barrier(0);
        compute(abuf1, abuf1 + T_TILE);
        __syncthreads();
      }
    }

    if constexpr (WGRAD) {
      // lane holds M index lane % 32 of N indices 8 (v / 4) + 4 (lane / 32) + v % 4:
      // each store writes 2 x 128 contiguous bytes of dW
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * TM + i * 32 + (lane & 31);
        if (m >= p.M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int n = n0 + wn * TN + j * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (n < p.N)
              static_cast<float*>(p.out)[(static_cast<int64_t>(e) * p.N + n) * p.M + m] = acc[i][j][v];
          }
      }
      continue;
    }
    // epilogue: lane holds M indices 8 (v / 4) + 4 (lane / 32) + v % 4 of N index lane % 32
    // (dx: the assignment rows of the lane's N indices, loaded together, and
    // branch-free buffer stores, so that the blocks do not wait one by one)
    int dx_sid[FN];
    __amdgpu_buffer_rsrc_t dx_rs = make_rsrc(p.out, 0);
    if constexpr (MODE == kDx) {
#pragma unroll
      for (int j = 0; j < FN; ++j) dx_sid[j] = p.sorted_ids[row0 + wn * TN + j * 32 + (lane & 31)];
      dx_rs = make_rsrc(p.out, static_cast<uint32_t>(p.A * p.M * 2));
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int nl = wn * TN + j * 32 + (lane & 31);
      if constexpr (MODE == kDh) {
        // dGU of this 32-row block: the saved pre-activations are all loaded
        // before the first is used, the results are packed in place into the
        // block's accumulators, and then all stored. (Loaded, computed and
        // stored one pair at a time, every pair waited for its loads, and the
        // registers' reuse made every pair wait for the stores before it too:
        // 32 dependent round trips a task.)
        // Buffer loads and stores with an out-of-range offset past column M
        // (zeros / dropped) keep the block free of branches.
        const int64_t r = row0 + nl;
        const __amdgpu_buffer_rsrc_t gu_rs = make_rsrc(p.gu, p.gu_bytes), o_rs = make_rsrc(p.out, p.gu_bytes);
        uint32_t goff[FM][4];
        i32x2 gq[FM][4], uq[FM][4];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int m = m0 + wm * TM + i * 32 + g * 8 + (lane >> 5) * 4;
            goff[i][g] = m < p.M ? static_cast<uint32_t>((r * 2 * p.M + m) * 2) : kOob;
            gq[i][g] = __builtin_amdgcn_raw_buffer_load_b64(gu_rs, goff[i][g], 0, 0);
            uq[i][g] = __builtin_amdgcn_raw_buffer_load_b64(gu_rs, goff[i][g] == kOob ? kOob : goff[i][g] + p.M * 2,
                                                            0, 0);
          }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const uint32_t gw[2] = {static_cast<uint32_t>(gq[i][g][0]), static_cast<uint32_t>(gq[i][g][1])};
            const uint32_t uw[2] = {static_cast<uint32_t>(uq[i][g][0]), static_cast<uint32_t>(uq[i][g][1])};
            float dg[4], du[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float dh = acc[i][j][g * 4 + v];
              const uint32_t gb = (gw[v >> 1] >> (16 * (v & 1))) & 0xFFFFu;
              const uint32_t ub = (uw[v >> 1] >> (16 * (v & 1))) & 0xFFFFu;
              const float gv = __uint_as_float(gb << 16), uv = __uint_as_float(ub << 16);
              const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gv));
              dg[v] = dh * uv * sg * (1.0f + gv * (1.0f - sg));
              du[v] = dh * gv * sg;
            }
            acc[i][j][g * 4] = __uint_as_float(pack_bf16x2(dg[0], dg[1]));
            acc[i][j][g * 4 + 1] = __uint_as_float(pack_bf16x2(dg[2], dg[3]));
            acc[i][j][g * 4 + 2] = __uint_as_float(pack_bf16x2(du[0], du[1]));
            acc[i][j][g * 4 + 3] = __uint_as_float(pack_bf16x2(du[2], du[3]));
          }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const i32x2 dgw = {__float_as_int(acc[i][j][g * 4]), __float_as_int(acc[i][j][g * 4 + 1])};
            const i32x2 duw = {__float_as_int(acc[i][j][g * 4 + 2]), __float_as_int(acc[i][j][g * 4 + 3])};
            __builtin_amdgcn_raw_buffer_store_b64(dgw, o_rs, goff[i][g], 0, 0);
            __builtin_amdgcn_raw_buffer_store_b64(duw, o_rs, goff[i][g] == kOob ? kOob : goff[i][g] + p.M * 2, 0, 0);
          }
        continue;
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (MODE == kDx) {
          // dx rows: lanes r and r + 32 hold the two 4-index halves of each
          // 8-index group (the guard m < M is uniform per group, as M % 8 ==
          // 0); one lane swap per word (v_permlane32_swap: the upper lanes'
          // first operand for the lower lanes' second) leaves lane r groups 0,
          // 1 and lane r + 32 groups 2, 3 whole, stored 16 bytes at a time
          const int mb = m0 + wm * TM + i * 32;
          const int sid = dx_sid[j];
          uint32_t o[4][2], from_lo[2][2], from_hi[2][2];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            o[g][0] = pack_bf16x2(acc[i][j][g * 4], acc[i][j][g * 4 + 1]);
            o[g][1] = pack_bf16x2(acc[i][j][g * 4 + 2], acc[i][j][g * 4 + 3]);
          }
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int w = 0; w < 2; ++w) {
              const auto x = __builtin_amdgcn_permlane32_swap(o[q][w], o[q + 2][w], false, false);
              from_lo[q][w] = x[0];
              from_hi[q][w] = x[1];
            }
          const bool upper = lane >= 32;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int m = mb + (upper ? q + 2 : q) * 8;
            const uint4 st = upper ? make_uint4(from_lo[q][0], from_lo[q][1], o[q + 2][0], o[q + 2][1])
                                   : make_uint4(o[q][0], o[q][1], from_hi[q][0], from_hi[q][1]);
            const uint32_t off = m < p.M && sid < p.A ? static_cast<uint32_t>((static_cast<int64_t>(sid) * p.M + m) * 2)
                                                      : kOob;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4v, st), dx_rs, off, 0, 0);
          }
          continue;
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int m = m0 + wm * TM + i * 32 + g * 8 + (lane >> 5) * 4;
          if (m >= p.M) continue;
          const float a4[4] = {acc[i][j][g * 4], acc[i][j][g * 4 + 1], acc[i][j][g * 4 + 2], acc[i][j][g * 4 + 3]};
          {
            const int sid = p.sorted_ids[row0 + nl];
            if (sid < p.A) {
              uint16_t* o = static_cast<uint16_t*>(p.out) + static_cast<int64_t>(sid) * p.M + m;
              *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(a4[0], a4[1]), pack_bf16x2(a4[2], a4[3]));
            }
          }
        }
      }
    }
  }
}

template <int MODE>
hipError_t launch(const Params& p, int64_t tasks, const DeviceInfo& dev, hipStream_t s) {
  int64_t grid = dev.num_cus;
  if (grid > tasks) grid = tasks;
  if (grid < 1) grid = 1;
  gemm_bwd_kernel<MODE><<<static_cast<unsigned>(grid), THREADS, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

bool gemm_bwd_supports(int block_m) { return block_m == 256; }

hipError_t launch_bwd_dh(const BwdArgs& g, const DeviceInfo& dev, hipStream_t s) {
  Params p{};
  p.a = static_cast<const uint16_t*>(g.w2);
  p.b = static_cast<const uint16_t*>(g.dy);
  p.gu = static_cast<const uint16_t*>(g.gu);
  p.sorted_ids = g.sorted_ids;
  p.tile_expert = g.tile_expert;
  p.num_tiles = g.num_tiles;
  p.out = g.dgu;
  p.A = g.A;
  p.M = g.I;
  p.N = g.block_m;
  p.K = g.H;
  p.E = g.E;
  p.block_m = g.block_m;
  p.b_bytes = static_cast<uint32_t>(g.cap * g.H * 2);
  p.gu_bytes = static_cast<uint32_t>(g.cap * 2 * g.I * 2);
  return launch<kDh>(p, (g.cap / g.block_m) * ((g.I + BO - 1) / BO), dev, s);
}

hipError_t launch_bwd_dx(const BwdArgs& g, const DeviceInfo& dev, hipStream_t s) {
  Params p{};
  p.a = static_cast<const uint16_t*>(g.w1);
  p.b = static_cast<const uint16_t*>(g.dgu);
  p.sorted_ids = g.sorted_ids;
  p.tile_expert = g.tile_expert;
  p.num_tiles = g.num_tiles;
  p.out = g.dx_rows;
  p.A = g.A;
  p.M = g.H;
  p.N = g.block_m;
  p.K = 2 * g.I;
  p.E = g.E;
  p.block_m = g.block_m;
  p.b_bytes = static_cast<uint32_t>(g.cap * 2 * g.I * 2);
  return launch<kDx>(p, (g.cap / g.block_m) * ((g.H + BO - 1) / BO), dev, s);
}

hipError_t launch_bwd_wgrad(const void* pm, const void* qn, int M, int N, const BwdArgs& g, float* dw,
                            const DeviceInfo& dev, hipStream_t s) {
  Params p{};
  p.a = static_cast<const uint16_t*>(pm);
  p.b = static_cast<const uint16_t*>(qn);
  p.offsets = g.offsets;
  p.num_tiles = g.num_tiles;
  p.out = dw;
  p.A = g.A;
  p.M = M;
  p.N = N;
  p.K = 0;
  p.E = g.E;
  p.block_m = g.block_m;
  p.a_bytes = static_cast<uint32_t>(g.cap * M * 2);
  p.b_bytes = static_cast<uint32_t>(g.cap * N * 2);
  return launch<kWgrad>(p, static_cast<int64_t>(g.E) * ((N + BO - 1) / BO) * ((M + BO - 1) / BO), dev, s);
}

}  // namespace moe
