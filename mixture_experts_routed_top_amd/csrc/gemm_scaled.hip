// Block-scaled grouped GEMMs on the gfx950 scaled f8f6f4 MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4), two numeric paths:
//
//  * FP8_BLOCK128 (TileScale PR #70, Design: FP8 E4M3 inputs and weights with
//    FP32 per-128 scales). The MFMA runs with unit E8M0 scales over one
//    128-wide K group (two 64-deep MFMAs into a fresh partial sum), then the
//    partial is promoted into the fp32 accumulator with the product of the
//    token's 1x128 scale and the weight's 128x128 block scale (the commit
//    notes of that PR keep the running sum in fp32: narrower accumulators lose
//    an order of magnitude of accuracy).
//  * MXFP4W_MXFP8A (FlashInfer PR #6465, Benchmark configuration: E2M1
//    weights carrying one shared scale per 32 K elements, E4M3 activations). The weights are E2M1, the
//    tokens E4M3, both with one E8M0 scale per 32 along K, which the MFMA
//    applies itself: each lane passes the scale of the 32-element K block it
//    holds ("GC-MoE on SM120", Abstract: FP4 weights on one operand, FP8
//    activations on the other, scale bytes chosen per instruction).
//
// Shared structure with the BF16 kernels: persistent workgroups over one flat
// (m-tile, n-tile) task list read from device memory; the weight rows are the
// MFMA "A" operand and the token rows "B", so each lane ends up with four
// consecutive output columns of one token; GEMM1 keeps gate row n and up row
// I + n in one workgroup and applies SwiGLU and the requantisation of h in
// registers (TileScale PR #70, commit notes: quantise straight from the
// fp32 accumulator into the store path); GEMM2 scatters bf16 rows to
// assignment order (FlashInfer PR #5129, Description).
//
// Operand layout of the 32x32x64 scaled MFMA (measured on gfx950 with an
// in-bounds probe of single MFMAs): an E2M1 operand in lane half h holds the
// 32 consecutive K elements 32h..32h+31 of its row (low nibble first); an
// E4M3 operand in lane half h holds K elements 16h..16h+15 in bytes 0..15 and
// 32+16h..32+16h+15 in bytes 16..31; the E8M0 scale passed by lane half h
// scales K block h (elements 32h..32h+31). The fragment reads below follow it.
//
// One k-step stages 128 K elements: a 128-byte token row (E4M3), a 128-byte
// (E4M3) or 64-byte (E2M1) weight row, and one 32-bit scale word per row
// (the fp32 1x128 token scale, or four E8M0 bytes). The 64- to 256-row tiles
// split each k-step's LDS stage as the BF16 kernels do: token rows and their
// scale words in one of two buffers, weight rows (with their MX scale words)
// in one of three, so that the weight rows, most of the L2 misses, stream two
// k-steps ahead, with one exact wait count per step (FP8 GEMM2 on the
// 64-expert H 7168 shape 1517 -> 1437 us at T = 8192, 232 -> 209 us at
// T = 512; MX T = 16384 GEMM1 807 -> 772 us, GEMM2 541 -> 513 us; same
// process). The 32-row tiles keep whole stages, double (MX) or quadruple
// (FP8) buffered, and so does the 256-row FP8 GEMM1 tile, whose split stages
// would need 162 KB of LDS (with its token scales in registers instead they
// fit in 160 KB, but ran 13% slower). 16-byte chunks are XOR-swizzled per
// row so that the fragment reads of 16 consecutive rows fall on distinct
// banks. The 32-row MX GEMM1 tile (small token counts, bound by the weight
// stream) stages two such k-steps at once:
// a 64-byte E2M1 slice is half an L2 line, and the number of requests a CU
// keeps in flight, not their size, limits the stream, so whole 128-byte
// weight slices carry twice the bytes per request.
#include "moe_common.cuh"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kXcds = 8;
constexpr int kGroup = 4;       // m-tiles of one expert that walk the n-tiles side by side
constexpr int kFp8Block = 1;
constexpr int kMx = 2;

// One row's 32 E4M3 codes of a 32-column fragment, held as in the MFMA
// output: lane r (< 32) has columns 8g .. 8g + 3 in q[g], lane r + 32 has
// columns 8g + 4 .. 8g + 7. One lane swap per pair of words
// (v_permlane32_swap: the upper lanes' first operand for the lower lanes'
// second) gives lane r columns 0 .. 15 and lane r + 32 columns 16 .. 31,
// each stored with one 16-byte store at dst (16-byte aligned). Called by
// every lane of the wave.
__device__ __forceinline__ void store_codes_x32(uint8_t* dst, const uint32_t (&q)[4], int lane) {
  const auto a = __builtin_amdgcn_permlane32_swap(q[0], q[2], false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(q[1], q[3], false, false);
  if (lane < 32)
    *reinterpret_cast<uint4*>(dst) = make_uint4(q[0], a[1], q[1], b[1]);
  else
    *reinterpret_cast<uint4*>(dst + 16) = make_uint4(a[0], q[2], b[0], q[3]);
}

template <int BM, int BN, int WM, int WN, bool GEMM1, int MODE, int NST_ = 2, int KSUB_ = 1>
struct Cfg {
  // LDS stages: 2 or 4 whole stages, or 3 = split: the token rows of a k-step
  // with their scale words in one of two buffers, its weight rows (with
  // their MX scale words) in one of three, so that the weight rows stream two
  // k-steps ahead
  static constexpr int NST = NST_;
  static constexpr bool SPLIT = NST_ == 3;
  // 128-K substeps per stage. MX stages two, so that a weight row's slice is
  // 128 bytes (256 E2M1): one whole L2 line per request instead of two halves
  static constexpr int KSUB = KSUB_;
  static constexpr int W_BYTES = MODE == kMx ? 64 * KSUB : 128;   // weight row bytes per stage
  static constexpr int B_ROWS = GEMM1 ? 2 * BN : BN;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int HALVES = GEMM1 ? 2 : 1;
  static constexpr int WAVES = WM * WN;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int A_SUB = BM * 128;                      // token rows of one substep
  static constexpr int A_REGION = A_SUB * KSUB;
  static constexpr int W_REGION = B_ROWS * W_BYTES;
  static constexpr int A_GROUPS_SUB = BM / 8;                 // 1 KB direct-to-LDS loads of token rows
  static constexpr int A_GROUPS = A_GROUPS_SUB * KSUB;
  static constexpr int W_GROUPS = W_REGION / 1024;            // ... of weight rows
  static constexpr int GROUPS = A_GROUPS + W_GROUPS;
  static constexpr int GPW = (GROUPS + WAVES - 1) / WAVES;    // data loads per wave per k-step
  // scale words per k-step: token rows (padded to whole 64-row groups, so that
  // one load never mixes the two operands), then (MX) weight rows
  static constexpr int S_TOK = (BM + 63) / 64 * 64;
  static constexpr int S_ROWS = S_TOK + (MODE == kMx ? B_ROWS : 0);
  static constexpr int S_GROUPS_SUB = (S_ROWS + 63) / 64;     // 256 B direct-to-LDS loads of scale words
  static constexpr int S_GROUPS = S_GROUPS_SUB * KSUB;
  static constexpr int SPW = (S_GROUPS + WAVES - 1) / WAVES;
  static constexpr int STAGE = A_REGION + W_REGION + S_GROUPS * 256;
  // split stages: token buffer = token rows + their scale words, weight
  // buffer = weight rows + (MX) their scale words; every wave issues GPW_T
  // token, SPW_T token-scale, GPW_W weight and SPW_W weight-scale loads a
  // k-step (spare scale slots load into a sink)
  static constexpr int S_TOK_G = S_TOK / 64, S_W_G = MODE == kMx ? B_ROWS / 64 : 0;
  static constexpr int T_BUF = A_REGION + S_TOK_G * 256, W_BUF = W_REGION + S_W_G * 256;
  static constexpr int GPW_T = A_GROUPS / WAVES, GPW_W = W_GROUPS / WAVES;
  static constexpr int SPW_T = (S_TOK_G + WAVES - 1) / WAVES, SPW_W = (S_W_G + WAVES - 1) / WAVES;
  static constexpr int LDS_STAGES = SPLIT ? 2 * T_BUF + 3 * W_BUF + 1024 : NST * STAGE + (NST > 2 ? 1024 : 0);
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile is a multiple of 32");
  static_assert(BM % 8 == 0 && W_REGION % 1024 == 0, "whole 1 KB load groups");
  // FP8: a wave's weight rows must lie in one 128-row scale block: tiles start
  // on multiples of BN, so BN a multiple of 128 (or 128 a multiple of BN) and
  // TN dividing 128 keep every wave's rows inside one block
  static_assert(MODE != kFp8Block || (TN <= 128 && 128 % TN == 0 && (BN % 128 == 0 || 128 % BN == 0)),
                "a wave's weight rows share one 128x128 scale block");
  static_assert(NST == 2 || NST == 3 || NST == 4, "double, split or quadruple buffering");
  static_assert(!SPLIT || (KSUB == 1 && A_GROUPS % WAVES == 0 && W_GROUPS % WAVES == 0 && B_ROWS % 64 == 0),
                "split stages: one substep, the same token and weight loads in every wave");
  static_assert(KSUB == 1 || (KSUB == 2 && MODE == kMx && NST == 2), "two substeps: MX, double buffered");
  static_assert(LDS_STAGES + WN * BM * 4 <= 160 * 1024, "the stages fit in LDS");
  static_assert((NST - 2) * (GPW + SPW) < 64, "outstanding loads fit the counter");
};

// XOR swizzles of the 16-byte chunks of an LDS row. gfx950's LDS has 64
// four-byte banks (256 bytes), and a 16-byte fragment read serves 16 lanes,
// 16 consecutive rows at one logical chunk, per bank sweep. 128-byte rows:
// rows 2j and 2j + 1 share the swizzle j (the even and the odd rows each
// reach 8 distinct chunks); 64-byte rows: rows 4j .. 4j + 3 share j.
__device__ __forceinline__ int swz128(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz64(int row) { return (row >> 2) & 3; }

__device__ __forceinline__ uint32_t a_off(int row, int c) {
  return static_cast<uint32_t>(row * 128 + ((c ^ swz128(row)) << 4));
}

template <int W_BYTES>
__device__ __forceinline__ uint32_t w_off(int row, int c) {
  if (W_BYTES == 128) return static_cast<uint32_t>(row * 128 + ((c ^ swz128(row)) << 4));
  return static_cast<uint32_t>(row * 64 + ((c ^ swz64(row)) << 4));
}

__device__ __forceinline__ i32x8 frag32(const char* p0, const char* p1) {
  const uint4 lo = *reinterpret_cast<const uint4*>(p0);
  const uint4 hi = *reinterpret_cast<const uint4*>(p1);
  return i32x8{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
               static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
}

__device__ __forceinline__ i32x8 frag16(const char* p) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  return i32x8{static_cast<int>(q.x), static_cast<int>(q.y), static_cast<int>(q.z), static_cast<int>(q.w),
               0, 0, 0, 0};
}

// Raw buffer accesses: a 32-bit byte offset against a descriptor covering one
// operand (or one expert's weights); offsets at or past the range read zeros.
constexpr uint32_t kOob = 0x7FFFFFF0u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(4))) const float* const_f32_ptr;   // read-only global memory

// Issue the direct-to-LDS loads of k-step kt into `stage`: the token and
// weight tiles in 1 KB groups (16 bytes a lane), then the k-step's scale words
// in 256 B groups (4 bytes a lane). k-steps past the end read zeros. With more
// than two stages every wave issues the same number of loads, GPW + SPW, so
// that one wait count fits all: a slot without a group loads zeros into
// `sink`, an LDS area nobody reads.
template <class C>
__device__ __forceinline__ void issue_loads(char* stage, char* sink, int kt, int nk, int nk128, int wave,
                                            __amdgpu_buffer_rsrc_t a_rsrc, __amdgpu_buffer_rsrc_t w_rsrc,
                                            __amdgpu_buffer_rsrc_t as_rsrc, __amdgpu_buffer_rsrc_t ws_rsrc,
                                            const uint32_t (&doff)[C::GPW], const uint32_t (&soff)[C::SPW],
                                            const uint32_t (&dsub)[C::GPW]) {
  constexpr bool kUniform = C::NST > 2;
  const bool live = kt < nk;
#pragma unroll
  for (int q = 0; q < C::GPW; ++q) {
    const int g = wave * C::GPW + q;
    const bool real = C::GROUPS % C::WAVES == 0 || g < C::GROUPS;
    if (real || kUniform) {
      const bool tok = g < C::A_GROUPS;
      const int ks = kt * C::KSUB + (tok ? g / C::A_GROUPS_SUB : 0);   // 128-K substep of a token group
      const __amdgpu_buffer_rsrc_t rsrc = tok ? a_rsrc : w_rsrc;
      char* const dst = real ? stage + g * 1024 : sink;
      // a weight chunk of the second substep past K (K ends inside the stage) is not fetched
      const bool ok = tok ? ks < nk128 : live && (C::KSUB == 1 || kt * C::KSUB + static_cast<int>(dsub[q]) < nk128);
      const uint32_t voff = ok && real ? doff[q] : kOob;
      const uint32_t soffset = tok ? static_cast<uint32_t>(ks) * 128 : static_cast<uint32_t>(kt) * C::W_BYTES;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)dst, 16, voff, soffset, 0, 0);
    }
  }
#pragma unroll
  for (int q = 0; q < C::SPW; ++q) {
    const int g = wave + q * C::WAVES;
    const bool real = g < C::S_GROUPS;
    if (real || kUniform) {
      const int gs = g % C::S_GROUPS_SUB, ks = kt * C::KSUB + g / C::S_GROUPS_SUB;
      const __amdgpu_buffer_rsrc_t rsrc = gs * 64 < C::S_TOK ? as_rsrc : ws_rsrc;
      char* const dst = real ? stage + C::A_REGION + C::W_REGION + g * 256 : sink;
      const uint32_t voff = ks < nk128 && real ? soff[q] : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)dst, 4, voff, static_cast<uint32_t>(ks) * 4, 0, 0);
    }
  }
}

// Split stages: the direct-to-LDS loads of k-step kt's token rows (1 KB
// groups) and their scale words (256 B groups) into token buffer `tb`, and of
// its weight rows and (MX) their scale words into weight buffer `wb`. A wave
// without a scale group of its own loads zeros into `sink`, so that every
// wave issues the same count. k-steps past the end read zeros.
template <class C>
__device__ __forceinline__ void issue_split_tokens(char* tb, char* sink, int kt, int nk, int wave,
                                                   __amdgpu_buffer_rsrc_t a_rsrc, __amdgpu_buffer_rsrc_t as_rsrc,
                                                   const uint32_t (&toff)[C::GPW_T],
                                                   const uint32_t (&tsoff)[C::SPW_T]) {
  const bool live = kt < nk;
#pragma unroll
  for (int q = 0; q < C::GPW_T; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr_t)(tb + (wave * C::GPW_T + q) * 1024), 16,
                                             live ? toff[q] : kOob, static_cast<uint32_t>(kt) * 128, 0, 0);
#pragma unroll
  for (int q = 0; q < C::SPW_T; ++q) {
    const int g = wave + q * C::WAVES;
    const bool real = g < C::S_TOK_G;
    char* const dst = real ? tb + C::A_REGION + g * 256 : sink;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(as_rsrc, (lds_ptr_t)dst, 4, live && real ? tsoff[q] : kOob,
                                             static_cast<uint32_t>(kt) * 4, 0, 0);
  }
}

template <class C>
__device__ __forceinline__ void issue_split_weights(char* wb, char* sink, int kt, int nk, int wave,
                                                    __amdgpu_buffer_rsrc_t w_rsrc, __amdgpu_buffer_rsrc_t ws_rsrc,
                                                    const uint32_t (&woff)[C::GPW_W],
                                                    const uint32_t (&wsoff)[C::SPW_W > 0 ? C::SPW_W : 1]) {
  const bool live = kt < nk;
#pragma unroll
  for (int q = 0; q < C::GPW_W; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, (lds_ptr_t)(wb + (wave * C::GPW_W + q) * 1024), 16,
                                             live ? woff[q] : kOob, static_cast<uint32_t>(kt) * C::W_BYTES, 0, 0);
#pragma unroll
  for (int q = 0; q < C::SPW_W; ++q) {
    const int g = wave + q * C::WAVES;
    const bool real = g < C::S_W_G;
    char* const dst = real ? wb + C::W_REGION + g * 256 : sink;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ws_rsrc, (lds_ptr_t)dst, 4, live && real ? wsoff[q] : kOob,
                                             static_cast<uint32_t>(kt) * 4, 0, 0);
  }
}

struct Params {
  const uint8_t* a;          // GEMM1: x codes [T, H]; GEMM2: h codes [cap, I]
  const void* a_scale;       // fp32 [rows, K/128] or E8M0 [rows, K/32]
  const uint8_t* w;          // FP8: E4M3 [E*N_w, K]; MX: packed E2M1 [E*N_w, K/2]
  const void* w_scale;       // FP8: fp32 [E*N_w/128, K/128]; MX: E8M0 [E*N_w, K/32]
  const int32_t* sorted_ids;
  const int32_t* tile_expert;
  const int32_t* num_tiles;
  void* out;                 // GEMM1: h codes [cap, I]; GEMM2: y bf16 [A, H]
  void* out_scale;           // GEMM1: fp32 [cap, I/128] or E8M0 [cap, I/32]
  float* h32;                // GEMM1, optional: the fp32 h before its requantisation [cap, I]
  int64_t A;
  uint32_t a_rows;           // rows of the token operand (T for GEMM1, cap for GEMM2)
  int E, H, I, k;
  int n_begin, n_end;        // the launch covers output columns [n_begin, n_end) (multiples of 128)
};

template <int BM, int BN, int WM, int WN, bool GEMM1, int MODE, int NST, int OCC, int KSUB>
__global__ __launch_bounds__(64 * WM * WN, OCC) void gemm_scaled_kernel(Params p) {
  using C = Cfg<BM, BN, WM, WN, GEMM1, MODE, NST, KSUB>;
  constexpr int WB = C::W_BYTES;
  // one LDS array per stage, so that the compiler can tell the stages being
  // filled by direct-to-LDS loads from the one being read
  constexpr bool SPLIT = C::SPLIT;
  __shared__ __attribute__((aligned(1024))) char stage0[SPLIT ? 16 : C::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[SPLIT ? 16 : C::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage2[NST == 4 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(1024))) char stage3[NST == 4 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(1024))) char sink[NST > 2 ? 1024 : 16];   // target of the padding loads
  // split stages: two token buffers (rows + scale words), three weight buffers
  __shared__ __attribute__((aligned(1024))) char tbuf0[SPLIT ? C::T_BUF : 16];
  __shared__ __attribute__((aligned(1024))) char tbuf1[SPLIT ? C::T_BUF : 16];
  __shared__ __attribute__((aligned(1024))) char wbuf0[SPLIT ? C::W_BUF : 16];
  __shared__ __attribute__((aligned(1024))) char wbuf1[SPLIT ? C::W_BUF : 16];
  __shared__ __attribute__((aligned(1024))) char wbuf2[SPLIT ? C::W_BUF : 16];
  __shared__ float red[WN][BM];   // per-row partial amax of each n-wave (FP8 requantisation)

  // the wave index is uniform across the wave: keep it in a scalar register so
  // that the LDS destinations and descriptors of the loads are scalar too
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int N = GEMM1 ? p.I : p.H;
  const int K = GEMM1 ? p.H : p.I;
  const int ntn = (p.n_end - p.n_begin + BN - 1) / BN;
  const int num_tiles = *p.num_tiles;
  const int total = num_tiles * ntn;
  const int nk128 = K / 128;                         // 128-K substeps
  const int nk = (nk128 + KSUB - 1) / KSUB;          // stages
  const int wrows = GEMM1 ? 2 * p.I : p.H;           // weight rows of one expert
  const int wrow_bytes = MODE == kMx ? K / 2 : K;
  const int srow_bytes = MODE == kMx ? K / 32 : (K / 128) * 4;   // scale bytes per token row

  // XCD-aware slice of the flat task list
  const int G = gridDim.x;
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const int per_xcd = (G + kXcds - 1 - xcd) / kXcds;
  const int64_t t0 = static_cast<int64_t>(total) * (xcd * (G / kXcds) + (xcd < G % kXcds ? xcd : G % kXcds)) / G;
  const int64_t t1 = static_cast<int64_t>(total) *
                     ((xcd + 1) * (G / kXcds) + (xcd + 1 < G % kXcds ? xcd + 1 : G % kXcds)) / G;

  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(p.a, p.a_rows * static_cast<uint32_t>(K));
  const __amdgpu_buffer_rsrc_t as_rsrc = make_rsrc(p.a_scale, p.a_rows * static_cast<uint32_t>(srow_bytes));

  // the m-tiles of one expert walk the n-tiles side by side when one
  // m-tile's walk reads more weight bytes than an XCD's 4 MB L2 holds and
  // a task stages at least as many weight rows as token rows (FP8 GEMM1:
  // 2463 -> 2265 us on the 64-expert H 7168 shape; its GEMM2, 256 token
  // rows against 128 weight rows, got 6% slower: there the m-tile walk,
  // whose 32 concurrent tasks on an XCD share one token tile, wins)
  const bool grouped = C::B_ROWS >= BM && static_cast<int64_t>(ntn) * C::B_ROWS * wrow_bytes > (int64_t{4} << 20);
  int probe = grouped && t0 + local < t1 ? grouped_probe(t0 + local, ntn, num_tiles, p.tile_expert, lane) : 0;
  for (int64_t task = t0 + local; task < t1; task += per_xcd) {
    int nt, mt, e;
    if (grouped) {
      grouped_task<kGroup>(task, ntn, num_tiles, p.tile_expert, lane, probe, nt, mt, e);
      if (task + per_xcd < t1) probe = grouped_probe(task + per_xcd, ntn, num_tiles, p.tile_expert, lane);
    } else {
      mt = static_cast<int>(task / ntn);
      nt = static_cast<int>(task - static_cast<int64_t>(mt) * ntn);
      e = p.tile_expert[mt];
    }
    const int64_t row0 = static_cast<int64_t>(mt) * BM;
    const int n0 = p.n_begin + nt * BN;
    // GEMM2: the destination rows of this lane's stores, loaded ahead of the
    // task's operand loads so that the epilogue does not start with a round trip
    int out_sid[C::FM];
#pragma unroll
    for (int i = 0; i < C::FM; ++i) out_sid[i] = GEMM1 ? 0 : p.sorted_ids[row0 + wm * C::TM + i * 32 + (lane & 31)];
    const __amdgpu_buffer_rsrc_t w_rsrc =
        make_rsrc(p.w + static_cast<int64_t>(e) * wrows * wrow_bytes, static_cast<uint32_t>(wrows) * wrow_bytes);
    const __amdgpu_buffer_rsrc_t ws_rsrc =
        MODE == kMx ? make_rsrc(static_cast<const uint8_t*>(p.w_scale) + static_cast<int64_t>(e) * wrows * (K / 32),
                                static_cast<uint32_t>(wrows) * (K / 32))
                    : as_rsrc;

    // token row r of the tile -> source row of the token operand (-1: pad)
    auto token_row = [&](int r) -> int64_t {
      if (GEMM1) {
        const int sid = p.sorted_ids[row0 + r];
        return sid < p.A ? sid / p.k : -1;
      }
      return row0 + r;
    };
    // weight row br of the tile -> row within expert e's weights (-1: past N)
    auto weight_row = [&](int br) -> int {
      if (GEMM1) {
        const int half = br >= BN ? 1 : 0;
        const int n = n0 + br - half * BN;
        return n < N ? half * p.I + n : -1;
      }
      const int n = n0 + br;
      return n < N ? n : -1;
    };

    // data loads: group g (1 KB) fills 8 token rows (g < A_GROUPS) or 1 KB of
    // weight rows; lane l writes the 16 bytes at l * 16 of the group
    uint32_t doff[C::GPW];
    uint32_t dsub[C::GPW];   // substep of this lane's weight chunk (two-substep stages)
#pragma unroll
    for (int q = 0; q < C::GPW; ++q) {
      const int g = wave * C::GPW + q;
      doff[q] = kOob;
      dsub[q] = 0;
      if (g < C::A_GROUPS) {
        const int row = (g % C::A_GROUPS_SUB) * 8 + (lane >> 3), pc = lane & 7;
        const int64_t src = token_row(row);
        if (src >= 0) doff[q] = static_cast<uint32_t>(src * K + ((pc ^ swz128(row)) << 4));
      } else if (g < C::GROUPS) {
        const int byte = (g - C::A_GROUPS) * 1024 + lane * 16;
        const int br = byte / WB, pc = (byte % WB) / 16;
        const int lc = WB == 128 ? (pc ^ swz128(br)) : (pc ^ swz64(br));
        const int wr = weight_row(br);
        if (wr >= 0) doff[q] = static_cast<uint32_t>(wr) * wrow_bytes + (lc << 4);
        dsub[q] = static_cast<uint32_t>(lc * 16 / 64) % C::KSUB;
      }
    }
    // scale-word loads: group g (256 B) holds the k-step's scale word of 64
    // rows: token rows first, then (MX) weight rows
    uint32_t soff_[C::SPW];
#pragma unroll
    for (int q = 0; q < C::SPW; ++q) {
      const int r = ((wave + q * C::WAVES) % C::S_GROUPS_SUB) * 64 + lane;
      soff_[q] = kOob;
      if (r < BM) {
        const int64_t src = token_row(r);
        if (src >= 0) soff_[q] = static_cast<uint32_t>(src * srow_bytes);
      } else if (r >= C::S_TOK && r < C::S_ROWS) {
        const int wr = weight_row(r - C::S_TOK);
        if (wr >= 0) soff_[q] = static_cast<uint32_t>(wr) * (K / 32);
      }
    }
    // FP8: the 128x128 weight-scale block row of each half of this wave's tile
    // (clamped to the expert's last block where the wave's columns lie past N:
    // their weight rows read as zeros)
    int64_t wsb[C::HALVES];
#pragma unroll
    for (int h = 0; h < C::HALVES; ++h) {
      const int n = n0 + wn * C::TN < N ? n0 + wn * C::TN : N - 1;
      wsb[h] = (static_cast<int64_t>(e) * wrows + (GEMM1 ? h * p.I : 0) + n) / 128;
    }

    auto load = [&](char* stage, int kt) {
      issue_loads<C>(stage, sink, kt, nk, nk128, wave, a_rsrc, w_rsrc, as_rsrc, ws_rsrc, doff, soff_, dsub);
    };

    f32x16 acc[C::HALVES][C::FM][C::FN];
#pragma unroll
    for (int h = 0; h < C::HALVES; ++h)
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[h][i][j] = f32x16{};
    // FP8: the scale product acc is expressed in (see compute)
    float fprev[C::HALVES][C::FM];
#pragma unroll
    for (int h = 0; h < C::HALVES; ++h)
#pragma unroll
      for (int i = 0; i < C::FM; ++i) fprev[h][i] = 0.0f;

    // tbase: the k-step's token rows; wbase: its weight rows; sbase: the token
    // rows' scale words; wsbase: (MX) the weight rows' scale words
    auto compute = [&](const char* tbase, const char* wbase, const char* sbase, const char* wsbase, int kt) {
      const int hl = lane >> 5;   // which 32-deep half of a 64-deep MFMA step this lane holds
      if (MODE == kMx) {
#pragma unroll
        for (int sub = 0; sub < C::KSUB; ++sub) {
          if (C::KSUB > 1 && kt * C::KSUB + sub >= nk128) break;   // K ends inside the stage
          const char* abase = tbase + sub * C::A_SUB;
          const uint32_t* sc = reinterpret_cast<const uint32_t*>(sbase + sub * C::S_GROUPS_SUB * 256);
          const uint32_t* wsc = reinterpret_cast<const uint32_t*>(wsbase + sub * C::S_GROUPS_SUB * 256);
          uint32_t tsc[C::FM];
#pragma unroll
          for (int i = 0; i < C::FM; ++i) tsc[i] = sc[wm * C::TM + i * 32 + (lane & 31)];
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const int blk = 2 * s + hl;               // 32-element K block of this lane's scales
            i32x8 xf[C::FM];
            int xs[C::FM];
#pragma unroll
            for (int i = 0; i < C::FM; ++i) {
              const int r = wm * C::TM + i * 32 + (lane & 31);
              xf[i] = frag32(abase + a_off(r, s * 4 + hl), abase + a_off(r, s * 4 + 2 + hl));
              xs[i] = static_cast<int>((tsc[i] >> (8 * blk)) & 0xFF);
            }
#pragma unroll
            for (int h = 0; h < C::HALVES; ++h) {
#pragma unroll
              for (int j = 0; j < C::FN; ++j) {
                const int r = h * BN + wn * C::TN + j * 32 + (lane & 31);
                const i32x8 wf = frag16(wbase + w_off<WB>(r, sub * 4 + s * 2 + hl));
                const int ws = static_cast<int>((wsc[r] >> (8 * blk)) & 0xFF);
#pragma unroll
                for (int i = 0; i < C::FM; ++i)
                  acc[h][i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf, xf[i], acc[h][i][j], 4, 0, 0,
                                                                               ws, 0, xs[i]);
              }
            }
          }
        }
      } else {
        const uint32_t* sc = reinterpret_cast<const uint32_t*>(sbase);
        // Per-128 promotion without a second accumulator set. Each scale s
        // splits into a power of two, which the MFMA applies itself through
        // its E8M0 operand scales (token: per lane, weight block: per wave),
        // and a mantissa m (split_e8m0). acc holds the sum in units of the
        // current step's mantissa product f = m_x * m_w, so each step
        // rescales acc by f_prev / f and adds the MFMA's products; the
        // epilogue multiplies by the last f. With the exponents applied
        // exactly by the MFMA, f lies in [1, 4) for normal scales and above
        // 2^-46 for any finite ones, so its hardware reciprocal (within one
        // ulp) is finite and f_prev / f stays between 2^-46 and 2^46 (a ratio
        // of two whole scale products overflows, or divides by a denormal,
        // for blocks of very different magnitudes); the ratio costs two
        // roundings, the rescale one. (A correctly rounded division here was
        // 4% slower on the H 7168 shape's GEMM1.) A pad row has s_x = 0: its
        // acc stays 0 and its last f is 0.
        int xb[C::FM];
        float xm[C::FM];
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
          xm[i] = split_e8m0(__uint_as_float(sc[wm * C::TM + i * 32 + (lane & 31)]), xb[i]);
        int wb[C::HALVES];
        float wmn[C::HALVES];
#pragma unroll
        for (int h = 0; h < C::HALVES; ++h)
          // a scalar load (the index is uniform and the scales are read-only
          // here): it waits on its own counter, not behind the stage loads
          wmn[h] = split_e8m0(((const_f32_ptr)p.w_scale)[__builtin_amdgcn_readfirstlane(
                                  static_cast<int>(wsb[h] * (K / 128) + kt))],
                              wb[h]);
#pragma unroll
        for (int h = 0; h < C::HALVES; ++h)
#pragma unroll
          for (int i = 0; i < C::FM; ++i) {
            const float f = xm[i] * wmn[h];
            const float ratio = f > 0.0f ? fprev[h][i] * __builtin_amdgcn_rcpf(f) : 1.0f;
            if (f > 0.0f) fprev[h][i] = f;
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
#pragma unroll
              for (int v = 0; v < 16; ++v) acc[h][i][j][v] *= ratio;
          }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          i32x8 xf[C::FM];
#pragma unroll
          for (int i = 0; i < C::FM; ++i) {
            const int r = wm * C::TM + i * 32 + (lane & 31);
            xf[i] = frag32(tbase + a_off(r, s * 4 + hl), tbase + a_off(r, s * 4 + 2 + hl));
          }
#pragma unroll
          for (int h = 0; h < C::HALVES; ++h) {
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
              const int r = h * BN + wn * C::TN + j * 32 + (lane & 31);
              const i32x8 wf = frag32(wbase + w_off<WB>(r, s * 4 + hl), wbase + w_off<WB>(r, s * 4 + 2 + hl));
#pragma unroll
              for (int i = 0; i < C::FM; ++i)
                acc[h][i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf, xf[i], acc[h][i][j], 0, 0, 0,
                                                                             wb[h], 0, xb[i]);
            }
          }
        }
      }
    };

    if constexpr (SPLIT) {
      // Split stages (as in the BF16 kernels): k-step s reads its token rows
      // and their scale words from token buffer s % 2 and its weight rows
      // (and MX weight scale words) from weight buffer s % 3. Issue order per
      // step: tokens of s + 1, then weights of s + 2; so when step s starts,
      // everything but the newest GPW_W + SPW_W loads (the weights of s + 1)
      // has landed. The barrier
      // after that wait also means every wave has finished step s - 1, whose
      // buffers step s refills. Six steps repeat the buffer pattern; k-steps
      // past the end are loaded as zeros but not computed.
      uint32_t toff[C::GPW_T], woff[C::GPW_W], tsoff[C::SPW_T], wsoff[C::SPW_W > 0 ? C::SPW_W : 1];
#pragma unroll
      for (int q = 0; q < C::GPW_T; ++q) {
        const int row = (wave * C::GPW_T + q) * 8 + (lane >> 3), pc = lane & 7;
        const int64_t src = token_row(row);
        toff[q] = src >= 0 ? static_cast<uint32_t>(src * K + ((pc ^ swz128(row)) << 4)) : kOob;
      }
#pragma unroll
      for (int q = 0; q < C::GPW_W; ++q) {
        const int byte = (wave * C::GPW_W + q) * 1024 + lane * 16;
        const int br = byte / WB, pc = (byte % WB) / 16;
        const int lc = WB == 128 ? (pc ^ swz128(br)) : (pc ^ swz64(br));
        const int wr = weight_row(br);
        woff[q] = wr >= 0 ? static_cast<uint32_t>(wr) * wrow_bytes + (lc << 4) : kOob;
      }
#pragma unroll
      for (int q = 0; q < C::SPW_T; ++q) {
        const int r = (wave + q * C::WAVES) * 64 + lane;
        const int64_t src = r < BM ? token_row(r) : -1;
        tsoff[q] = src >= 0 ? static_cast<uint32_t>(src * srow_bytes) : kOob;
      }
#pragma unroll
      for (int q = 0; q < (C::SPW_W > 0 ? C::SPW_W : 1); ++q) {
        const int r = (wave + q * C::WAVES) * 64 + lane;
        const int wr = C::SPW_W > 0 && r < C::B_ROWS ? weight_row(r) : -1;
        wsoff[q] = wr >= 0 ? static_cast<uint32_t>(wr) * (K / 32) : kOob;
      }
      auto load_t = [&](char* tb, int kt) {
        issue_split_tokens<C>(tb, sink, kt, nk, wave, a_rsrc, as_rsrc, toff, tsoff);
      };
      auto load_w = [&](char* wb, int kt) {
        issue_split_weights<C>(wb, sink, kt, nk, wave, w_rsrc, ws_rsrc, woff, wsoff);
      };
      auto step = [&](char* tb, char* wb, char* tb_next, char* wb_next2, int kt) {
        wait_vmcnt<C::GPW_W + C::SPW_W>();
        barrier_no_fence();
        load_t(tb_next, kt + 1);
        load_w(wb_next2, kt + 2);
        __builtin_amdgcn_sched_barrier(0);
        compute(tb, wb, tb + C::A_REGION, wb + C::W_REGION, kt);
      };
      load_t(tbuf0, 0);
      load_w(wbuf0, 0);
      load_w(wbuf1, 1);
      for (int kt = 0;; kt += 6) {
        step(tbuf0, wbuf0, tbuf1, wbuf2, kt);
        if (kt + 1 >= nk) break;
        step(tbuf1, wbuf1, tbuf0, wbuf0, kt + 1);
        if (kt + 2 >= nk) break;
        step(tbuf0, wbuf2, tbuf1, wbuf1, kt + 2);
        if (kt + 3 >= nk) break;
        step(tbuf1, wbuf0, tbuf0, wbuf2, kt + 3);
        if (kt + 4 >= nk) break;
        step(tbuf0, wbuf1, tbuf1, wbuf0, kt + 4);
        if (kt + 5 >= nk) break;
        step(tbuf1, wbuf2, tbuf0, wbuf1, kt + 5);
        if (kt + 6 >= nk) break;
      }
      // the loads issued past the end have landed and every wave is done
      // with LDS before the epilogue and the next task's loads
      wait_vmcnt<0>();
      barrier_no_fence();
    } else if constexpr (NST == 2) {
      // k-step s+1 streams into one stage while the MFMAs consume k-step s
      load(stage0, 0);
      __syncthreads();
      for (int kt = 0; kt < nk; kt += 2) {
        load(stage1, kt + 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(stage0, stage0 + C::A_REGION, stage0 + C::A_REGION + C::W_REGION,
                stage0 + C::A_REGION + C::W_REGION + C::S_TOK * 4, kt);
        __syncthreads();
        if (kt + 1 >= nk) break;
        load(stage0, kt + 2);
        __builtin_amdgcn_sched_barrier(0);
        compute(stage1, stage1 + C::A_REGION, stage1 + C::A_REGION + C::W_REGION,
                stage1 + C::A_REGION + C::W_REGION + C::S_TOK * 4, kt + 1);
        __syncthreads();
      }
    } else {
      static_assert(NST == 4, "four whole stages");
      // four stages (tiles this small are bound by the weight stream, which
      // wants more bytes in flight): k-step s is read from one stage while
      // k-steps s+1 .. s+3 stream into the others. Each step waits for its
      // own stage (the two younger k-steps stay in flight), meets the other
      // waves, and refills the stage read in the step before with k-step s+3.
      load(stage0, 0);
      load(stage1, 1);
      load(stage2, 2);
      for (int kt = 0; kt < nk; kt += 4) {
        wait_vmcnt<2 * (C::GPW + C::SPW)>();
        barrier_no_fence();
        load(stage3, kt + 3);
        __builtin_amdgcn_sched_barrier(0);
        compute(stage0, stage0 + C::A_REGION, stage0 + C::A_REGION + C::W_REGION,
                stage0 + C::A_REGION + C::W_REGION + C::S_TOK * 4, kt);
        if (kt + 1 >= nk) break;
        wait_vmcnt<2 * (C::GPW + C::SPW)>();
        barrier_no_fence();
        load(stage0, kt + 4);
        __builtin_amdgcn_sched_barrier(0);
        compute(stage1, stage1 + C::A_REGION, stage1 + C::A_REGION + C::W_REGION,
                stage1 + C::A_REGION + C::W_REGION + C::S_TOK * 4, kt + 1);
        if (kt + 2 >= nk) break;
        wait_vmcnt<2 * (C::GPW + C::SPW)>();
        barrier_no_fence();
        load(stage1, kt + 5);
        __builtin_amdgcn_sched_barrier(0);
        compute(stage2, stage2 + C::A_REGION, stage2 + C::A_REGION + C::W_REGION,
                stage2 + C::A_REGION + C::W_REGION + C::S_TOK * 4, kt + 2);
        if (kt + 3 >= nk) break;
        wait_vmcnt<2 * (C::GPW + C::SPW)>();
        barrier_no_fence();
        load(stage2, kt + 6);
        __builtin_amdgcn_sched_barrier(0);
        compute(stage3, stage3 + C::A_REGION, stage3 + C::A_REGION + C::W_REGION,
                stage3 + C::A_REGION + C::W_REGION + C::S_TOK * 4, kt + 3);
      }
      // drain the loads issued past the end (zeros) and meet, before the
      // epilogue and the next task's loads
      wait_vmcnt<0>();
      barrier_no_fence();
    }

    // ------------------------------------------------------------ epilogue
    // (FP8: acc is in units of the last scale product, applied where it is read)
    if (GEMM1) {
      // h = silu(g) * u for every accumulator element, then requantise along I
      // (h overwrites the gate accumulators in place)
      f32x16 (&hv)[C::FM][C::FN] = acc[0];
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float g = acc[0][i][j][v] * (MODE == kFp8Block ? fprev[0][i] : 1.0f);
            const float u = acc[C::HALVES - 1][i][j][v] * (MODE == kFp8Block ? fprev[C::HALVES - 1][i] : 1.0f);
            hv[i][j][v] = g / (1.0f + expf(-g)) * u;
          }
      if (p.h32 != nullptr) {
        // the values the requantisation below reads, for checking it bit for bit
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int n = n0 + wn * C::TN + j * 32 + g * 8 + (lane >> 5) * 4;
              if (n < N)
                *reinterpret_cast<f32x4*>(p.h32 + (row0 + wm * C::TM + i * 32 + (lane & 31)) * N + n) =
                    f32x4{hv[i][j][4 * g], hv[i][j][4 * g + 1], hv[i][j][4 * g + 2], hv[i][j][4 * g + 3]};
            }
      }
      uint8_t* hq = static_cast<uint8_t*>(p.out);
      if (MODE == kFp8Block) {
        // one 1x128 block per token row: this workgroup's BN = 128 columns
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
          float am = 0.0f;
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) am = __builtin_fmaxf(am, __builtin_fabsf(hv[i][j][v]));
          am = __builtin_fmaxf(am, __shfl_xor(am, 32));
          if (lane < 32) red[wn][wm * C::TM + i * 32 + lane] = am;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
          const int m = wm * C::TM + i * 32 + (lane & 31);
          float am = 0.0f;
#pragma unroll
          for (int w = 0; w < WN; ++w) am = __builtin_fmaxf(am, red[w][m]);
          const float s = am > 0.0f ? __fdiv_rn(am, 448.0f) : 1.0f;
          const int64_t row = row0 + m;
#pragma unroll
          for (int j = 0; j < C::FN; ++j) {
            uint32_t q[4];
#pragma unroll
            for (int g = 0; g < 4; ++g)
              q[g] = pack_e4m3x4(__fdiv_rn(hv[i][j][4 * g], s), __fdiv_rn(hv[i][j][4 * g + 1], s),
                                 __fdiv_rn(hv[i][j][4 * g + 2], s), __fdiv_rn(hv[i][j][4 * g + 3], s));
            store_codes_x32(hq + row * N + n0 + wn * C::TN + j * 32, q, lane);
          }
          if (wn == 0 && lane < 32) static_cast<float*>(p.out_scale)[row * (N / 128) + n0 / 128] = s;
        }
        __syncthreads();   // red is reused by the next task
      } else {
        // one 1x32 block per (token row, 32-column fragment): the lane and its
        // partner lane^32 hold the 32 columns between them
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
          const int m = wm * C::TM + i * 32 + (lane & 31);
          const int64_t row = row0 + m;
#pragma unroll
          for (int j = 0; j < C::FN; ++j) {
            float am = 0.0f;
#pragma unroll
            for (int v = 0; v < 16; ++v) am = __builtin_fmaxf(am, __builtin_fabsf(hv[i][j][v]));
            am = __builtin_fmaxf(am, __shfl_xor(am, 32));
            const int x = mx_scale_exponent(am, 8);
            const float inv = mx_inv_scale(x);
            const int nb = n0 + wn * C::TN + j * 32;
            if (nb >= N) continue;   // a ragged last column tile: whole 32-column fragments past I
            uint32_t q[4];
#pragma unroll
            for (int g = 0; g < 4; ++g)
              q[g] = pack_e4m3x4(hv[i][j][4 * g] * inv, hv[i][j][4 * g + 1] * inv, hv[i][j][4 * g + 2] * inv,
                                 hv[i][j][4 * g + 3] * inv);
            store_codes_x32(hq + row * N + nb, q, lane);
            if (lane < 32) static_cast<uint8_t*>(p.out_scale)[row * (N / 32) + nb / 32] = static_cast<uint8_t>(x + 127);
          }
        }
      }
    } else {
      uint16_t* y = static_cast<uint16_t*>(p.out);
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int m = wm * C::TM + i * 32 + (lane & 31);
        const int sid = out_sid[i];
        const bool row_ok = sid < p.A;
        const float fs = MODE == kFp8Block ? fprev[0][i] : 1.0f;
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          // lanes r and r + 32 hold columns 8g .. 8g + 3 and 8g + 4 .. 8g + 7 of
          // the same row: one lane swap per word (v_permlane32_swap: the upper
          // lanes' first operand for the lower lanes' second) leaves lane r
          // groups 0, 1 and lane r + 32 groups 2, 3 whole, stored 16 bytes at
          // a time (every lane takes part in the swap; pad rows store nothing)
          uint32_t u[4][2], from_lo[2][2], from_hi[2][2];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            u[g][0] = pack_bf16x2(acc[0][i][j][4 * g] * fs, acc[0][i][j][4 * g + 1] * fs);
            u[g][1] = pack_bf16x2(acc[0][i][j][4 * g + 2] * fs, acc[0][i][j][4 * g + 3] * fs);
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
            if (row_ok && n < N) *reinterpret_cast<uint4*>(y + static_cast<int64_t>(sid) * N + n) = st;   // N % 128 == 0
          }
        }
      }
    }
  }
}

// OCC workgroups per CU: the 32-row tiles of small token counts are bound by
// the weight stream, and a second workgroup per CU fills the gaps one
// workgroup's pipeline leaves between tasks (LDS and registers must fit OCC)
template <int BM, int BN, int WM, int WN, bool GEMM1, int MODE, int NST = 2, int OCC = 1, int KSUB = 1>
hipError_t launch(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s, int n_begin = 0, int n_end = -1) {
  using C = Cfg<BM, BN, WM, WN, GEMM1, MODE, NST, KSUB>;
  static_assert(OCC * (C::LDS_STAGES + WN * BM * 4) <= 160 * 1024, "OCC workgroups fit in LDS");
  Params p;
  p.a = static_cast<const uint8_t*>(g.a);
  p.a_scale = g.a_scale;
  p.w = static_cast<const uint8_t*>(g.w);
  p.w_scale = g.w_scale;
  p.sorted_ids = g.sorted_ids;
  p.tile_expert = g.tile_expert;
  p.num_tiles = g.num_tiles;
  p.out = g.out;
  p.out_scale = g.out_scale;
  p.h32 = GEMM1 ? static_cast<float*>(g.h32) : nullptr;
  p.A = g.T * g.k;
  p.a_rows = static_cast<uint32_t>(GEMM1 ? g.T : g.cap);
  p.E = g.E;
  p.H = g.H;
  p.I = g.I;
  p.k = g.k;
  const int N = GEMM1 ? g.I : g.H;
  p.n_begin = n_begin;
  p.n_end = n_end < 0 ? N : n_end;
  const int64_t max_tasks = (g.cap / BM) * ((p.n_end - n_begin + BN - 1) / BN);
  int64_t grid = static_cast<int64_t>(dev.num_cus) * OCC;
  if (grid > max_tasks) grid = max_tasks;
  if (grid < 1) grid = 1;
  gemm_scaled_kernel<BM, BN, WM, WN, GEMM1, MODE, NST, OCC, KSUB><<<static_cast<unsigned>(grid), C::THREADS, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_gemm1_mx_tiles(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
  switch (g.block_m) {
    case 256: return launch<256, 128, 4, 2, true, kMx, 3>(g, dev, s);
    case 128: {
      // I % 256 == 128 (the MXFP4 shape's 640): the last 256-column tile
      // would be half empty, a fifth of the MFMA work on zero weight rows;
      // 128-column tiles take the last 128 columns in a second launch
      // (same-process medians: T = 16384 827 -> 777 us, T = 8192 554 -> 524)
      if (g.I % 256 == 0 || g.I < 256) return launch<128, 256, 4, 2, true, kMx, 3>(g, dev, s);
      const hipError_t e = launch<128, 256, 4, 2, true, kMx, 3>(g, dev, s, 0, g.I - 128);
      if (e != hipSuccess) return e;
      return launch<128, 128, 4, 2, true, kMx, 3>(g, dev, s, g.I - 128);
    }
    case 64: return launch<64, 256, 1, 8, true, kMx, 3>(g, dev, s);
    case 32: return launch<32, 256, 1, 8, true, kMx, 2, 1, 2>(g, dev, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm2_mx_tiles(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
  switch (g.block_m) {
    case 256: return launch<256, 256, 4, 2, false, kMx, 3>(g, dev, s);
    case 128: return launch<128, 512, 2, 4, false, kMx, 3>(g, dev, s);
    case 64: return launch<64, 512, 1, 8, false, kMx, 3>(g, dev, s);
    case 32: return launch<32, 512, 1, 8, false, kMx, 2, 2>(g, dev, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm1_fp8_tiles(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
  switch (g.block_m) {
    case 256: return launch<256, 128, 4, 2, true, kFp8Block>(g, dev, s);
    case 128: return launch<128, 128, 2, 4, true, kFp8Block, 3>(g, dev, s);
    case 64: return launch<64, 128, 2, 4, true, kFp8Block, 3>(g, dev, s);
    case 32: return launch<32, 128, 1, 4, true, kFp8Block, 4>(g, dev, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm2_fp8_tiles(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
  switch (g.block_m) {
    case 256: return launch<256, 128, 4, 2, false, kFp8Block, 3>(g, dev, s);
    case 128: return launch<128, 256, 2, 4, false, kFp8Block, 3>(g, dev, s);
    case 64: return launch<64, 256, 2, 4, false, kFp8Block, 3>(g, dev, s);
    case 32: return launch<32, 256, 1, 4, false, kFp8Block, 4>(g, dev, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool gemm_fp8_supports(int block_m) { return block_m == 32 || block_m == 64 || block_m == 128 || block_m == 256; }
bool gemm_mx_supports(int block_m) { return block_m == 32 || block_m == 64 || block_m == 128 || block_m == 256; }

hipError_t launch_gemm1_fp8(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
  return launch_gemm1_fp8_tiles(g, dev, s);
}
hipError_t launch_gemm2_fp8(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
  return launch_gemm2_fp8_tiles(g, dev, s);
}
hipError_t launch_gemm1_mx(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
  return launch_gemm1_mx_tiles(g, dev, s);
}
hipError_t launch_gemm2_mx(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
  return launch_gemm2_mx_tiles(g, dev, s);
}

}  // namespace moe
