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
//  * MXFP4W_MXFP8A (FlashInfer PR #6465, Benchmark configuration: MXFP4
//    weights with K32 scaling, FP8 activations). The weights are E2M1, the
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
// (the fp32 1x128 token scale, or four E8M0 bytes). LDS is double buffered;
// 16-byte chunks are XOR-swizzled per row so that the fragment reads of 8
// consecutive rows fall on distinct banks.
#include "moe_common.cuh"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kFp8Block = 1;
constexpr int kMx = 2;

template <int BM, int BN, int WM, int WN, bool GEMM1, int MODE>
struct Cfg {
  static constexpr int W_BYTES = MODE == kMx ? 64 : 128;   // weight row bytes per k-step
  static constexpr int B_ROWS = GEMM1 ? 2 * BN : BN;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int HALVES = GEMM1 ? 2 : 1;
  static constexpr int A_LOADS = BM * 8 / kThreads;         // 16-byte chunks per thread
  static constexpr int W_CPR = W_BYTES / 16;                // chunks per weight row
  static constexpr int W_LOADS = B_ROWS * W_CPR / kThreads;
  static constexpr int A_REGION = BM * 128;
  static constexpr int W_REGION = B_ROWS * W_BYTES;
  static constexpr int STAGE = A_REGION + W_REGION + (BM + B_ROWS) * 4;
  static_assert(WM * WN == 4, "4 waves");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile is a multiple of 32");
  static_assert(A_LOADS * kThreads == BM * 8 && W_LOADS * kThreads == B_ROWS * W_CPR, "whole loads");
  static_assert(MODE != kFp8Block || TN <= 128, "a wave's weight rows share one 128x128 scale block");
};

__device__ __forceinline__ uint32_t a_off(int row, int c) {
  return static_cast<uint32_t>(row * 128 + ((c ^ (row & 7)) << 4));
}

template <int W_BYTES>
__device__ __forceinline__ uint32_t w_off(int row, int c) {
  if (W_BYTES == 128) return static_cast<uint32_t>(row * 128 + ((c ^ (row & 7)) << 4));
  return static_cast<uint32_t>(row * 64 + ((c ^ ((row >> 2) & 3)) << 4));
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
  int64_t A;
  int H, I, k;
};

template <int BM, int BN, int WM, int WN, bool GEMM1, int MODE>
__global__ __launch_bounds__(kThreads, 1) void gemm_scaled_kernel(Params p) {
  using C = Cfg<BM, BN, WM, WN, GEMM1, MODE>;
  constexpr int WB = C::W_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];
  __shared__ float red[WN][BM];   // per-row partial amax of each n-wave (FP8 requantisation)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int N = GEMM1 ? p.I : p.H;
  const int K = GEMM1 ? p.H : p.I;
  const int ntn = (N + BN - 1) / BN;
  const int total = *p.num_tiles * ntn;
  const int nk = K / 128;
  const int wrows_per_expert = GEMM1 ? 2 * p.I : p.H;
  const int a_chunk = tid & 7, a_lrow = tid >> 3;                    // 32 token rows per slab
  const int w_chunk = tid % C::W_CPR, w_lrow = tid / C::W_CPR;       // weight rows per slab
  constexpr int W_SLAB = kThreads / C::W_CPR;

  for (int task = blockIdx.x; task < total; task += gridDim.x) {
    const int mt = task / ntn, nt = task - mt * ntn;
    const int e = p.tile_expert[mt];
    const int64_t row0 = static_cast<int64_t>(mt) * BM;
    const int n0 = nt * BN;

    // token rows staged by this thread
    const uint8_t* a_src[C::A_LOADS];
    bool a_ok[C::A_LOADS];
#pragma unroll
    for (int q = 0; q < C::A_LOADS; ++q) {
      const int r = a_lrow + 32 * q;
      int64_t src_row;
      if (GEMM1) {
        const int sid = p.sorted_ids[row0 + r];
        a_ok[q] = sid < p.A;
        src_row = a_ok[q] ? sid / p.k : 0;
      } else {
        a_ok[q] = true;
        src_row = row0 + r;
      }
      a_src[q] = p.a + src_row * K;
    }
    // weight rows staged by this thread
    const uint8_t* w_src[C::W_LOADS];
    bool w_ok[C::W_LOADS];
#pragma unroll
    for (int q = 0; q < C::W_LOADS; ++q) {
      const int br = w_lrow + W_SLAB * q;
      int n, off;
      if (GEMM1) {
        const int half = br >= BN ? 1 : 0;
        n = n0 + br - half * BN;
        off = half * p.I + n;
      } else {
        n = n0 + br;
        off = n;
      }
      w_ok[q] = n < N;
      const int64_t wrow = static_cast<int64_t>(e) * wrows_per_expert + (w_ok[q] ? off : 0);
      w_src[q] = p.w + wrow * (MODE == kMx ? K / 2 : K);
    }
    // scale words: thread tid < BM stages token row tid; tid < B_ROWS stages weight row tid (MX)
    int64_t sa_row = -1;
    if (tid < BM) {
      if (GEMM1) {
        const int sid = p.sorted_ids[row0 + tid];
        sa_row = sid < p.A ? sid / p.k : -1;
      } else {
        sa_row = row0 + tid;
      }
    }
    int64_t sw_row = -1;
    if (MODE == kMx && tid < C::B_ROWS) {
      int n, off;
      if (GEMM1) {
        const int half = tid >= BN ? 1 : 0;
        n = n0 + tid - half * BN;
        off = half * p.I + n;
      } else {
        n = n0 + tid;
        off = n;
      }
      if (n < N) sw_row = static_cast<int64_t>(e) * wrows_per_expert + off;
    }
    // FP8: the 128x128 weight-scale block row of each half of this wave's tile
    int64_t wsb[C::HALVES];
#pragma unroll
    for (int h = 0; h < C::HALVES; ++h) {
      const int off = (GEMM1 ? h * p.I : 0) + n0 + wn * C::TN;
      wsb[h] = (static_cast<int64_t>(e) * wrows_per_expert + off) / 128;
    }

    uint4 ra[C::A_LOADS], rw[C::W_LOADS];
    uint32_t rsa = 0, rsw = 0;
    auto load = [&](int kt) {
#pragma unroll
      for (int q = 0; q < C::A_LOADS; ++q)
        ra[q] = a_ok[q] ? *reinterpret_cast<const uint4*>(a_src[q] + kt * 128 + a_chunk * 16)
                        : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < C::W_LOADS; ++q)
        rw[q] = w_ok[q] ? *reinterpret_cast<const uint4*>(w_src[q] + kt * WB + w_chunk * 16)
                        : make_uint4(0, 0, 0, 0);
      if (MODE == kMx) {
        rsa = sa_row >= 0 ? reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(p.a_scale) +
                                                              sa_row * (K / 32))[kt]
                          : 0x7F7F7F7Fu;
        rsw = sw_row >= 0 ? reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(p.w_scale) +
                                                              sw_row * (K / 32))[kt]
                          : 0x7F7F7F7Fu;
      } else {
        rsa = sa_row >= 0 ? __float_as_uint(static_cast<const float*>(p.a_scale)[sa_row * (K / 128) + kt]) : 0u;
      }
    };
    auto store = [&](int stage) {
      char* base = smem + stage * C::STAGE;
#pragma unroll
      for (int q = 0; q < C::A_LOADS; ++q) *reinterpret_cast<uint4*>(base + a_off(a_lrow + 32 * q, a_chunk)) = ra[q];
#pragma unroll
      for (int q = 0; q < C::W_LOADS; ++q)
        *reinterpret_cast<uint4*>(base + C::A_REGION + w_off<WB>(w_lrow + W_SLAB * q, w_chunk)) = rw[q];
      uint32_t* sc = reinterpret_cast<uint32_t*>(base + C::A_REGION + C::W_REGION);
      if (tid < BM) sc[tid] = rsa;
      if (MODE == kMx && tid < C::B_ROWS) sc[BM + tid] = rsw;
    };

    f32x16 acc[C::HALVES][C::FM][C::FN];
#pragma unroll
    for (int h = 0; h < C::HALVES; ++h)
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[h][i][j] = f32x16{};

    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) load(kt + 1);
      const char* base = smem + (kt & 1) * C::STAGE;
      const uint32_t* sc = reinterpret_cast<const uint32_t*>(base + C::A_REGION + C::W_REGION);
      const int hl = lane >> 5;   // which 32-deep half of a 64-deep MFMA step this lane holds

      // per-lane token scale (FP8: fp32 value; MX: 4 E8M0 bytes)
      uint32_t tsc[C::FM];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) tsc[i] = sc[wm * C::TM + i * 32 + (lane & 31)];
      float wsc[C::HALVES];
      if (MODE == kFp8Block) {
#pragma unroll
        for (int h = 0; h < C::HALVES; ++h)
          wsc[h] = static_cast<const float*>(p.w_scale)[wsb[h] * (K / 128) + kt];
      }

      if (MODE == kMx) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int blk = 2 * s + hl;                 // 32-element K block of this lane
          i32x8 xf[C::FM];
          int xs[C::FM];
#pragma unroll
          for (int i = 0; i < C::FM; ++i) {
            const int r = wm * C::TM + i * 32 + (lane & 31);
            xf[i] = frag32(base + a_off(r, s * 4 + hl), base + a_off(r, s * 4 + 2 + hl));
            xs[i] = static_cast<int>((tsc[i] >> (8 * blk)) & 0xFF);
          }
#pragma unroll
          for (int h = 0; h < C::HALVES; ++h) {
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
              const int r = h * BN + wn * C::TN + j * 32 + (lane & 31);
              const i32x8 wf = frag16(base + C::A_REGION + w_off<WB>(r, s * 2 + hl));
              const int ws = static_cast<int>((sc[BM + r] >> (8 * blk)) & 0xFF);
#pragma unroll
              for (int i = 0; i < C::FM; ++i)
                acc[h][i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf, xf[i], acc[h][i][j], 4, 0, 0, ws,
                                                                             0, xs[i]);
            }
          }
        }
      } else {
        f32x16 part[C::HALVES][C::FM][C::FN];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          i32x8 xf[C::FM];
#pragma unroll
          for (int i = 0; i < C::FM; ++i) {
            const int r = wm * C::TM + i * 32 + (lane & 31);
            xf[i] = frag32(base + a_off(r, s * 4 + hl), base + a_off(r, s * 4 + 2 + hl));
          }
#pragma unroll
          for (int h = 0; h < C::HALVES; ++h) {
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
              const int r = h * BN + wn * C::TN + j * 32 + (lane & 31);
              const i32x8 wf = frag32(base + C::A_REGION + w_off<WB>(r, s * 4 + hl),
                                      base + C::A_REGION + w_off<WB>(r, s * 4 + 2 + hl));
#pragma unroll
              for (int i = 0; i < C::FM; ++i)
                part[h][i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    wf, xf[i], s == 0 ? f32x16{} : part[h][i][j], 0, 0, 0, 127, 0, 127);
            }
          }
        }
#pragma unroll
        for (int h = 0; h < C::HALVES; ++h)
#pragma unroll
          for (int i = 0; i < C::FM; ++i) {
            const float f = __uint_as_float(tsc[i]) * wsc[h];
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
#pragma unroll
              for (int v = 0; v < 16; ++v) acc[h][i][j][v] = __builtin_fmaf(f, part[h][i][j][v], acc[h][i][j][v]);
          }
      }
      if (kt + 1 < nk) store((kt + 1) & 1);
      __syncthreads();
    }

    // ------------------------------------------------------------ epilogue
    if (GEMM1) {
      // h = silu(g) * u for every accumulator element, then requantise along I
      float hv[C::FM][C::FN][16];
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float g = acc[0][i][j][v], u = acc[C::HALVES - 1][i][j][v];
            hv[i][j][v] = g / (1.0f + expf(-g)) * u;
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
          for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int n = n0 + wn * C::TN + j * 32 + g * 8 + (lane >> 5) * 4;
              const uint32_t q = pack_e4m3x4(__fdiv_rn(hv[i][j][4 * g], s), __fdiv_rn(hv[i][j][4 * g + 1], s),
                                             __fdiv_rn(hv[i][j][4 * g + 2], s), __fdiv_rn(hv[i][j][4 * g + 3], s));
              *reinterpret_cast<uint32_t*>(hq + row * N + n) = q;
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
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int n = nb + g * 8 + (lane >> 5) * 4;
              const uint32_t q = pack_e4m3x4(hv[i][j][4 * g] * inv, hv[i][j][4 * g + 1] * inv,
                                             hv[i][j][4 * g + 2] * inv, hv[i][j][4 * g + 3] * inv);
              *reinterpret_cast<uint32_t*>(hq + row * N + n) = q;
            }
            if (lane < 32) static_cast<uint8_t*>(p.out_scale)[row * (N / 32) + nb / 32] = static_cast<uint8_t>(x + 127);
          }
        }
      }
    } else {
      uint16_t* y = static_cast<uint16_t*>(p.out);
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int m = wm * C::TM + i * 32 + (lane & 31);
        const int sid = p.sorted_ids[row0 + m];
        if (sid >= p.A) continue;
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = n0 + wn * C::TN + j * 32 + g * 8 + (lane >> 5) * 4;
            if (n < N) {
              uint2 st;
              st.x = pack_bf16x2(acc[0][i][j][4 * g], acc[0][i][j][4 * g + 1]);
              st.y = pack_bf16x2(acc[0][i][j][4 * g + 2], acc[0][i][j][4 * g + 3]);
              *reinterpret_cast<uint2*>(y + static_cast<int64_t>(sid) * N + n) = st;
            }
          }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, bool GEMM1, int MODE>
hipError_t launch(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
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
  p.A = g.T * g.k;
  p.H = g.H;
  p.I = g.I;
  p.k = g.k;
  const int N = GEMM1 ? g.I : g.H;
  const int64_t max_tasks = (g.cap / BM) * ((N + BN - 1) / BN);
  int64_t grid = dev.num_cus;
  if (grid > max_tasks) grid = max_tasks;
  if (grid < 1) grid = 1;
  gemm_scaled_kernel<BM, BN, WM, WN, GEMM1, MODE><<<static_cast<unsigned>(grid), kThreads, 0, s>>>(p);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_gemm1(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
  switch (g.block_m) {
    case 128: return launch<128, 128, 2, 2, true, MODE>(g, dev, s);
    case 64: return launch<64, 128, 2, 2, true, MODE>(g, dev, s);
    case 32: return launch<32, 128, 1, 4, true, MODE>(g, dev, s);
    default: return hipErrorInvalidValue;
  }
}

template <int MODE>
hipError_t launch_gemm2(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
  switch (g.block_m) {
    case 128: return launch<128, 256, 2, 2, false, MODE>(g, dev, s);
    case 64: return launch<64, 256, 2, 2, false, MODE>(g, dev, s);
    case 32: return launch<32, 256, 1, 4, false, MODE>(g, dev, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool gemm_fp8_supports(int block_m) { return block_m == 32 || block_m == 64 || block_m == 128; }
bool gemm_mx_supports(int block_m) { return block_m == 32 || block_m == 64 || block_m == 128; }

hipError_t launch_gemm1_fp8(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
  return launch_gemm1<kFp8Block>(g, dev, s);
}
hipError_t launch_gemm2_fp8(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
  return launch_gemm2<kFp8Block>(g, dev, s);
}
hipError_t launch_gemm1_mx(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
  return launch_gemm1<kMx>(g, dev, s);
}
hipError_t launch_gemm2_mx(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
  return launch_gemm2<kMx>(g, dev, s);
}

}  // namespace moe
