// BF16 grouped GEMMs over the expert-sorted rows (FlashInfer PR #5129,
// Description: GEMM1 writes padded expert-sorted rows, GEMM2 reads them
// contiguously and scatters back to assignment order; TileScale PR #70,
// Design: GEMM1 + SwiGLU in one kernel, fp32 accumulation).
//
// Design for gfx950:
//   * persistent workgroups walk one flat task list: task = (m-tile of the
//     sorted rows, n-tile of the output columns); the m-tile count is read
//     from device memory, so the host never waits for the router;
//   * MFMA v_mfma_f32_32x32x16_bf16 with the weight rows as the MFMA "A"
//     operand and the token rows as "B" (output transposed in registers:
//     each lane ends up with four consecutive output columns of one token,
//     which become one 8-byte store);
//   * 4 waves per workgroup, LDS double buffered (global -> registers for
//     k-step s+1 while the MFMAs consume k-step s); 128-byte LDS rows with
//     the 16-byte chunk index XOR-swizzled by (row & 7) so that the MFMA
//     fragment reads of 8 consecutive rows hit distinct banks;
//   * GEMM1 keeps the gate rows n and up rows I + n of the same output
//     column in one workgroup, so SwiGLU runs in registers in the epilogue.
#include "moe_common.cuh"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kBK = 64;        // bf16 elements per k-step (128 bytes per LDS row)
constexpr int kThreads = 256;

template <int BM, int BN, int WM, int WN, bool GEMM1>
struct Cfg {
  static constexpr int B_ROWS = GEMM1 ? 2 * BN : BN;  // weight rows staged per k-step
  static constexpr int TM = BM / WM;                  // token rows per wave
  static constexpr int TN = BN / WN;                  // output columns per wave
  static constexpr int FM = TM / 32;
  static constexpr int FN = TN / 32;
  static constexpr int HALVES = GEMM1 ? 2 : 1;
  static constexpr int A_LOADS = BM * 8 / kThreads;   // 16-byte chunks per thread
  static constexpr int B_LOADS = B_ROWS * 8 / kThreads;
  static constexpr int STAGE = (BM + B_ROWS) * 128;   // bytes per LDS stage
  static_assert(WM * WN == 4, "4 waves");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile is a multiple of 32");
  static_assert(BM * 8 % kThreads == 0 && B_ROWS * 8 % kThreads == 0, "whole loads");
};

__device__ __forceinline__ uint32_t lds_off(int row, int chunk) {
  return static_cast<uint32_t>(row * 128 + ((chunk ^ (row & 7)) << 4));
}

__device__ __forceinline__ bf16x8 lds_frag(const char* base, int row, int chunk) {
  const uint4 v = *reinterpret_cast<const uint4*>(base + lds_off(row, chunk));
  return __builtin_bit_cast(bf16x8, v);
}

struct Params {
  const uint16_t* a;       // GEMM1: x [T, H]; GEMM2: h [cap, I]
  const uint16_t* w;       // GEMM1: W1 [E, 2I, H]; GEMM2: W2 [E, H, I]
  const int32_t* sorted_ids;
  const int32_t* tile_expert;
  const int32_t* num_tiles;
  uint16_t* out;           // GEMM1: h [cap, I]; GEMM2: y [A, H]
  int64_t A;
  int H, I, k;
};

template <int BM, int BN, int WM, int WN, bool GEMM1>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(Params p) {
  using C = Cfg<BM, BN, WM, WN, GEMM1>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int N = GEMM1 ? p.I : p.H;      // output columns
  const int K = GEMM1 ? p.H : p.I;      // reduction length
  const int ntn = (N + BN - 1) / BN;
  const int total = *p.num_tiles * ntn;
  const int nk = (K + kBK - 1) / kBK;
  const int chunk = tid & 7;
  const int lrow = tid >> 3;            // 0..31: row within a 32-row load slab

  for (int task = blockIdx.x; task < total; task += gridDim.x) {
    const int mt = task / ntn, nt = task - mt * ntn;
    const int e = p.tile_expert[mt];
    const int64_t row0 = static_cast<int64_t>(mt) * BM;
    const int n0 = nt * BN;

    // sources of the rows this thread stages
    const uint16_t* a_src[C::A_LOADS];
    bool a_ok[C::A_LOADS];
#pragma unroll
    for (int q = 0; q < C::A_LOADS; ++q) {
      const int r = lrow + 32 * q;
      if (GEMM1) {
        const int sid = p.sorted_ids[row0 + r];
        a_ok[q] = sid < p.A;
        a_src[q] = p.a + static_cast<int64_t>(a_ok[q] ? sid / p.k : 0) * K;
      } else {
        a_ok[q] = true;
        a_src[q] = p.a + (row0 + r) * K;
      }
    }
    const uint16_t* b_src[C::B_LOADS];
    bool b_ok[C::B_LOADS];
#pragma unroll
    for (int q = 0; q < C::B_LOADS; ++q) {
      const int br = lrow + 32 * q;
      int64_t wrow;
      int n;
      if (GEMM1) {
        const int half = br >= BN ? 1 : 0;
        n = n0 + br - half * BN;
        wrow = static_cast<int64_t>(e) * 2 * p.I + half * p.I + n;
      } else {
        n = n0 + br;
        wrow = static_cast<int64_t>(e) * p.H + n;
      }
      b_ok[q] = n < N;
      b_src[q] = p.w + (b_ok[q] ? wrow : 0) * K;
    }

    uint4 ra[C::A_LOADS], rb[C::B_LOADS];
    auto load = [&](int kt) {
      const int col = kt * kBK + chunk * 8;
      const bool kin = col < K;
#pragma unroll
      for (int q = 0; q < C::A_LOADS; ++q)
        ra[q] = (a_ok[q] && kin) ? *reinterpret_cast<const uint4*>(a_src[q] + col) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < C::B_LOADS; ++q)
        rb[q] = (b_ok[q] && kin) ? *reinterpret_cast<const uint4*>(b_src[q] + col) : make_uint4(0, 0, 0, 0);
    };
    auto store = [&](int stage) {
      char* base = smem + stage * C::STAGE;
#pragma unroll
      for (int q = 0; q < C::A_LOADS; ++q)
        *reinterpret_cast<uint4*>(base + lds_off(lrow + 32 * q, chunk)) = ra[q];
#pragma unroll
      for (int q = 0; q < C::B_LOADS; ++q)
        *reinterpret_cast<uint4*>(base + lds_off(BM + lrow + 32 * q, chunk)) = rb[q];
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
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        const int ch = kk * 2 + (lane >> 5);
        bf16x8 xf[C::FM];
#pragma unroll
        for (int i = 0; i < C::FM; ++i) xf[i] = lds_frag(base, wm * C::TM + i * 32 + (lane & 31), ch);
#pragma unroll
        for (int h = 0; h < C::HALVES; ++h) {
#pragma unroll
          for (int j = 0; j < C::FN; ++j) {
            const bf16x8 wf = lds_frag(base, BM + h * BN + wn * C::TN + j * 32 + (lane & 31), ch);
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
              acc[h][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, xf[i], acc[h][i][j], 0, 0, 0);
          }
        }
      }
      if (kt + 1 < nk) store((kt + 1) & 1);
      __syncthreads();
    }

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
            if (GEMM1) {
              const float uv = acc[C::HALVES - 1][i][j][g * 4 + r];
              o[r] = gv / (1.0f + expf(-gv)) * uv;
            } else {
              o[r] = gv;
            }
          }
          if (row_ok && n < N) {
            uint2 st;
            st.x = pack_bf16x2(o[0], o[1]);
            st.y = pack_bf16x2(o[2], o[3]);
            *reinterpret_cast<uint2*>(p.out + dst_row * N + n) = st;
          }
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, bool GEMM1>
hipError_t launch(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
  Params p;
  p.a = static_cast<const uint16_t*>(g.a);
  p.w = static_cast<const uint16_t*>(g.w);
  p.sorted_ids = g.sorted_ids;
  p.tile_expert = g.tile_expert;
  p.num_tiles = g.num_tiles;
  p.out = static_cast<uint16_t*>(g.out);
  p.A = g.T * g.k;
  p.H = g.H;
  p.I = g.I;
  p.k = g.k;
  const int N = GEMM1 ? g.I : g.H;
  const int64_t max_tasks = (g.cap / BM) * ((N + BN - 1) / BN);
  int64_t grid = dev.num_cus;
  if (grid > max_tasks) grid = max_tasks;
  if (grid < 1) grid = 1;
  gemm_bf16_kernel<BM, BN, WM, WN, GEMM1><<<static_cast<unsigned>(grid), kThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

bool gemm_bf16_supports(int block_m) { return block_m == 32 || block_m == 64 || block_m == 128; }

hipError_t launch_gemm1_bf16(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
  switch (g.block_m) {
    case 128: return launch<128, 128, 2, 2, true>(g, dev, s);
    case 64: return launch<64, 128, 2, 2, true>(g, dev, s);
    case 32: return launch<32, 128, 1, 4, true>(g, dev, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm2_bf16(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s) {
  switch (g.block_m) {
    case 128: return launch<128, 256, 2, 2, false>(g, dev, s);
    case 64: return launch<64, 256, 2, 2, false>(g, dev, s);
    case 32: return launch<32, 256, 1, 4, false>(g, dev, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
