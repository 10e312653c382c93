// Host-side launchers of the gfx950 kernels. Each launcher assumes its
// arguments were validated by the C ABI front end (moe_api.cpp) and only
// enqueues work on `stream`; it returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

struct DeviceInfo {
  int num_cus;   // compute units of the current device
};

hipError_t launch_route(const float* logits, int64_t T, int E, int k, int score, int n_shared,
                        int32_t* ids, float* w, hipStream_t s);

// align_sort: chunked, deterministic counting sort (see align_sort.hip).
constexpr int kAlignChunk = 1024;          // assignments per chunk of the counting pass
size_t align_sort_ws_bytes(int64_t T, int k, int E);
// The fixed align_sort scratch (no allocation): assignments it covers, its
// size, and this device's address of it (looked up once per device).
constexpr int64_t kNoAllocMaxA = int64_t{1} << 18;
size_t align_sort_scratch_bytes();
hipError_t align_sort_scratch(void** ptr);
hipError_t launch_align_sort(const int32_t* ids, int64_t T, int k, int E, int block_m,
                             int32_t* counts, int32_t* offsets, int32_t* sorted_ids,
                             int32_t* tile_expert, int32_t* num_tiles, int64_t cap,
                             void* ws, hipStream_t s);

hipError_t launch_quantize_fp8(const uint16_t* in, int64_t rows, int64_t cols, int block_rows,
                               uint8_t* q, float* scale, hipStream_t s);
hipError_t launch_quantize_mx(const uint16_t* in, int64_t rows, int64_t cols, bool fp4,
                              uint8_t* q, uint8_t* e8m0, hipStream_t s);

hipError_t launch_combine(const uint16_t* y, const float* w, int64_t T, int k, int H,
                          uint16_t* out, const DeviceInfo& dev, hipStream_t s);

// Grouped GEMMs. `gemm1` selects GEMM1 + SwiGLU (x gathered by token) versus
// GEMM2 (h rows contiguous, output scattered to assignment order).
struct GemmArgs {
  const void* a;          // GEMM1: x [T, H]; GEMM2: h [cap, I]
  const void* a_scale;
  const void* w;          // GEMM1: W1; GEMM2: W2
  const void* w_scale;
  const int32_t* sorted_ids;
  const int32_t* tile_expert;
  const int32_t* num_tiles;
  void* out;              // GEMM1: h [cap, I]; GEMM2: y [A, H]
  void* out_scale;        // GEMM1 quantised h scales
  int64_t T;
  int H, I, E, k, block_m;
  int64_t cap;
  void* h32 = nullptr;    // GEMM1, optional: fp32 h [cap, I] before its storage rounding
  void* split_ws = nullptr;   // BF16, optional: K-split workspace (split_ws_bytes), counters zero between calls
};

// Workspace of the BF16 grouped GEMMs (gemm_bf16.hip): one int32 counter per
// K-split slot (the first 4096 bytes), the per-XCD item queues (a claim and
// a finish counter per XCD, 128 bytes apart, from kQueueOffset), then two
// fp32 partial tiles per slot, each as large as the largest tile (256 x 256),
// from kWsCounterBytes. A split round holds at most half as many tasks as an
// XCD has workgroups, so a grid of `grid` workgroups uses at most
// kSplitXcds * split_slots_per_xcd slots.
constexpr int kSplitXcds = 8;
__host__ __device__ constexpr int split_slots_per_xcd(int grid) {
  return ((grid + kSplitXcds - 1) / kSplitXcds + 1) / 2;
}
constexpr size_t kQueueOffset = 4096;          // split counters of grids up to 2048 workgroups before it
constexpr int kQueueStride = 32;               // int32 per XCD: claim at 0, finish at kQueueStride / 2
constexpr size_t kWsCounterBytes = 8192;       // every counter; zero between calls
constexpr size_t kSplitTileFloats = 256 * 256;
constexpr int kSplitMaxGrid = 2048;
inline size_t split_ws_bytes(int grid) {
  return kWsCounterBytes +
         static_cast<size_t>(kSplitXcds) * split_slots_per_xcd(grid) * 2 * kSplitTileFloats * sizeof(float);
}

// GEMM2 with the weighted combine fused: gate weights [T*k] fp32, the
// combined output [T, H] bf16, and the per-(token, column tile) counters
// (T * ceil(H / 128) int32 at most; zero before the call, zero after it).
struct CombineArgs {
  const float* topk_w;
  uint16_t* out;
  int32_t* counters;
};

bool gemm_bf16_supports(int block_m);
hipError_t launch_gemm2_combine_bf16(const GemmArgs& g, const CombineArgs& c, const DeviceInfo& dev, hipStream_t s);
hipError_t launch_gemm1_bf16(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s);
hipError_t launch_gemm2_bf16(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s);
hipError_t launch_gemm1_relu2_bf16(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s);

// Backward (BF16): operands of the dgrad and weight-gradient GEMMs.
struct BwdArgs {
  const void* w1;          // [E, 2I, H]
  const void* w2;          // [E, H, I]
  const void* dy;          // [cap, H] sorted rows
  const void* gu;          // [cap, 2I] saved pre-activations
  void* dgu;               // [cap, 2I] (written by dh, read by dx)
  void* dx_rows;           // [A, H] assignment order
  const int32_t* sorted_ids;
  const int32_t* tile_expert;
  const int32_t* num_tiles;
  const int32_t* offsets;  // [E + 1] padded offsets
  int64_t A;
  int H, I, E, block_m;
  int64_t cap;
};
bool gemm_bwd_supports(int block_m);
hipError_t launch_bwd_dh(const BwdArgs& g, const DeviceInfo& dev, hipStream_t s);
hipError_t launch_bwd_dx(const BwdArgs& g, const DeviceInfo& dev, hipStream_t s);
hipError_t launch_bwd_wgrad(const void* pm, const void* qn, int M, int N, const BwdArgs& g, float* dw,
                            const DeviceInfo& dev, hipStream_t s);
hipError_t launch_backward_combine(const uint16_t* dout, const float* w, const uint16_t* y,
                                   const int32_t* sorted_ids, const int32_t* num_tiles, int block_m, int64_t A,
                                   int kk, int H, int64_t cap, uint16_t* dy, float* dw, hipStream_t s);
hipError_t launch_route_backward(const float* w, const int32_t* ids, const float* dw, int64_t T, int E, int k,
                                 int kk, int score, float* dlogits, hipStream_t s);
hipError_t launch_gather_rows(const uint16_t* x, const int32_t* sorted_ids, const int32_t* num_tiles, int block_m,
                              int64_t A, int kk, int H, int64_t cap, uint16_t* out, hipStream_t s);

bool gemm_fp8_supports(int block_m);
hipError_t launch_gemm1_fp8(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s);
hipError_t launch_gemm2_fp8(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s);

bool gemm_mx_supports(int block_m);
hipError_t launch_gemm1_mx(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s);
hipError_t launch_gemm2_mx(const GemmArgs& g, const DeviceInfo& dev, hipStream_t s);

}  // namespace moe
