// C ABI front end: argument validation (host only, before anything is
// enqueued), workspace / capacity queries, tile selection and dispatch to the
// gfx950 kernels. See include/moe_mi355x.h for the contract of every call.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "../../include/moe_mi355x.h"
#include "moe_launch.h"

namespace {

constexpr int kMaxDevices = 64;

struct DevCache {
  std::once_flag once;
  bool ok = false;
  moe::DeviceInfo info{};
};
DevCache g_dev[kMaxDevices];

// Architecture check and CU count of the current device, cached per device.
moe_status_t current_device(moe::DeviceInfo* out) {
  int d = -1;
  if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= kMaxDevices) return MOE_ERR_DEVICE;
  DevCache& c = g_dev[d];
  std::call_once(c.once, [&c, d] {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, d) != hipSuccess) return;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return;
    c.info.num_cus = prop.multiProcessorCount;
    c.ok = c.info.num_cus > 0;
  });
  if (!c.ok) return MOE_ERR_DEVICE;
  *out = c.info;
  return MOE_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool valid_block_m(int32_t bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128 || bm == 256; }

bool valid_dtype(int32_t dt) {
  return dt == MOE_DTYPE_BF16 || dt == MOE_DTYPE_FP8_BLOCK128 || dt == MOE_DTYPE_MXFP4W_MXFP8A;
}

int64_t capacity(int64_t T, int32_t k, int32_t E, int32_t bm) {
  const int64_t A = T * k;
  const int64_t ne = A < E ? A : E;
  const int64_t bound = A + ne * (bm - 1);
  return (bound + bm - 1) / bm * bm;
}

moe_status_t launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

// The optional K-split workspace of the grouped GEMMs: NULL, or 256-byte
// aligned and at least moe_grouped_gemm_workspace_bytes() bytes.
moe_status_t check_split_ws(const void* ws, size_t ws_bytes, const moe::DeviceInfo& dev) {
  if (!ws) return MOE_OK;
  if (dev.num_cus > moe::kSplitMaxGrid || ws_bytes < moe::split_ws_bytes(dev.num_cus)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// Shape and pointer checks shared by both grouped GEMMs.
moe_status_t check_gemm(int32_t dtype, const void* act, const void* act_scale, const void* w,
                        const void* w_scale, const int32_t* sorted_ids, const int32_t* tile_expert,
                        const int32_t* num_tiles, int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                        int32_t block_m, int64_t cap, const void* out, const void* out_scale,
                        bool gemm1, bool gated = true) {
  if (!valid_dtype(dtype)) return MOE_ERR_INVALID_ARG;
  if (T < 0 || H <= 0 || I <= 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > E || k > MOE_MAX_TOPK)
    return MOE_ERR_INVALID_ARG;
  if (!valid_block_m(block_m)) return MOE_ERR_INVALID_ARG;
  if (T > (int64_t{1} << 31) / k) return MOE_ERR_INVALID_ARG;
  if (cap != capacity(T, k, E, block_m) || cap >= (int64_t{1} << 31)) return MOE_ERR_INVALID_ARG;
  switch (dtype) {
    case MOE_DTYPE_BF16:
      if (H % 8 || I % 8) return MOE_ERR_UNSUPPORTED_SHAPE;
      if (!moe::gemm_bf16_supports(block_m)) return MOE_ERR_UNSUPPORTED_SHAPE;
      break;
    case MOE_DTYPE_FP8_BLOCK128:
      if (H % 128 || I % 128) return MOE_ERR_UNSUPPORTED_SHAPE;
      if (!moe::gemm_fp8_supports(block_m)) return MOE_ERR_UNSUPPORTED_SHAPE;
      break;
    default:
      if (H % 128 || I % 128) return MOE_ERR_UNSUPPORTED_SHAPE;
      if (!moe::gemm_mx_supports(block_m)) return MOE_ERR_UNSUPPORTED_SHAPE;
      break;
  }
  // the kernels address the token operand and one expert's weights with 32-bit
  // byte offsets
  const int64_t elt = dtype == MOE_DTYPE_BF16 ? 2 : 1;
  const int64_t act_bytes = gemm1 ? T * H * elt : cap * I * elt;
  const int64_t wexp_bytes = (gemm1 && gated ? int64_t{2} * I * H : int64_t{H} * I) * elt;
  if (act_bytes >= (int64_t{1} << 31) || wexp_bytes >= (int64_t{1} << 31)) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (T == 0) return MOE_OK;
  if (!act || !w || !sorted_ids || !tile_expert || !num_tiles || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned(act, 16) || !aligned(w, 16) || !aligned(out, 16)) return MOE_ERR_INVALID_ARG;
  if (!aligned(sorted_ids, 4) || !aligned(tile_expert, 4) || !aligned(num_tiles, 4))
    return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_DTYPE_BF16) {
    if (!act_scale || !w_scale) return MOE_ERR_INVALID_ARG;
    if (!aligned(act_scale, 4) || !aligned(w_scale, 4)) return MOE_ERR_INVALID_ARG;
    if (gemm1 && (!out_scale || !aligned(out_scale, 4))) return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "MOE_ERR_UNSUPPORTED_SHAPE";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
    default: return "MOE_ERR_UNKNOWN";
  }
}

moe_status_t moe_route_shared(const float* logits, int64_t T, int32_t E, int32_t k, int32_t score,
                              int32_t n_shared, int32_t* topk_ids, float* topk_w, void* stream) {
  if (T < 0 || E < 1 || k < 1 || k > E || n_shared < 0 || k + n_shared > MOE_MAX_TOPK)
    return MOE_ERR_INVALID_ARG;
  if (E + n_shared > MOE_MAX_EXPERTS) return MOE_ERR_INVALID_ARG;
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (T > (int64_t{1} << 31) / (k + n_shared)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4)) return MOE_ERR_INVALID_ARG;
  moe::DeviceInfo dev;
  if (moe_status_t st = current_device(&dev)) return st;
  return launched(moe::launch_route(logits, T, E, k, score, n_shared, topk_ids, topk_w,
                                    static_cast<hipStream_t>(stream)));
}

moe_status_t moe_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t score,
                       int32_t* topk_ids, float* topk_w, void* stream) {
  return moe_route_shared(logits, T, E, k, score, 0, topk_ids, topk_w, stream);
}

int32_t moe_pick_block_m(int32_t dtype, int64_t T, int32_t k, int32_t E, int32_t H, int32_t I) {
  if (!valid_dtype(dtype) || T < 0 || k < 1 || E < 1 || k > E || H <= 0 || I <= 0) return -1;
  const int64_t A = T * k;
  const int64_t mean = A / E;  // mean rows per expert
  // BF16 (all tiles stream their weight rows two k-steps ahead): 256-row
  // tiles stage the fewest bytes per MFMA and win from about 160 rows per
  // expert, 128-row ones from 64, 64-row ones from 24; measured over the
  // Qwen3-30B-A3B, Scout and Nemotron shapes at T = 256 .. 8192 (the whole
  // forward, each row-tile size in turn), this picks the fastest or one
  // within 5%
  if (dtype == MOE_DTYPE_BF16) {
    if (mean >= 160) return 256;
    if (mean >= 64) return 128;
    if (mean >= 24) return 64;
    return 32;
  }
  // MXFP4 x MXFP8 (same measurement over T = 1024 .. 16384 of the
  // 512-expert shape): 128-row tiles from about 56 rows per expert (at 160
  // rows 1020 against 1121 us with 64-row tiles), 64-row ones from 28
  if (dtype == MOE_DTYPE_MXFP4W_MXFP8A) {
    if (mean >= 56) return 128;
    if (mean >= 28) return 64;
    return 32;
  }
  // FP8 128-block (same measurement over T = 256 .. 8192 of the 64-expert
  // H 7168 shape): 256-row tiles from about 384 rows per expert (the 128- and
  // 64-row tiles split their LDS stages, the 256-row GEMM1 tile cannot: at
  // 256 rows 1097 against 1041 TFLOP/s with 256-row tiles, at 512 rows 1238
  // against 1281), 128-row ones from 48 (at 64 rows 564 against 480 TFLOP/s
  // with 64-row tiles)
  if (mean >= 384) return 256;
  if (mean >= 48) return 128;
  if (mean >= 24) return 64;
  return 32;
}

int64_t moe_sorted_capacity(int64_t T, int32_t k, int32_t E, int32_t block_m) {
  if (T < 0 || k < 1 || E < 1 || !valid_block_m(block_m)) return -1;
  return capacity(T, k, E, block_m);
}

size_t moe_align_sort_workspace_bytes(int64_t T, int32_t k, int32_t E) {
  if (T < 0 || k < 1 || E < 1 || E > MOE_MAX_EXPERTS) return 0;
  return moe::align_sort_ws_bytes(T, k, E);
}

moe_status_t moe_align_sort(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t block_m,
                            int32_t* counts, int32_t* offsets, int32_t* sorted_ids, int32_t* tile_expert,
                            int32_t* num_tiles, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > E || k > MOE_MAX_TOPK)
    return MOE_ERR_INVALID_ARG;
  if (!valid_block_m(block_m)) return MOE_ERR_INVALID_ARG;
  if (T > (int64_t{1} << 31) / k) return MOE_ERR_INVALID_ARG;
  const int64_t cap = capacity(T, k, E, block_m);
  if (cap >= (int64_t{1} << 31)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!topk_ids || !counts || !offsets || !sorted_ids || !tile_expert || !num_tiles)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(topk_ids, 4) || !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(sorted_ids, 4) ||
      !aligned(tile_expert, 4) || !aligned(num_tiles, 4))
    return MOE_ERR_INVALID_ARG;
  if (ws_bytes < moe::align_sort_ws_bytes(T, k, E) || !ws || !aligned(ws, 4)) return MOE_ERR_WORKSPACE;
  moe::DeviceInfo dev;
  if (moe_status_t st = current_device(&dev)) return st;
  return launched(moe::launch_align_sort(topk_ids, T, k, E, block_m, counts, offsets, sorted_ids,
                                         tile_expert, num_tiles, cap, ws,
                                         static_cast<hipStream_t>(stream)));
}

moe_status_t moe_align_sort_noalloc(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t block_m,
                                    int32_t* counts, int32_t* offsets, int32_t* sorted_ids, int32_t* tile_expert,
                                    int32_t* num_tiles, void* stream) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > E || k > MOE_MAX_TOPK)
    return MOE_ERR_INVALID_ARG;
  if (!valid_block_m(block_m)) return MOE_ERR_INVALID_ARG;
  if (T > (int64_t{1} << 31) / k) return MOE_ERR_INVALID_ARG;
  const int64_t cap = capacity(T, k, E, block_m);
  if (cap >= (int64_t{1} << 31)) return MOE_ERR_INVALID_ARG;
  // the fixed scratch covers MOE_NOALLOC_MAX_ASSIGNMENTS assignments
  if (T * k > MOE_NOALLOC_MAX_ASSIGNMENTS) return MOE_ERR_WORKSPACE;
  if (moe::align_sort_ws_bytes(T, k, E) > moe::align_sort_scratch_bytes()) return MOE_ERR_WORKSPACE;
  if (T == 0) return MOE_OK;
  if (!topk_ids || !counts || !offsets || !sorted_ids || !tile_expert || !num_tiles) return MOE_ERR_INVALID_ARG;
  if (!aligned(topk_ids, 4) || !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(sorted_ids, 4) ||
      !aligned(tile_expert, 4) || !aligned(num_tiles, 4))
    return MOE_ERR_INVALID_ARG;
  moe::DeviceInfo dev;
  if (moe_status_t st = current_device(&dev)) return st;
  void* ws = nullptr;
  if (moe::align_sort_scratch(&ws) != hipSuccess || ws == nullptr) return MOE_ERR_DEVICE;
  return launched(moe::launch_align_sort(topk_ids, T, k, E, block_m, counts, offsets, sorted_ids,
                                         tile_expert, num_tiles, cap, ws, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_quantize_fp8(const uint16_t* in, int64_t rows, int64_t cols, int32_t block_rows,
                              uint8_t* q, float* scale, void* stream) {
  if (rows < 0 || cols < 0 || (block_rows != 1 && block_rows != 128)) return MOE_ERR_INVALID_ARG;
  if (rows % block_rows || cols % 128) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (rows == 0 || cols == 0) return MOE_OK;
  if (!in || !q || !scale) return MOE_ERR_INVALID_ARG;
  if (!aligned(in, 16) || !aligned(q, 8) || !aligned(scale, 4)) return MOE_ERR_INVALID_ARG;
  moe::DeviceInfo dev;
  if (moe_status_t st = current_device(&dev)) return st;
  return launched(moe::launch_quantize_fp8(in, rows, cols, block_rows, q, scale,
                                           static_cast<hipStream_t>(stream)));
}

moe_status_t moe_quantize_mxfp8(const uint16_t* in, int64_t rows, int64_t cols, uint8_t* q, uint8_t* e8m0,
                                void* stream) {
  if (rows < 0 || cols < 0) return MOE_ERR_INVALID_ARG;
  if (cols % 32) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (rows == 0 || cols == 0) return MOE_OK;
  if (!in || !q || !e8m0) return MOE_ERR_INVALID_ARG;
  if (!aligned(in, 16) || !aligned(q, 8)) return MOE_ERR_INVALID_ARG;
  moe::DeviceInfo dev;
  if (moe_status_t st = current_device(&dev)) return st;
  return launched(moe::launch_quantize_mx(in, rows, cols, false, q, e8m0, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_quantize_mxfp4(const uint16_t* in, int64_t rows, int64_t cols, uint8_t* q, uint8_t* e8m0,
                                void* stream) {
  if (rows < 0 || cols < 0) return MOE_ERR_INVALID_ARG;
  if (cols % 32) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (rows == 0 || cols == 0) return MOE_OK;
  if (!in || !q || !e8m0) return MOE_ERR_INVALID_ARG;
  if (!aligned(in, 16) || !aligned(q, 4)) return MOE_ERR_INVALID_ARG;
  moe::DeviceInfo dev;
  if (moe_status_t st = current_device(&dev)) return st;
  return launched(moe::launch_quantize_mx(in, rows, cols, true, q, e8m0, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_grouped_gemm_swiglu(int32_t dtype, const void* x, const void* x_scale, const void* w1,
                                     const void* w1_scale, const int32_t* sorted_ids,
                                     const int32_t* tile_expert, const int32_t* num_tiles, int64_t T,
                                     int32_t H, int32_t I, int32_t E, int32_t k, int32_t block_m, int64_t cap,
                                     void* h, void* h_scale, void* ws, size_t ws_bytes, void* stream) {
  if (moe_status_t st = check_gemm(dtype, x, x_scale, w1, w1_scale, sorted_ids, tile_expert, num_tiles, T, H,
                                   I, E, k, block_m, cap, h, h_scale, true))
    return st;
  if (T == 0) return MOE_OK;
  if (ws && !aligned(ws, 256)) return MOE_ERR_INVALID_ARG;
  moe::DeviceInfo dev;
  if (moe_status_t st = current_device(&dev)) return st;
  if (moe_status_t st = check_split_ws(ws, ws_bytes, dev)) return st;
  moe::GemmArgs g{x, x_scale, w1, w1_scale, sorted_ids, tile_expert, num_tiles, h, h_scale,
                  T, H, I, E, k, block_m, cap};
  g.split_ws = ws;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case MOE_DTYPE_BF16:
      g.out_scale = nullptr;   // (h_scale is ignored on the BF16 path)
      return launched(moe::launch_gemm1_bf16(g, dev, s));
    case MOE_DTYPE_FP8_BLOCK128: return launched(moe::launch_gemm1_fp8(g, dev, s));
    default: return launched(moe::launch_gemm1_mx(g, dev, s));
  }
}

moe_status_t moe_grouped_gemm_swiglu_h32(int32_t dtype, const void* x, const void* x_scale, const void* w1,
                                         const void* w1_scale, const int32_t* sorted_ids,
                                         const int32_t* tile_expert, const int32_t* num_tiles, int64_t T,
                                         int32_t H, int32_t I, int32_t E, int32_t k, int32_t block_m, int64_t cap,
                                         void* h, void* h_scale, float* h32, void* ws, size_t ws_bytes,
                                         void* stream) {
  if (moe_status_t st = check_gemm(dtype, x, x_scale, w1, w1_scale, sorted_ids, tile_expert, num_tiles, T, H,
                                   I, E, k, block_m, cap, h, h_scale, true))
    return st;
  if (T == 0) return MOE_OK;
  if (!h32 || !aligned(h32, 16)) return MOE_ERR_INVALID_ARG;
  if (ws && !aligned(ws, 256)) return MOE_ERR_INVALID_ARG;
  moe::DeviceInfo dev;
  if (moe_status_t st = current_device(&dev)) return st;
  if (moe_status_t st = check_split_ws(ws, ws_bytes, dev)) return st;
  moe::GemmArgs g{x, x_scale, w1, w1_scale, sorted_ids, tile_expert, num_tiles, h, h_scale,
                  T, H, I, E, k, block_m, cap};
  g.h32 = h32;
  g.split_ws = ws;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case MOE_DTYPE_BF16:
      g.out_scale = nullptr;
      return launched(moe::launch_gemm1_bf16(g, dev, s));
    case MOE_DTYPE_FP8_BLOCK128: return launched(moe::launch_gemm1_fp8(g, dev, s));
    default: return launched(moe::launch_gemm1_mx(g, dev, s));
  }
}

moe_status_t moe_grouped_gemm_swiglu_save(const void* x, const void* w1, const int32_t* sorted_ids,
                                          const int32_t* tile_expert, const int32_t* num_tiles, int64_t T,
                                          int32_t H, int32_t I, int32_t E, int32_t k, int32_t block_m, int64_t cap,
                                          void* h, void* gu, void* stream) {
  if (moe_status_t st = check_gemm(MOE_DTYPE_BF16, x, nullptr, w1, nullptr, sorted_ids, tile_expert, num_tiles, T,
                                   H, I, E, k, block_m, cap, h, nullptr, true))
    return st;
  if (T == 0) return MOE_OK;
  if (!gu || !aligned(gu, 16)) return MOE_ERR_INVALID_ARG;
  moe::DeviceInfo dev;
  if (moe_status_t st = current_device(&dev)) return st;
  moe::GemmArgs g{x, nullptr, w1, nullptr, sorted_ids, tile_expert, num_tiles, h, gu, T, H, I, E, k, block_m, cap};
  return launched(moe::launch_gemm1_bf16(g, dev, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_grouped_gemm_relu2(int32_t dtype, const void* x, const void* x_scale, const void* w1,
                                    const void* w1_scale, const int32_t* sorted_ids, const int32_t* tile_expert,
                                    const int32_t* num_tiles, int64_t T, int32_t H, int32_t I, int32_t E,
                                    int32_t k, int32_t block_m, int64_t cap, void* h, void* h_scale, void* ws,
                                    size_t ws_bytes, void* stream) {
  if (moe_status_t st = check_gemm(dtype, x, x_scale, w1, w1_scale, sorted_ids, tile_expert, num_tiles, T, H,
                                   I, E, k, block_m, cap, h, h_scale, true, false))
    return st;
  if (dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (T == 0) return MOE_OK;
  if (ws && !aligned(ws, 256)) return MOE_ERR_INVALID_ARG;
  moe::DeviceInfo dev;
  if (moe_status_t st = current_device(&dev)) return st;
  if (moe_status_t st = check_split_ws(ws, ws_bytes, dev)) return st;
  moe::GemmArgs g{x, x_scale, w1, w1_scale, sorted_ids, tile_expert, num_tiles, h, h_scale,
                  T, H, I, E, k, block_m, cap};
  g.split_ws = ws;
  return launched(moe::launch_gemm1_relu2_bf16(g, dev, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_grouped_gemm_down(int32_t dtype, const void* h, const void* h_scale, const void* w2,
                                   const void* w2_scale, const int32_t* sorted_ids, const int32_t* tile_expert,
                                   const int32_t* num_tiles, int64_t T, int32_t H, int32_t I, int32_t E,
                                   int32_t k, int32_t block_m, int64_t cap, uint16_t* y, void* ws, size_t ws_bytes,
                                   void* stream) {
  if (moe_status_t st = check_gemm(dtype, h, h_scale, w2, w2_scale, sorted_ids, tile_expert, num_tiles, T, H, I,
                                   E, k, block_m, cap, y, nullptr, false))
    return st;
  if (T == 0) return MOE_OK;
  if (ws && !aligned(ws, 256)) return MOE_ERR_INVALID_ARG;
  moe::DeviceInfo dev;
  if (moe_status_t st = current_device(&dev)) return st;
  if (moe_status_t st = check_split_ws(ws, ws_bytes, dev)) return st;
  moe::GemmArgs g{h, h_scale, w2, w2_scale, sorted_ids, tile_expert, num_tiles, y, nullptr,
                  T, H, I, E, k, block_m, cap};
  g.split_ws = ws;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case MOE_DTYPE_BF16: return launched(moe::launch_gemm2_bf16(g, dev, s));
    case MOE_DTYPE_FP8_BLOCK128: return launched(moe::launch_gemm2_fp8(g, dev, s));
    default: return launched(moe::launch_gemm2_mx(g, dev, s));
  }
}

size_t moe_grouped_gemm_workspace_bytes(void) {
  moe::DeviceInfo dev;
  if (current_device(&dev) != MOE_OK || dev.num_cus > moe::kSplitMaxGrid) return 0;
  return moe::split_ws_bytes(dev.num_cus);
}

size_t moe_down_combine_workspace_bytes(int64_t T, int32_t H) {
  if (T < 0 || H <= 0) return 0;
  return static_cast<size_t>(T) * static_cast<size_t>((H + 127) / 128) * sizeof(int32_t);
}

moe_status_t moe_grouped_gemm_down_combine(int32_t dtype, const void* h, const void* h_scale, const void* w2,
                                           const void* w2_scale, const int32_t* sorted_ids,
                                           const int32_t* tile_expert, const int32_t* num_tiles, int64_t T,
                                           int32_t H, int32_t I, int32_t E, int32_t k, int32_t block_m, int64_t cap,
                                           uint16_t* y, const float* topk_w, uint16_t* out, int32_t* counters,
                                           size_t counters_bytes, void* stream) {
  if (moe_status_t st = check_gemm(dtype, h, h_scale, w2, w2_scale, sorted_ids, tile_expert, num_tiles, T, H, I,
                                   E, k, block_m, cap, y, nullptr, false))
    return st;
  if (dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED_SHAPE;
  // the kernel addresses y with 32-bit byte offsets
  if (T * k * static_cast<int64_t>(H) * 2 >= (int64_t{1} << 31)) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (T == 0) return MOE_OK;
  if (!topk_w || !out || !counters || !aligned(out, 16) || !aligned(topk_w, 4) || !aligned(counters, 4))
    return MOE_ERR_INVALID_ARG;
  if (counters_bytes < moe_down_combine_workspace_bytes(T, H)) return MOE_ERR_WORKSPACE;
  moe::DeviceInfo dev;
  if (moe_status_t st = current_device(&dev)) return st;
  moe::GemmArgs g{h, h_scale, w2, w2_scale, sorted_ids, tile_expert, num_tiles, y, nullptr,
                  T, H, I, E, k, block_m, cap};
  moe::CombineArgs c{topk_w, out, counters};
  return launched(moe::launch_gemm2_combine_bf16(g, c, dev, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------ backward (BF16)
namespace {

moe_status_t check_bwd(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t block_m, int64_t cap) {
  if (T < 0 || H <= 0 || I <= 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > E || k > MOE_MAX_TOPK)
    return MOE_ERR_INVALID_ARG;
  if (!valid_block_m(block_m)) return MOE_ERR_INVALID_ARG;
  if (T > (int64_t{1} << 31) / k) return MOE_ERR_INVALID_ARG;
  if (cap != capacity(T, k, E, block_m) || cap >= (int64_t{1} << 31)) return MOE_ERR_INVALID_ARG;
  if (H % 8 || I % 8) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (!moe::gemm_bwd_supports(block_m)) return MOE_ERR_UNSUPPORTED_SHAPE;
  // 32-bit buffer offsets: the sorted-row operands and one expert's weights
  const int64_t big = cap * int64_t{2} * I * 2 > cap * int64_t{H} * 2 ? cap * int64_t{2} * I * 2 : cap * int64_t{H} * 2;
  if (big >= (int64_t{1} << 31) || int64_t{2} * I * H * 2 >= (int64_t{1} << 31)) return MOE_ERR_UNSUPPORTED_SHAPE;
  return MOE_OK;
}

}  // namespace

moe_status_t moe_backward_combine(const uint16_t* dout, const float* topk_w, const uint16_t* y,
                                  const int32_t* sorted_ids, const int32_t* num_tiles, int64_t T, int32_t k,
                                  int32_t H, int32_t block_m, int64_t cap, uint16_t* dy, float* dw, void* stream) {
  if (T < 0 || k < 1 || k > MOE_MAX_TOPK || H <= 0 || cap < 0 || !valid_block_m(block_m)) return MOE_ERR_INVALID_ARG;
  if (H % 8) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (T == 0 || cap == 0) return MOE_OK;
  if (!dout || !topk_w || !y || !sorted_ids || !num_tiles || !dy || !dw) return MOE_ERR_INVALID_ARG;
  if (!aligned(dout, 16) || !aligned(y, 16) || !aligned(dy, 16) || !aligned(topk_w, 4) || !aligned(dw, 4))
    return MOE_ERR_INVALID_ARG;
  moe::DeviceInfo dev;
  if (moe_status_t st = current_device(&dev)) return st;
  return launched(moe::launch_backward_combine(dout, topk_w, y, sorted_ids, num_tiles, block_m, T * k, k, H, cap,
                                               dy, dw, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_route_backward(const float* topk_w, const int32_t* topk_ids, const float* dw, int64_t T,
                                int32_t E, int32_t k, int32_t n_shared, int32_t score, float* dlogits,
                                void* stream) {
  if (T < 0 || E < 1 || k < 1 || k > E || n_shared < 0 || k + n_shared > MOE_MAX_TOPK) return MOE_ERR_INVALID_ARG;
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!topk_w || !topk_ids || !dw || !dlogits) return MOE_ERR_INVALID_ARG;
  moe::DeviceInfo dev;
  if (moe_status_t st = current_device(&dev)) return st;
  return launched(moe::launch_route_backward(topk_w, topk_ids, dw, T, E, k, k + n_shared, score, dlogits,
                                             static_cast<hipStream_t>(stream)));
}

moe_status_t moe_gather_rows(const uint16_t* x, const int32_t* sorted_ids, const int32_t* num_tiles, int64_t T,
                             int32_t k, int32_t H, int32_t block_m, int64_t cap, uint16_t* x_sorted, void* stream) {
  if (T < 0 || k < 1 || H <= 0 || cap < 0 || !valid_block_m(block_m)) return MOE_ERR_INVALID_ARG;
  if (H % 8) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (T == 0 || cap == 0) return MOE_OK;
  if (!x || !sorted_ids || !num_tiles || !x_sorted || !aligned(x, 16) || !aligned(x_sorted, 16))
    return MOE_ERR_INVALID_ARG;
  moe::DeviceInfo dev;
  if (moe_status_t st = current_device(&dev)) return st;
  return launched(moe::launch_gather_rows(x, sorted_ids, num_tiles, block_m, T * k, k, H, cap, x_sorted,
                                          static_cast<hipStream_t>(stream)));
}

moe_status_t moe_grouped_gemm_dh(const void* dy, const void* w2, const void* gu, const int32_t* sorted_ids,
                                 const int32_t* tile_expert, const int32_t* num_tiles, int64_t T, int32_t H,
                                 int32_t I, int32_t E, int32_t k, int32_t block_m, int64_t cap, void* dgu,
                                 void* stream) {
  if (moe_status_t st = check_bwd(T, H, I, E, k, block_m, cap)) return st;
  if (T == 0) return MOE_OK;
  if (!dy || !w2 || !gu || !dgu || !sorted_ids || !tile_expert || !num_tiles) return MOE_ERR_INVALID_ARG;
  if (!aligned(dy, 16) || !aligned(w2, 16) || !aligned(gu, 16) || !aligned(dgu, 16)) return MOE_ERR_INVALID_ARG;
  moe::DeviceInfo dev;
  if (moe_status_t st = current_device(&dev)) return st;
  moe::BwdArgs g{nullptr, w2, dy, gu, dgu, nullptr, sorted_ids, tile_expert, num_tiles, nullptr,
                 T * k, H, I, E, block_m, cap};
  return launched(moe::launch_bwd_dh(g, dev, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_grouped_gemm_dx(const void* dgu, const void* w1, const int32_t* sorted_ids,
                                 const int32_t* tile_expert, const int32_t* num_tiles, int64_t T, int32_t H,
                                 int32_t I, int32_t E, int32_t k, int32_t block_m, int64_t cap, void* dx_rows,
                                 void* stream) {
  if (moe_status_t st = check_bwd(T, H, I, E, k, block_m, cap)) return st;
  if (T == 0) return MOE_OK;
  if (!dgu || !w1 || !dx_rows || !sorted_ids || !tile_expert || !num_tiles) return MOE_ERR_INVALID_ARG;
  if (!aligned(dgu, 16) || !aligned(w1, 16) || !aligned(dx_rows, 16)) return MOE_ERR_INVALID_ARG;
  moe::DeviceInfo dev;
  if (moe_status_t st = current_device(&dev)) return st;
  moe::BwdArgs g{w1, nullptr, nullptr, nullptr, const_cast<void*>(dgu), dx_rows, sorted_ids, tile_expert, num_tiles,
                 nullptr, T * k, H, I, E, block_m, cap};
  return launched(moe::launch_bwd_dx(g, dev, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_grouped_gemm_wgrad(const void* p_rows, const void* q_rows, int32_t M, int32_t N,
                                    const int32_t* offsets, int64_t T, int32_t E, int32_t k, int32_t block_m,
                                    int64_t cap, float* dw, void* stream) {
  if (M <= 0 || N <= 0) return MOE_ERR_INVALID_ARG;
  if (moe_status_t st = check_bwd(T, N, M, E, k, block_m, cap)) return st;
  if (T == 0) return MOE_OK;
  if (cap * int64_t{M} * 2 >= (int64_t{1} << 31) || cap * int64_t{N} * 2 >= (int64_t{1} << 31))
    return MOE_ERR_UNSUPPORTED_SHAPE;
  if (!p_rows || !q_rows || !offsets || !dw) return MOE_ERR_INVALID_ARG;
  if (!aligned(p_rows, 16) || !aligned(q_rows, 16) || !aligned(dw, 16)) return MOE_ERR_INVALID_ARG;
  moe::DeviceInfo dev;
  if (moe_status_t st = current_device(&dev)) return st;
  moe::BwdArgs g{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, offsets,
                 T * k, 0, 0, E, block_m, cap};
  return launched(moe::launch_bwd_wgrad(p_rows, q_rows, M, N, g, dw, dev, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_combine(const uint16_t* y, const float* topk_w, int64_t T, int32_t k, int32_t H,
                         uint16_t* out, void* stream) {
  if (T < 0 || k < 1 || k > MOE_MAX_TOPK || H <= 0) return MOE_ERR_INVALID_ARG;
  if (H % 8) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (T == 0) return MOE_OK;
  if (!y || !topk_w || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned(y, 16) || !aligned(out, 16) || !aligned(topk_w, 4)) return MOE_ERR_INVALID_ARG;
  moe::DeviceInfo dev;
  if (moe_status_t st = current_device(&dev)) return st;
  return launched(moe::launch_combine(y, topk_w, T, k, H, out, dev, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
