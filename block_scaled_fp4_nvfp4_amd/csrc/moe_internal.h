// Internal interfaces between the MoE forward's translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/fp4moe.h"

namespace fp4 {

constexpr int kPermBlock = 256;   // pairs per workgroup of the permutation passes
constexpr int kMaxExperts = 8192; // LDS histogram bound of the permutation
constexpr int kGemmTileM = 64;    // token rows per grouped-GEMM tile

struct WsPlan {
  size_t total, error_flag, counts, offsets, pair_of_row, row_of_pair, active, tile_offsets;
  size_t block_counts, block_invalid, x_tensor_scale, h_tensor_scale, h;
  size_t xq_codes, xq_scales, hq_codes, hq_scales, o;
  size_t sx_codes, sx_scales, sh, sh_codes, sh_scales, s_out;
  size_t x_deq, h_deq;  // MXFP4 x MXFP8 decode: dequantized MXFP8 x (bf16) and h (f32)
  size_t h_amax_part;   // NVFP4 grouped path: max |h| per gate_up workgroup
};

struct WsPtrs {
  int32_t *error_flag, *counts, *offsets, *pair_of_row, *row_of_pair, *active, *tile_offsets;
  int32_t *block_counts, *block_invalid;
  float *x_ts, *h_ts, *h;
  uint8_t* xq_codes;
  void* xq_scales;
  uint8_t* hq_codes;
  void* hq_scales;
  float* o;
  uint8_t *sx_codes, *sx_scales;
  float* sh;
  uint8_t *sh_codes, *sh_scales;
  float* s_out;
  uint16_t* x_deq;
  float* h_deq;
  float* h_amax_part;
};

// Records the caller's stage events (moe_fp4_forward_profiled); no-op without events.
struct Marker {
  void* const* events;
  hipStream_t st;
  int operator()(int i) const {
    if (events && hipEventRecord(reinterpret_cast<hipEvent_t>(events[i]), st) != hipSuccess)
      return FP4_ERR_HIP;
    return FP4_OK;
  }
};

int plan_workspace(const moe_fp4_layer* L, int64_t T, WsPlan* w);
bool w4a8_gemv(const moe_fp4_layer* L, int64_t T);
WsPtrs ws_pointers(const WsPlan& p, void* base);

// grouped MFMA path (quantized activations): steps 2-5 of the forward
int launch_grouped(const moe_fp4_layer* L, const uint16_t* x, int64_t T, const WsPtrs& w,
                   int max_active, hipStream_t st, const Marker& mark);
// shared expert: writes sigmoid(x . g) * shared(x) to w.s_out [T, H]
int launch_shared_expert(const moe_fp4_layer* L, const uint16_t* x, int64_t T, const WsPtrs& w,
                         hipStream_t st);

}  // namespace fp4
