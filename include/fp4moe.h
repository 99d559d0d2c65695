/*
 * fp4moe.h - C ABI of the block-scaled FP4 routed-expert MoE library (gfx950).
 *
 * Formats, as the model cards on block_scaled_fp4_nvfp4 state them:
 *  - NVFP4: E2M1 values packed two per byte, one E4M3 block scale per 16 values
 *    ("weight_scale"), one FP32 tensor scale per tensor ("weight_scale_2");
 *    activations use the tensor scale amax/2688 ("Local-Hessian NVFP4
 *    experts", opening section); gate and up share one tensor scale (same
 *    passage); one tensor scale per expert (section "What is different about it").
 *  - The per-block 4/6 choice: the block scale maps the block max to 6 or to 4,
 *    whichever gives the smaller exact post-rounding squared error ("dabsLabs
 *    NVFP4 (4/6-optimal scales)", section "What makes this build different").
 *  - MXFP4: E2M1 values with one UE8M0 scale per 32 ("MXFP4-FP8-R12",
 *    section "Quantization format").
 *  - MXFP8: E4M3 values, one power-of-two scale per 32, e = ceil(log2(amax/448))
 *    ("FP4-Local AZ", section "The shared expert").
 *  - Block FP8: E4M3 weights with one FP32 scale per 128 x 128 tile, dynamic
 *    E4M3 activations with one FP32 scale per (row, 128 columns)
 *    ("MXFP4-FP8-R12", runtime contract table: retained block-FP8 experts on a
 *    dynamic-FP8 path).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers of the current HIP device; the
 *    caller owns every buffer.  The library never allocates or frees device
 *    memory.  State kept between calls: a thread-local error text and, per
 *    device, one helper stream with two events (created by the first forward
 *    of a layer with a shared expert; the shared expert runs on it,
 *    overlapped with the routed experts, forked from and joined back into
 *    the caller's stream), the device's compute-unit count, one bit per
 *    GEMM kernel recording that its dynamic-LDS limit has been raised, and
 *    the address of the device's scratch array of moe_fp4_forward_noalloc
 *    (the array itself is part of the loaded code object).
 *  - `stream` is a hipStream_t (NULL = default stream).  Calls only enqueue
 *    work and return; a launch failure returns FP4_ERR_HIP, asynchronous faults
 *    surface at the caller's next synchronisation.
 *  - Layouts are row-major; blocks run along the last (reduction) dimension.
 *    Packed 4-bit codes: element 2i in the low nibble of byte i, element 2i+1 in
 *    the high nibble; the nibble's bit 3 is the sign.
 *  - Errors are negative fp4_status values; fp4_last_error() describes the last
 *    one raised on the calling thread.  A zero-sized problem is a no-op (FP4_OK).
 */
#ifndef FP4MOE_H
#define FP4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP4_OK = 0,
  FP4_ERR_INVALID_ARG = -1, /* null pointer, unknown enum, k out of range   */
  FP4_ERR_SHAPE = -2,       /* a dimension is not a multiple of its block    */
  FP4_ERR_UNSUPPORTED = -3, /* combination of formats not provided           */
  FP4_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required    */
  FP4_ERR_HIP = -5          /* a HIP launch or runtime call failed           */
} fp4_status;

typedef enum {
  FP4_FMT_NVFP4 = 0,     /* E2M1 codes [.., cols/2], E4M3 scales [.., cols/16], f32 tensor scale */
  FP4_FMT_MXFP4 = 1,     /* E2M1 codes [.., cols/2], UE8M0 scales [.., cols/32]                  */
  FP4_FMT_MXFP8 = 2,     /* E4M3 codes [.., cols],   UE8M0 scales [.., cols/32]                  */
  FP4_FMT_FP8_BLOCK = 3, /* E4M3 codes [b, rows, cols], f32 scales [b, rows/128, cols/128]        */
  FP4_FMT_FP8_ROW = 4,   /* E4M3 codes [.., cols],   f32 scales [.., cols/128] (per row)          */
  FP4_FMT_NONE = 5       /* 16-bit activations (weight-only quantization)                        */
} fp4_format;

typedef enum {
  FP4_RULE_RTN = 0,    /* block max mapped to 6 (the amax/6 plan)                       */
  FP4_RULE_4OVER6 = 1, /* per block, the amax/6 or the block-max-to-4 plan, whichever has
                          the strictly smaller exact squared error (ties keep amax/6)      */
  FP4_RULE_SWEEP = 2   /* scale sweep (the "MSE sweep" the LocalHessian-Experts card names
                          in "What is different about it"; reading: NVFP4 tries every E4M3
                          scale from the amax/6 plan's code to the block-max-to-4 plan's
                          code, keeping the first with the smallest exact squared error;
                          for MXFP4 those plans are the only power-of-two candidates, so it
                          equals FP4_RULE_4OVER6)                                          */
} fp4_rule;

typedef enum { FP4_DT_BF16 = 0, FP4_DT_F32 = 1 } fp4_dtype;

typedef enum {
  FP4_TS_DYNAMIC = 0, /* NVFP4: compute S = fp32(amax / 2688) per tensor, write it */
  FP4_TS_STATIC = 1   /* NVFP4: read the caller's tensor scale                     */
} fp4_ts_mode;

/*
 * fp4_quantize - quantize `batch` independent tensors x[batch][rows][cols].
 *
 *  fmt      NVFP4, MXFP4 (rule applies), MXFP8, FP8_BLOCK or FP8_ROW.
 *  rule     FP4_RULE_RTN, FP4_RULE_4OVER6 or FP4_RULE_SWEEP (NVFP4 and MXFP4 only;
 *           ignored otherwise).
 *  x        bf16 or f32 values, `x_dtype`; must be finite.
 *  codes    out: packed E2M1 [batch, rows, cols/2] (NVFP4, MXFP4) or E4M3 bytes
 *           [batch, rows, cols] (MXFP8, FP8_*).
 *  scales   out: E4M3 bytes [batch, rows, cols/16] (NVFP4), UE8M0 bytes
 *           [batch, rows, cols/32] (MXFP4, MXFP8), f32 [batch, rows/128, cols/128]
 *           (FP8_BLOCK) or f32 [batch, rows, cols/128] (FP8_ROW).
 *  tensor_scale  NVFP4 only, f32 [batch]: written (FP4_TS_DYNAMIC) or read
 *           (FP4_TS_STATIC).  One tensor per batch item, so a fused gate_up
 *           [2I, H] quantized as one item shares its scale between gate and up.
 *  m4_flags optional out (may be NULL), one byte per block: 1 where the
 *           block-max-to-4 plan was chosen; under FP4_RULE_SWEEP with NVFP4, the
 *           chosen scale code minus the amax/6 plan's code (0: the amax/6 plan).
 * Shape errors: cols % 16 (NVFP4), % 32 (MX), % 128 (FP8_*), rows % 128 (FP8_BLOCK).
 */
int fp4_quantize(int fmt, int rule, int ts_mode, const void* x, int x_dtype,
                 int64_t batch, int64_t rows, int64_t cols, uint8_t* codes,
                 void* scales, float* tensor_scale, uint8_t* m4_flags,
                 void* stream);

/*
 * fp4_quantize_hessian - NVFP4 quantization of `experts` expert matrices
 * x[experts][rows][cols] with block scales chosen by a Hessian-weighted search
 * ("Local-Hessian NVFP4 experts", section "What is different about it": the
 * per-group weight scales come from a Hessian-weighted search instead of the
 * plain amax / MSE sweep, and only weight_scale values differ; section
 * "Results": experts with fewer than 64 routed calibration rows keep plain
 * max).  The search is named, not defined, there; the reading taken:
 *   candidates  every E4M3 scale code from the amax/6 plan's to the
 *               block-max-to-4 plan's, codes E2M1 round-to-nearest-even;
 *   error       d^T H_b d per 16-value block, d = x - xhat (signed), H_b the
 *               16 x 16 diagonal block of the expert's input Hessian for the
 *               block's columns; the first candidate with the smallest exact
 *               error is kept (exact: float64 with a proven error bound, and
 *               exact fixed-point arithmetic where the bound cannot decide).
 *  x            bf16 or f32 (`x_dtype`), finite, 16-byte aligned.
 *  hessian      f32 [experts][cols/16][16][16], H_b of every column block
 *               (finite; the search uses sum_ij H_b[i][j] d_i d_j as given).
 *  calib_rows   int32 [experts]: calibration rows behind each expert's
 *               Hessian; fewer than 64 -> the amax/6 plan for all its blocks.
 *  codes, scales, tensor_scale  out, as fp4_quantize NVFP4 with
 *               FP4_TS_DYNAMIC (tensor scale amax/2688 per expert, unchanged
 *               by the search); codes 8-byte aligned.
 *  choice       optional out (may be NULL), one byte per block: the chosen
 *               scale code minus the amax/6 plan's.
 * Errors: cols % 16 -> FP4_ERR_SHAPE; bad dtype, null or misaligned pointer
 * -> FP4_ERR_INVALID_ARG.  Stream-ordered, asynchronous.
 */
int fp4_quantize_hessian(const void* x, int x_dtype, int64_t experts, int64_t rows, int64_t cols,
                         const float* hessian, const int32_t* calib_rows, uint8_t* codes,
                         uint8_t* scales, float* tensor_scale, uint8_t* choice, void* stream);

/*
 * fp4_dequantize - decode codes/scales (layouts as fp4_quantize) to
 * out[batch][rows][cols] in `out_dtype`.  f32 output is the correctly rounded
 * value g * s * S (NVFP4), g * 2^e (MX) or v * sigma (FP8_*); bf16 output is
 * that f32 value rounded to nearest-even bf16.
 */
int fp4_dequantize(int fmt, const uint8_t* codes, const void* scales,
                   const float* tensor_scale, int64_t batch, int64_t rows,
                   int64_t cols, void* out, int out_dtype, void* stream);

/*
 * fp4_block_error - the squared quantization error of every block, the
 * quantity the 4/6 rule compares between its two candidate scales
 * ("dabsLabs NVFP4", section "What makes this build different"):
 *   err[g] = sum over block g of (x - xhat)^2,
 * x [batch][rows][cols] (bf16 or f32, 16-byte aligned) and its NVFP4 (blocks
 * of 16) or MXFP4 (blocks of 32) quantization (codes, scales, tensor_scale
 * as fp4_quantize wrote them), xhat the f32 value fp4_dequantize gives; each
 * difference, square and sum rounded to f32.  err: f32 [batch][rows][cols /
 * block], device memory, caller-owned.  Errors: other formats ->
 * FP4_ERR_UNSUPPORTED; cols % block -> FP4_ERR_SHAPE; null or misaligned
 * pointer -> FP4_ERR_INVALID_ARG.  Stream-ordered, asynchronous.
 */
int fp4_block_error(int fmt, const void* x, int x_dtype, int64_t batch, int64_t rows,
                    int64_t cols, const uint8_t* codes, const void* scales,
                    const float* tensor_scale, float* err, void* stream);

/*
 * One routed-expert MoE layer.  E experts, hidden H, expert intermediate I,
 * top-k routing.  Expert weights are stacked: fused gate_up W13 [E, 2I, H]
 * (rows [0, I) gate, [I, 2I) up) and down W2 [E, H, I], in the layouts of
 * fp4_quantize with batch = E ("dabsLabs NVFP4", section "What makes this
 * build different": stacked [512, out, in] with fused gate_up).  Widths and k
 * are runtime values ("FP4-Local AZ": the engine must read the routing width
 * and the shared-expert width from the configuration).
 *
 * Supported (w_fmt, a_fmt) pairs:
 *   (NVFP4, NONE)      W4A16: bf16 x, f32 intermediate h
 *   (MXFP4, NONE)      W4A16 with MX weights
 *   (NVFP4, NVFP4)     W4A4: x and h dynamically quantized with tensor scale
 *                      amax/2688 over all of x [T, H] and all of h [T*k, I]
 *                      and amax/6 block scales (unless input_scale /
 *                      inter_scale give static tensor scales)
 *   (MXFP4, MXFP8)     MXFP4 weights x dynamic MXFP8 activations
 *   (FP8_BLOCK, FP8_ROW) block-FP8 weights x dynamic per-(row,128) FP8 activations
 * Optional shared expert (shared_inter > 0): MXFP8 Ws13 [2*Si, H] and Ws2
 * [H, Si] with dynamic MXFP8 activations, scaled per token by
 * sigmoid(x . shared_gate) (bf16 gate [H] on unquantized x) and added to y
 * ("FP4-Local AZ", section "The shared expert" and its table of differences).
 */
typedef struct {
  int32_t w_fmt, a_fmt;
  int32_t num_experts, hidden, inter, top_k;
  const uint8_t* w13;
  const void* w13_scale;
  const float* w13_scale_2; /* NVFP4: [E] */
  const uint8_t* w2;
  const void* w2_scale;
  const float* w2_scale_2;  /* NVFP4: [E] */
  const float* input_scale; /* NVFP4 activations: optional static S_x (device f32[1]) */
  const float* inter_scale; /* NVFP4 activations: optional static S_h (device f32[1]) */
  int32_t shared_inter;     /* 0: no shared expert */
  const uint8_t* ws13;      /* MXFP8 codes [2*Si, H] */
  const uint8_t* ws13_scale;/* UE8M0 [2*Si, H/32] */
  const uint8_t* ws2;       /* MXFP8 codes [H, Si] */
  const uint8_t* ws2_scale; /* UE8M0 [H, Si/32] */
  const uint16_t* shared_gate; /* bf16 [H] */
  /* Optional (may be NULL): W13 / W2 in the tiled order of
   * moe_fp4_tile_weights, with (NVFP4, MXFP4) their tiled scales; block FP8
   * keeps its 128 x 128 block scales in w13_scale / w2_scale and takes no
   * tiled scales.  The grouped GEMMs of the quantized-activation paths read
   * the tiled copies where their kernels take that order (NVFP4: always;
   * MXFP4 gate_up: always, down: inter = 640, the model's width; block FP8:
   * gate_up at hidden = 2560, down at inter = 640) and the row-major
   * tensors elsewhere; the decode GEMVs read the row-major tensors, which
   * stay required. */
  const uint8_t* w13_tiled;
  const uint8_t* w13_scale_tiled;
  const uint8_t* w2_tiled;
  const uint8_t* w2_scale_tiled;
} moe_fp4_layer;

/* Byte offsets of the stage buffers inside the forward's workspace, for
 * inspection by tests (written by moe_fp4_forward, except h on the MXFP4 x
 * MXFP8 grouped path with inter a multiple of 128, and on the block-FP8 path
 * where its gate_up GEMM takes 128-output tiles (tiled W13, hidden 2560, at
 * least 16 workgroups per CU): there h leaves the gate_up GEMM already
 * quantized and only hq_codes / hq_scales hold it). */
typedef struct {
  size_t total;          /* required workspace bytes                              */
  size_t error_flag;     /* int32: nonzero if a topk id was out of range (the next
                            int32 is the permutation's own arrival counter)      */
  size_t counts;         /* int32 [E]   pairs per expert                           */
  size_t offsets;        /* int32 [E+1] first sorted row of each expert            */
  size_t pair_of_row;    /* int32 [T*k] pair (t*k + j) held by each sorted row      */
  size_t row_of_pair;    /* int32 [T*k] sorted row of each pair                     */
  size_t x_tensor_scale; /* f32: S_x (NVFP4 activations)                            */
  size_t h_tensor_scale; /* f32: S_h (NVFP4 activations)                            */
  size_t h;              /* f32 [T*k, I]  SiLU(gate)*up in sorted row order (rows of
                            skipped pairs, sorted last, unspecified)             */
  size_t hq_codes;       /* quantized h codes (layout of a_fmt), sorted row order    */
  size_t hq_scales;      /* quantized h scales                                       */
  size_t o;              /* [T*k, H] down projection per sorted row (unweighted):
                            f32 on the GEMV paths (bf16 or MXFP8 activations at
                            decode sizes); fp16, rounded to nearest even from the
                            f32 accumulator, in the first half of this region on
                            the grouped MFMA path                                */
} moe_fp4_ws_layout;

int moe_fp4_workspace_layout(const moe_fp4_layer* layer, int64_t tokens,
                             moe_fp4_ws_layout* out);
int moe_fp4_workspace_size(const moe_fp4_layer* layer, int64_t tokens,
                           size_t* bytes);

/*
 * moe_fp4_forward - y[T, H] (f32) = routed-expert FFN of x[T, H] (bf16).
 *  topk_ids     int32 [T, k], expert of each (token, slot); 0 <= id < E.  A pair
 *               with an id out of range is skipped and sets the workspace error
 *               flag (checked by the caller after synchronising).
 *  topk_weights f32 [T, k], routing weights, applied after the down projection.
 *  workspace    >= moe_fp4_workspace_size bytes of device memory.
 * Routing (softmax / top-k) is done by the caller.
 * Precision: f32 accumulation throughout.  With quantized activations (the
 * grouped MFMA path) each pair's unweighted down output is held in fp16
 * between the down GEMM and the combine: a layer whose |o| can exceed 65504
 * gets inf in y there.
 * Shape errors (FP4_ERR_SHAPE): hidden or inter not a multiple of 32 (128 for
 * the quantized-activation pairs and block FP8; shared width a multiple of
 * 128).  FP4_ERR_UNSUPPORTED: k > 32, E > 8192, or, for weight-only layers,
 * hidden > 4096 or inter > 1024 (the decode GEMVs hold a row pair's codes in
 * registers).
 */
int moe_fp4_forward(const moe_fp4_layer* layer, const uint16_t* x, int64_t tokens,
                    const int32_t* topk_ids, const float* topk_weights, float* y,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_fp4_route - top-k routing of `tokens` tokens over E experts, on the GPU:
 * the caller-side step in front of moe_fp4_forward.  The routing width k is a
 * runtime value (FP4-Local-AZ card, "What is different from NVIDIA's
 * checkpoint": 10 or 5 routed experts per token, read from the configuration).
 *  logits       f32 [tokens, E], router logits (finite).
 *  bias         f32 [E] per-expert bias added to the logits, or NULL.
 *  topk_ids     out int32 [tokens, k]: the experts of the k largest
 *               l' = fp32(logit + bias), largest first; equal values keep the
 *               lower expert id first.
 *  topk_weights out f32 [tokens, k]: softmax over the k selected l'
 *               (renormalized top-k), computed in fp64 and rounded to f32.
 * Errors: k < 1, k > E or k > 32 -> FP4_ERR_INVALID_ARG; E > 1024 ->
 * FP4_ERR_UNSUPPORTED; tokens == 0 is a no-op.  Stream-ordered, asynchronous.
 */
int moe_fp4_route(const float* logits, const float* bias, int64_t tokens, int num_experts,
                  int top_k, int32_t* topk_ids, float* topk_weights, void* stream);

/*
 * moe_fp4_tile_weights - copy of stacked expert weights in the layout of
 * fp4_quantize, NVFP4 (codes [E, rows, cols/2], E4M3 scales [E, rows,
 * cols/16]), MXFP4 (codes [E, rows, cols/2], UE8M0 scales [E, rows, cols/32])
 * or block FP8 (E4M3 codes [E, rows, cols]; its block scales need no copy:
 * scales / tiled_scales are ignored and may be NULL), into the order the
 * grouped GEMMs stream them: per expert, per group of 16 rows, per 128-wide
 * K step, the 16 rows' code bytes as PH kilobytes of 64 bytes per row (PH = 1
 * for E2M1; 2 for E4M3, bytes 0-63 of each row then 64-127), and the 16
 * rows' SB scale bytes of the step (SB = 8 for NVFP4, 4 for MXFP4):
 *   tiled_codes [E][rows/16][cols/128][PH][16][64]
 *   tiled_scales[E][rows/16][cols/128][16][SB]
 * The same bytes, rearranged, so that one load instruction of the GEMM moves
 * one contiguous kilobyte instead of sixteen 64-byte pieces of different
 * rows.  Done once when a layer is loaded; the output buffers (same sizes as
 * the inputs, device memory, caller-owned) go in moe_fp4_layer.w13_tiled /
 * w13_scale_tiled (or w2_tiled / w2_scale_tiled).  Errors: other formats ->
 * FP4_ERR_UNSUPPORTED; rows % 16 or cols % 128 -> FP4_ERR_SHAPE; a null or
 * misaligned pointer (codes 16 bytes, scales SB) -> FP4_ERR_INVALID_ARG.
 * Stream-ordered, asynchronous.
 */
int moe_fp4_tile_weights(int w_fmt, const uint8_t* codes, const uint8_t* scales, int64_t experts,
                         int64_t rows, int64_t cols, uint8_t* tiled_codes, uint8_t* tiled_scales,
                         void* stream);

/*
 * moe_fp4_forward_profiled - moe_fp4_forward that also records HIP events
 * (hipEvent_t, created by the caller) on `stream` at the stage boundaries, for
 * per-kernel timing: events[0] before the first launch, then after the
 * permutation [1], activation quantization [2], gate_up [3], quantization of
 * h [4], down [5], shared expert [6] and combine [7].  A stage that does not
 * run in the layer's mode still gets its event (zero duration).  n_events
 * must be 8.
 */
int moe_fp4_forward_profiled(const moe_fp4_layer* layer, const uint16_t* x, int64_t tokens,
                             const int32_t* topk_ids, const float* topk_weights, float* y,
                             void* workspace, size_t workspace_bytes, void* stream,
                             void* const* events, int n_events);

/*
 * moe_fp4_forward_noalloc - moe_fp4_forward for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  The same kernels in the same order, with the
 * workspace taken from a scratch array that the library holds on each device
 * (FP4_NOALLOC_SCRATCH_BYTES, kept until the process ends) and the shared
 * expert run on the caller's stream ahead of the routed experts.  The caller
 * still passes x, the routing and y, as for moe_fp4_forward.
 *  - Allocates nothing: no device memory, streams or events are created
 *    (the first call on a device looks up that device's scratch address).
 *  - A layer and token count whose workspace (moe_fp4_workspace_size)
 *    exceeds FP4_NOALLOC_SCRATCH_BYTES returns FP4_ERR_WORKSPACE before any
 *    launch; at 512 experts, hidden 2560, inter 640 and top-10 that is above
 *    about 500 tokens.
 *  - Every call on a device shares that device's scratch, which keeps the
 *    last call's contents; no call reads what an earlier one left (every
 *    buffer is written before it is read).  Calls on one stream are ordered;
 *    calls that overlap on one device (several streams or host threads)
 *    race on the scratch and give undefined results.
 *  - The out-of-range-id flag of the workspace is not readable here: ids
 *    must lie in [0, E).
 */
#define FP4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_fp4_forward_noalloc(const moe_fp4_layer* layer, const uint16_t* x, int64_t tokens,
                            const int32_t* topk_ids, const float* topk_weights, float* y, void* stream);

const char* fp4_status_string(int status);
const char* fp4_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FP4MOE_H */
