/*
 * fp4moe_probe.h - device-ceiling microbenchmarks of libfp4moe.so (gfx950).
 *
 * The rooflines of the library's kernels are stated against the vendor peaks
 * (HBM 8 TB/s; dense MFMA 2.5 PFLOP/s fp16 / bf16, 5.0 fp8, 10.1 fp4) and
 * against what the device delivers to a plain kernel; these calls measure the
 * latter.  They do the measured work only: the caller times them (HIP events
 * on `stream`) and owns every buffer (device pointers).  Errors: negative
 * fp4_status values, as in fp4moe.h.
 */
#ifndef FP4MOE_PROBE_H
#define FP4MOE_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` (a multiple of 16; src 16-byte aligned) by `grid`
 * workgroups of 256 threads, 16-byte loads, four in flight per thread per
 * step.  sink: one uint32 that is written only in the (practically never
 * met) case that the XOR of everything read equals a fixed constant. */
int fp4_probe_read(const void* src, size_t bytes, int grid, uint32_t* sink, void* stream);

enum {
  FP4_PROBE_MFMA_F16 = 0,     /* v_mfma_f32_16x16x32_f16: 16384 FLOPs per instruction  */
  FP4_PROBE_MFMA_BF16 = 1,    /* v_mfma_f32_16x16x32_bf16: 16384                         */
  FP4_PROBE_MFMA_FP8_FP8 = 2, /* v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 x E4M3: 65536   */
  FP4_PROBE_MFMA_FP8_FP4 = 3, /* the same, E4M3 x E2M1: 65536                             */
  FP4_PROBE_MFMA_FP4_FP4 = 4, /* the same, E2M1 x E2M1: 65536                             */
  FP4_PROBE_MFMA_F16_32 = 5,  /* v_mfma_f32_32x32x16_f16: 32768                            */
  FP4_PROBE_MFMA_FP8_32 = 6,  /* v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 x E4M3: 131072    */
  FP4_PROBE_MFMA_FP4_32 = 7   /* the same, E2M1 x E2M1: 131072                            */
};

/* MFMA issue rate: `grid` workgroups of 4 waves, each wave `iters` rounds of
 * 8 independent MFMAs of `kind`; out: f32 [grid * 256 * 4] (the accumulators,
 * so the work is kept).  FLOPs = grid * 4 * iters * 8 * (FLOPs per instruction).
 * clocks: null, or uint64 [128] receiving, for workgroups b < min(grid, 64),
 * the shader-clock cycles (clocks[2 b]) and 100 MHz constant-clock ticks
 * (clocks[2 b + 1]) that the workgroup's first wave spent in its MFMA loop;
 * 0.1 GHz * cycles / ticks is the shader clock under that load. */
int fp4_probe_mfma(int kind, int iters, int grid, float* out, uint64_t* clocks, void* stream);

enum {
  FP4_PROBE_STORE_O = 0,  /* the down GEMM's epilogue stores o [T*k, H] (f32)                   */
  FP4_PROBE_COMBINE = 1,  /* y[t] = sum_j w[t, j] o[row(t, j)] (the library's combine pattern)  */
  FP4_PROBE_ATOMIC_Y = 2  /* the same epilogue adds w * o into y [T, H] with fp32 atomics       */
};

/* The routing-weighted combine two ways, for T tokens, top-k, hidden H
 * (a multiple of 128): pair_of_row / row_of_pair int32 [T*k] (sorted rows
 * by expert, as the forward's permutation), w f32 [T*k]; o f32 [T*k, H],
 * y f32 [T, H] (zero it before FP4_PROBE_ATOMIC_Y).  The epilogue writes a
 * fixed function of (row, column) as its value. */
int fp4_probe_combine(int mode, const int32_t* pair_of_row, const int32_t* row_of_pair, const float* w,
                      int64_t tokens, int top_k, int hidden, float* o, float* y, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FP4MOE_PROBE_H */
