// Host-side helpers of the C ABI: status codes, the thread-local error text,
// launch checking.
#pragma once
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/fp4moe.h"

namespace fp4 {

void set_last_error(const char* fmt, ...);

inline int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  set_last_error("%s: %s", fp4_status_string(status), buf);
  return status;
}

inline int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(FP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return FP4_OK;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// While alive, this thread's stream-capture mode is relaxed, so the one-time
// per-device set-up calls (raising a kernel's dynamic-LDS limit, creating
// the shared expert's helper stream and events) are allowed even when the
// first forward on a device is issued inside a graph capture.
struct RelaxedCapture {
  hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
  bool ok;
  RelaxedCapture() { ok = hipThreadExchangeStreamCaptureMode(&mode) == hipSuccess; }
  ~RelaxedCapture() {
    if (ok) (void)hipThreadExchangeStreamCaptureMode(&mode);
  }
};

inline unsigned grid_1d(int64_t n, int threads) {
  return (unsigned)((n + threads - 1) / threads);
}

// number of compute units of the current device (cached per device id)
int device_cu_count();

// MXFP8 quantization of rows x cols (bf16 -> bf16 or f32 -> f32) that also
// writes the exact values of the codes to `deq` (the layout of the input)
int mxfp8_quantize_dequant(const void* x, int x_dtype, int64_t rows, int64_t cols, uint8_t* codes,
                           uint8_t* scales, void* deq, int deq_dtype, hipStream_t st);

// NVFP4 tensor scales tensor_scale[b] = fp32(fp64(amax_b) / 2688) of `batch`
// tensors of `per` values each (bf16 or f32 x)
int nv_tensor_scales(const void* x, int x_dtype, int64_t batch, int64_t per, float* tensor_scale,
                     hipStream_t st);

// NVFP4 tensor scale s[0] = fp32(fp64(amax) / 2688) of one tensor whose amax
// is the max of nparts non-negative partial maxima at part (device)
int nv_tensor_scale_from_parts(const float* part, int64_t nparts, float* s, hipStream_t st);

}  // namespace fp4

#define FP4_CHECK(expr)                  \
  do {                                   \
    int _st = (expr);                    \
    if (_st != FP4_OK) return _st;       \
  } while (0)
