// Grouped MFMA GEMMs of the MoE forward (quantized activations) and the
// shared expert.
#include <hip/hip_runtime.h>

#include "host_common.h"
#include "moe_internal.h"

namespace fp4 {

int launch_grouped(const moe_fp4_layer* L, const uint16_t* x, int64_t T, const WsPtrs& w,
                   int max_active, hipStream_t st) {
  (void)L; (void)x; (void)T; (void)w; (void)max_active; (void)st;
  return fail(FP4_ERR_UNSUPPORTED, "quantized-activation path not built yet");
}

int launch_shared_expert(const moe_fp4_layer* L, const uint16_t* x, int64_t T, const WsPtrs& w,
                         hipStream_t st) {
  (void)L; (void)x; (void)T; (void)w; (void)st;
  return fail(FP4_ERR_UNSUPPORTED, "shared expert not built yet");
}

}  // namespace fp4
