// Shared pieces of the MoE forward: workspace layout, decoders of packed
// weights into MFMA / dot-product operands.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4_device.h"

namespace fp4 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-byte loads and stores through native vector types (a struct-of-uint
// array of such values would be demoted to scratch memory).
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// 8 E2M1 nibbles (one dword, element i in bits 4i..4i+3) -> 8 bf16 values
// as 4 packed pairs (e0,e1), (e2,e3), (e4,e5), (e6,e7).  The gfx950 scaled
// convert takes byte `sel` of the dword, low nibble first; with scale 1.0 it
// is exact (every E2M1 value is a bf16 value).
__device__ __forceinline__ void e2m1x8_to_bf16x8(uint32_t d, uint32_t (&p)[4]) {
  p[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 0));
  p[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 1));
  p[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 2));
  p[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 3));
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// 8 E2M1 nibbles -> 8 floats in element order (same convert, f32 result).
__device__ __forceinline__ void e2m1x8_to_f32x8(uint32_t d, float (&f)[8]) {
  f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
  f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
  f32x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
  f32x2_t e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
  f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y;
  f[4] = c.x; f[5] = c.y; f[6] = e.x; f[7] = e.y;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8): vmcnt <= n only, and vmcnt <= n with lgkmcnt = 0.
constexpr int vmcnt_only(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int vmcnt_lgkm0(int n) { return (n & 15) | (7 << 4) | ((n >> 4) << 14); }

// SiLU(g) = g / (1 + e^-g), as g times the hardware reciprocal (about 1 ulp)
// of 1 + e^-g: two VALU instructions where the IEEE divide takes about ten,
// in epilogues that evaluate it 32 times per lane.  g very negative gives
// 1 + e^-g = inf and a signed zero, as the divide does.
__device__ __forceinline__ float silu_f32(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

}  // namespace fp4
