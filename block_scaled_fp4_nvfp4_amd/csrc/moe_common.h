// Shared pieces of the MoE forward: workspace layout, decoders of packed
// weights into MFMA / dot-product operands.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4_device.h"

namespace fp4 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// 8 E2M1 nibbles (one dword, element i in bits 4i..4i+3) -> 8 bf16 values as
// 4 packed pairs, using v_perm_b32 as an 8-entry byte table.  The pairs come
// out as (e0,e2), (e4,e6), (e1,e3), (e5,e7); the activations they multiply are
// permuted the same way (permute_pairs_like_e2m1).
// bf16 of the magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6: high bytes 00 3F 3F 3F 40
// 40 40 40, low bytes 00 00 80 C0 00 40 80 C0.
__device__ __forceinline__ void e2m1x8_to_bf16x8(uint32_t d, uint32_t (&p)[4]) {
  const uint32_t hi_lo = 0x3F3F3F00u, hi_hi = 0x40404040u;
  const uint32_t lo_lo = 0xC0800000u, lo_hi = 0xC0804000u;
  uint32_t ev = d & 0x07070707u;          // magnitudes of elements 0,2,4,6 (one per byte)
  uint32_t od = (d >> 4) & 0x07070707u;   // magnitudes of elements 1,3,5,7
  uint32_t ev_lo = __builtin_amdgcn_perm(lo_hi, lo_lo, ev);
  uint32_t ev_hi = __builtin_amdgcn_perm(hi_hi, hi_lo, ev) | ((d << 4) & 0x80808080u);
  uint32_t od_lo = __builtin_amdgcn_perm(lo_hi, lo_lo, od);
  uint32_t od_hi = __builtin_amdgcn_perm(hi_hi, hi_lo, od) | (d & 0x80808080u);
  // bytes of ev_lo are selectors 0..3, bytes of ev_hi selectors 4..7
  p[0] = __builtin_amdgcn_perm(ev_hi, ev_lo, 0x05010400u);  // (e0, e2)
  p[1] = __builtin_amdgcn_perm(ev_hi, ev_lo, 0x07030602u);  // (e4, e6)
  p[2] = __builtin_amdgcn_perm(od_hi, od_lo, 0x05010400u);  // (e1, e3)
  p[3] = __builtin_amdgcn_perm(od_hi, od_lo, 0x07030602u);  // (e5, e7)
}

// 8 bf16 activations given as 4 natural pairs (x0,x1),(x2,x3),(x4,x5),(x6,x7)
// -> the pair order of e2m1x8_to_bf16x8: (x0,x2),(x4,x6),(x1,x3),(x5,x7).
__device__ __forceinline__ void permute_pairs_like_e2m1(const uint32_t (&n)[4], uint32_t (&p)[4]) {
  p[0] = __builtin_amdgcn_perm(n[1], n[0], 0x05040100u);  // x0 | x2
  p[1] = __builtin_amdgcn_perm(n[3], n[2], 0x05040100u);  // x4 | x6
  p[2] = __builtin_amdgcn_perm(n[1], n[0], 0x07060302u);  // x1 | x3
  p[3] = __builtin_amdgcn_perm(n[3], n[2], 0x07060302u);  // x5 | x7
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

}  // namespace fp4
