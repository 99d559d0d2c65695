// Device helpers for the E2M1 / E4M3 / UE8M0 formats (gfx950).
//
// NVFP4 = E2M1 values, an E4M3 scale per 16 values and an FP32 tensor scale
// (dabsLabs NVFP4 card, "What makes this build different"; Local-Hessian NVFP4
// card, opening section); MXFP4 = E2M1 with a UE8M0 scale per 32
// (MXFP4-FP8-R12 card, "Quantization format"); MXFP8 = E4M3 values with a
// power-of-two scale per 32 (FP4-Local AZ card, "The shared expert").
//
// Every rounding decision here is exact: scales are rounded from float64
// quotients that cannot sit within float64 rounding error of an E4M3 decision
// point unless they are exactly on it, and E2M1 codes are decided by comparing
// |x| with float32 thresholds rounded in the direction that keeps each
// comparison exact (see e2m1_thresholds).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4 {

constexpr float kE4M3Max = 448.0f;
constexpr double kNvTensorDivisor = 2688.0;  // E2M1 max 6 times E4M3 max 448

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// float32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// E4M3 (FN) byte -> float; 0x7F/0xFF never occur in scales written here.
// Branch-free: the subnormal form is selected, not branched to.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float nor = __uint_as_float(((e + 120u) << 23) | (m << 20));
  const float sub = (float)m * 0.001953125f;  // m * 2^-9
  const float mag = e ? nor : sub;
  return __uint_as_float(__float_as_uint(mag) | ((c & 0x80u) << 24));
}

// E4M3 code of the exact quotient Q = a / (M S) (a >= 0; M = 4 or 6; S a
// float in [2^-100, 2^100]), round to nearest even, saturating at 448, given
// any q within 2^-10 of Q relatively.  Rounding q's bit pattern to a multiple
// of 2^19 gives the 5-significant-bit value nearest q: either an E4M3 value
// (then Q rounds to it) or the midpoint of two adjacent E4M3 values c, c+1
// (then Q lies between them and the sign of a - (M mid) S, exact in one fma
// since M mid has at most 7 significant bits, picks the side; a tie picks the
// even code).  Returns 0xFF when q is in the subnormal range (0, 2^-6), which
// the caller settles exactly.
__device__ __forceinline__ uint32_t e4m3_of_quotient(float a, float q, float M, float S) {
  const uint32_t midb = (__float_as_uint(q) + 0x40000u) & 0xFFF80000u;
  uint32_t c = (((midb >> 23) - 120u) << 3) | ((midb >> 20) & 7u);
  const float d = fmaf(-(M * __uint_as_float(midb & 0x7FFFFFFFu)), S, a);
  const bool is_mid = (midb & 0x80000u) != 0u;
  c += (uint32_t)(is_mid && (d > 0.0f || (d == 0.0f && (c & 1u))));
  c = q >= 448.0f ? 0x7Eu : c;
  c = q < 0x1p-6f ? 0xFFu : c;
  return q == 0.0f ? 0u : c;
}

// E2M1 magnitude code (0..7) -> float: 0, .5, 1, 1.5, 2, 3, 4, 6
__device__ __forceinline__ float e2m1_mag_to_f32(uint32_t c) {
  return c >= 2 ? __uint_as_float((c + 252u) << 22) : 0.5f * (float)c;
}

// UE8M0 byte -> 2^(c-127) as double (exact for c in 0..254)
__device__ __forceinline__ double ue8m0_to_f64(uint32_t c) {
  return ldexp(1.0, (int)c - 127);
}

// Round a non-negative double to the nearest E4M3 code, ties to even,
// saturating at 448 (0x7E).  Exact for any double input.
__device__ __forceinline__ uint32_t e4m3_rne_sat_f64(double q) {
  if (!(q > 0.0)) return 0u;
  if (q >= 448.0) return 0x7Eu;
  int e;
  (void)frexp(q, &e);           // q in [2^(e-1), 2^e)
  int E = e - 1;                // unbiased exponent of q
  if (E < -6) {                 // subnormal range: quantum 2^-9; code = n (n == 8 is 2^-6)
    double n = rint(ldexp(q, 9));
    return (uint32_t)n;
  }
  double n = rint(ldexp(q, 3 - E));  // in [8, 16]
  uint32_t code = ((uint32_t)(E + 7) << 3) + ((uint32_t)n - 8u);
  return code > 0x7Eu ? 0x7Eu : code;
}

// Round a non-negative float to the nearest E4M3 code (ties to even,
// saturating).  Exact: the scalings are by powers of two.
__device__ __forceinline__ uint32_t e4m3_rne_sat_f32(float v) {
  if (!(v > 0.0f)) return 0u;
  if (v >= 448.0f) return 0x7Eu;
  int E = (int)((__float_as_uint(v) >> 23) & 0xFF) - 127;
  if (E < -6) return (uint32_t)rintf(ldexpf(v, 9));
  float n = rintf(ldexpf(v, 3 - E));
  uint32_t code = ((uint32_t)(E + 7) << 3) + ((uint32_t)n - 8u);
  return code > 0x7Eu ? 0x7Eu : code;
}

// E4M3 code of a non-negative float q <= 448 by the hardware convert
// (round to nearest even; the bit-exact tests pin it against exact rounding,
// subnormal codes and ties included).
__device__ __forceinline__ uint32_t e4m3_hw(float q) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q, 0.0f, 0, false) & 0xFFu;
}

// Largest float <= T and smallest float >= T, for a non-negative double T.
__device__ __forceinline__ float f32_round_down(double T) {
  const float f = (float)T;
  return __uint_as_float(__float_as_uint(f) - (uint32_t)((double)f > T));
}
__device__ __forceinline__ float f32_round_up(double T) {
  const float f = (float)T;
  return __uint_as_float(__float_as_uint(f) + (uint32_t)((double)f < T));
}

// Thresholds deciding the E2M1 code of |x| / unit.  The E2M1 midpoints are
// 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5; at a tie the even code wins, so the
// magnitude code is
//   sum_{j even} [|x| > mid_j*unit] + sum_{j odd} [|x| >= mid_j*unit].
// mid_j*unit is exact in double (<= 3 + 28 significant bits); for a float
// |x|, "|x| > T" equals "|x| > round_down(T)" and "|x| >= T" equals
// "|x| >= round_up(T)", so float comparisons decide exactly.  unit == 0
// gives thresholds of +inf (all codes 0).
struct E2M1Thresholds {
  float t[7];
};

__device__ __forceinline__ E2M1Thresholds e2m1_thresholds(double unit) {
  E2M1Thresholds th;
  const double mids[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  // computed for every unit and then raised to +inf when unit == 0 (a max,
  // not a branch: the compiler would otherwise branch around each threshold)
  const bool pos = unit > 0.0;
  const double u = pos ? unit : 1.0;
  const float floor_t = pos ? 0.0f : __builtin_inff();
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    const double T = mids[j] * u;
    const float t = (j & 1) ? f32_round_up(T) : f32_round_down(T);
    th.t[j] = fmaxf(t, floor_t);
  }
  return th;
}

// The count above is monotone in the thresholds, so it is found by a
// three-level binary search (three exact comparisons instead of seven).
// Thresholds are chosen by bit selects on all-ones / all-zero masks, so the
// search compiles to straight-line code.
__device__ __forceinline__ float bitsel(uint32_t mask, float if_set, float if_clear) {
  return __uint_as_float((__float_as_uint(if_set) & mask) | (__float_as_uint(if_clear) & ~mask));
}
__device__ __forceinline__ uint32_t e2m1_code(float a, const E2M1Thresholds& th) {
  const uint32_t m3 = 0u - (uint32_t)(a >= th.t[3]);
  const uint32_t mm = 0u - (uint32_t)(a >= bitsel(m3, th.t[5], th.t[1]));
  const float tl = bitsel(m3, bitsel(mm, th.t[6], th.t[4]), bitsel(mm, th.t[2], th.t[0]));
  return (m3 & 4u) | (mm & 2u) | (uint32_t)(a > tl);
}

// Eight magnitude codes (nibble i = code of element i, sign bits clear) ->
// their E2M1 values, through the hardware convert (exact with scale 1.0).
__device__ __forceinline__ void e2m1x8_mags(uint32_t d, float (&g)[8]) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
  const f2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
  const f2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
  const f2 e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
  g[0] = a.x; g[1] = a.y; g[2] = b.x; g[3] = b.y;
  g[4] = c.x; g[5] = c.y; g[6] = e.x; g[7] = e.y;
}

// Smallest e with M * 2^e >= a (a > 0 finite), M in {4, 6, 448}, clamped to
// [-127, 127]; a == 0 gives -127.  Exact integer logic on frexp.
__device__ __forceinline__ int mx_exponent(float a, float M) {
  if (!(a > 0.0f)) return -127;
  int p;
  float f = frexpf(a, &p);     // a = f * 2^p, f in [0.5, 1)
  int pm;
  float fm = frexpf(M, &pm);   // M = fm * 2^pm
  // M * 2^e >= a  <=>  fm * 2^(pm+e) >= f * 2^p
  int e = (fm >= f) ? (p - pm) : (p - pm + 1);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Exact E4M3 code (saturating) of a / sigma for a >= 0, sigma > 0 floats.
// The float quotient q = RN(a / sigma) rounds to the same code as the exact
// quotient unless q lands exactly on an E4M3 midpoint (RN is monotone and
// every midpoint is a float); only then is a compared with midpoint * sigma,
// exactly in double (5 + 24 significant bits), to pick the side.
__device__ __forceinline__ bool e4m3_is_midpoint(float q) {
  const bool normal_mid = (__float_as_uint(q) & 0x000FFFFFu) == 0x00080000u;  // half of the 3-bit ulp
  const float t = q * 1024.0f;  // subnormal quantum 2^-9: midpoints are odd multiples of 2^-10
  const bool sub_mid = (t == rintf(t)) & (((int)t & 1) != 0);
  return q >= 0.015625f ? normal_mid : sub_mid;
}
__device__ __forceinline__ uint32_t e4m3_fix_midpoint(uint32_t c, float q, float a, float sigma) {
  const double A = (double)a, M = (double)q * (double)sigma;
  const float vc = __builtin_amdgcn_cvt_f32_fp8((int)c, 0);
  if (A > M && vc < q) return c + 1;
  if (A < M && vc > q) return c - 1;
  return c;
}
__device__ __forceinline__ uint32_t e4m3_exact_quotient(float a, float sigma) {
  const float q = fminf(a / sigma, kE4M3Max);
  const uint32_t c = e4m3_hw(q);
  return e4m3_is_midpoint(q) ? e4m3_fix_midpoint(c, q, a, sigma) : c;
}

}  // namespace fp4
