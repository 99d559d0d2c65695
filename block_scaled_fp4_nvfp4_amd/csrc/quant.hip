// Quantizers and dequantizers behind fp4_quantize / fp4_dequantize (gfx950).
//
// NVFP4 with the 4/6 block-scale choice (dabsLabs NVFP4 card, "What makes
// this build different"), tensor scale amax/2688 shared by a fused gate_up
// (Local-Hessian NVFP4 card, opening section), MXFP4 (MXFP4-FP8-R12 card,
// "Quantization format"), MXFP8 (FP4-Local AZ card, "The shared expert") and
// block FP8 (MXFP4-FP8-R12 card, runtime contract table).
//
// The 4/6 choice needs, per block and plan M, the exact error
//   err_M = sum (|x_i| - g_i s_M S)^2 = sum x_i^2 - 2 s_M S GX_M + s_M^2 S^2 G2_M
// with G2_M = sum g_i^2 and GX_M = sum g_i |x_i| (g the E2M1 magnitudes).  So
//   err_6 - err_4 = S * (S * A - 2 * B),
//   A = s6^2 G2_6 - s4^2 G2_4,  B = s6 GX_6 - s4 GX_4,
// and M=4 wins iff S*A - 2*B > 0.  G2 is a multiple of 1/4 below 2^12; for bf16
// inputs every g|x| has <= 10 significant bits and the nonzero ones span
// fewer than 21 bits, so GX is exact in float; A, B and S*A are exact in
// double and the one rounding of S*A - 2*B cannot change its sign.  For f32
// inputs GX is accumulated in double (exact for the same reason, 24+2 bits).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <type_traits>

#include "fp4_device.h"
#include "host_common.h"

#pragma clang fp contract(off)

namespace fp4 {

static thread_local std::string g_last_error;

void set_last_error(const char* fmt, ...) {
  char buf[768];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

int device_cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// ------------------------------------------------------------ element loads

template <int N>
__device__ __forceinline__ void load_vals(const uint16_t* p, float (&v)[N]) {
  static_assert(N % 8 == 0, "");
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < N / 8; ++i) {
    uint4 w = q[i];
    uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = __uint_as_float(d[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(d[j] & 0xFFFF0000u);
    }
  }
}

template <int N>
__device__ __forceinline__ void load_vals(const float* p, float (&v)[N]) {
  static_assert(N % 4 == 0, "");
  const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    float4 w = q[i];
    v[4 * i] = w.x;
    v[4 * i + 1] = w.y;
    v[4 * i + 2] = w.z;
    v[4 * i + 3] = w.w;
  }
}

__device__ __forceinline__ float load_val(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ __forceinline__ float load_val(const float* p) { return *p; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// ------------------------------------------------------------------ kernels

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// amax of each tensor (batch item) as float bits, combined with atomicMax on
// the bit pattern (non-negative floats order like their bit patterns).  Each
// workgroup reduces in LDS first, so a tensor receives one atomic per
// workgroup (a few per CU) rather than one per wave.
template <typename T>
__global__ void __launch_bounds__(256) tensor_amax_kernel(const T* x, int64_t per_tensor,
                                                          uint32_t* amax_bits) {
  const T* base = x + (int64_t)blockIdx.y * per_tensor;
  float m = 0.0f;
  int64_t stride = (int64_t)gridDim.x * 256 * 8;
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; i < per_tensor; i += stride) {
    float v[8];
    load_vals<8>(base + i, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
  }
  m = wave_max(m);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (a > 0.0f) atomicMax(amax_bits + blockIdx.y, __float_as_uint(a));
  }
}

// Partial maxima of |x| over one tensor of n values (n % 8 == 0): workgroup b
// writes the max over its share to part[b].  Each lane keeps four 8-value
// loads in flight.
template <typename T>
__global__ void __launch_bounds__(256) amax_parts_kernel(const T* __restrict__ x, int64_t n,
                                                         float* __restrict__ part) {
  const int64_t S = (int64_t)gridDim.x * 256 * 8;
  float m = 0.0f;
  int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  for (; i + 3 * S < n; i += 4 * S) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load_vals<8>(x + i + u * S, v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[u][j]));
  }
  for (; i < n; i += S) {
    float v[8];
    load_vals<8>(x + i, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
  }
  m = wave_max(m);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// S = fp32(fp64(amax) / 2688) of tensor y from its nparts partial maxima at
// part + y * stride; one workgroup per tensor.
__global__ void __launch_bounds__(256) nv_scale_from_parts_kernel(const float* __restrict__ part, int64_t stride,
                                                                  int nparts, float* __restrict__ s) {
  const float* p = part + (int64_t)blockIdx.x * stride;
  float m = 0.0f;
  int i = threadIdx.x;
  for (; i + 3 * 256 < nparts; i += 4 * 256) {  // four loads in flight per lane
    const float a = p[i], b = p[i + 256], c = p[i + 512], d = p[i + 768];
    m = fmaxf(m, fmaxf(fmaxf(a, b), fmaxf(c, d)));
  }
  for (; i < nparts; i += 256) m = fmaxf(m, p[i]);
  m = wave_max(m);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    s[blockIdx.x] = (float)((double)a / kNvTensorDivisor);
  }
}

// S = fp32(fp64(amax) / 2688), in place over the amax bits.
__global__ void nv_tensor_scale_kernel(float* s, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) s[i] = (float)((double)s[i] / kNvTensorDivisor);
}

template <typename T> struct GxAcc { using type = float; };
template <> struct GxAcc<float> { using type = double; };

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// 4 x the E2M1 midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 in 5-bit fields
constexpr uint64_t kE2M1Mid4 = 1ull | 3ull << 5 | 5ull << 10 | 7ull << 15 | 10ull << 20 | 14ull << 25 |
                               20ull << 30;

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }

// Signed E2M1 codes of eight values (nibble j <- element j) by the hardware
// convert: round to nearest, ties to even, saturating at 6, sign kept for
// values that round to zero.  The scaled forms divide by 2^(exponent of p2).
__device__ __forceinline__ uint32_t fp4x8_of_product(const float* v, float r) {
  uint32_t d = 0;
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[0] * r, v[1] * r, 1.0f, 0);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[2] * r, v[3] * r, 1.0f, 1);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[4] * r, v[5] * r, 1.0f, 2);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[6] * r, v[7] * r, 1.0f, 3);
  return d;
}
__device__ __forceinline__ uint32_t fp4x8_scaled(const float* v, float p2) {
  uint32_t d = 0;
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[0], v[1], p2, 0);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[2], v[3], p2, 1);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[4], v[5], p2, 2);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[6], v[7], p2, 3);
  return d;
}
__device__ __forceinline__ uint32_t fp4x8_scaled(const uint32_t* raw, float p2) {
  uint32_t d = 0;
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(d, as_bf16x2(raw[0]), p2, 0);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(d, as_bf16x2(raw[1]), p2, 1);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(d, as_bf16x2(raw[2]), p2, 2);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(d, as_bf16x2(raw[3]), p2, 3);
  return d;
}

// G2 += sum g^2 and GX += sum g*x over eight signed codes and their inputs
// (g and x share a sign, so g*x = g|x|).  bf16 inputs: the codes decode to
// bf16 exactly and the bf16 dot products add exact terms whose sums are
// exact in float (see the head of this file); f32 inputs: GX in double.
__device__ __forceinline__ void fp4x8_sums(uint32_t d, const uint32_t* raw, float& g2, float& gx) {
  bf16x2_t g;
  g = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 0);
  g2 = __builtin_amdgcn_fdot2_f32_bf16(g, g, g2, false);
  gx = __builtin_amdgcn_fdot2_f32_bf16(g, as_bf16x2(raw[0]), gx, false);
  g = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 1);
  g2 = __builtin_amdgcn_fdot2_f32_bf16(g, g, g2, false);
  gx = __builtin_amdgcn_fdot2_f32_bf16(g, as_bf16x2(raw[1]), gx, false);
  g = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 2);
  g2 = __builtin_amdgcn_fdot2_f32_bf16(g, g, g2, false);
  gx = __builtin_amdgcn_fdot2_f32_bf16(g, as_bf16x2(raw[2]), gx, false);
  g = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 3);
  g2 = __builtin_amdgcn_fdot2_f32_bf16(g, g, g2, false);
  gx = __builtin_amdgcn_fdot2_f32_bf16(g, as_bf16x2(raw[3]), gx, false);
}
__device__ __forceinline__ void fp4x8_sums(uint32_t d, const float* v, float& g2, double& gx) {
  float g[8];
  e2m1x8_mags(d, g);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    g2 = fmaf(g[j], g[j], g2);  // exact: a multiple of 1/4 below 2^12
    gx = fma((double)g[j], (double)v[j], gx);
  }
}

// Reference plan by exact comparisons: signed codes of x / unit (unit exact
// in double) and the plan's sums, for units outside [2^-100, 2^100] where the
// hardware-convert plan is not shown exact.
template <int BS, typename Acc>
__device__ __forceinline__ void exact_plan(const float (&v)[BS], double unit, uint32_t (&pk)[BS / 8],
                                           float& g2, Acc& gx) {
  const E2M1Thresholds th = e2m1_thresholds(unit);
  g2 = 0.0f;
  gx = 0;
#pragma unroll
  for (int w = 0; w < BS / 8; ++w) {
    uint32_t d = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) d |= e2m1_code(fabsf(v[8 * w + j]), th) << (4 * j);
    float gm[8];
    e2m1x8_mags(d, gm);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      g2 = fmaf(gm[j], gm[j], g2);
      gx += (Acc)gm[j] * (Acc)fabsf(v[8 * w + j]);
    }
    pk[w] = d | (pk[w] & 0x88888888u);  // signs of x, as the hardware codes already carry them
  }
}

// One thread per block of BS values (16: NVFP4, 32: MXFP4).
//
// NVFP4 codes: with u = s*S (s the block's E4M3 scale) and r ~ 1/u within
// 2^-23, the codes of x*r(1-2^-20) and x*r(1+2^-20) bracket the code of the
// exact quotient x/u (the rounding is monotone), so where the two agree the
// code is exact; where they differ one exact comparison decides.
// MXFP4 codes: x / 2^e is exact, so the hardware convert is exact.
template <int BS, bool MX, bool FOUR_SIX, typename T, bool SWEEP = false>
__global__ void __launch_bounds__(256) quant_fp4_kernel(
    const T* __restrict__ x, int64_t blocks_per_tensor, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, const float* __restrict__ tensor_scale,
    uint8_t* __restrict__ m4_flags, const T* __restrict__ next_x, float* __restrict__ next_part,
    int64_t part_stride, int next_tensors) {
  constexpr bool BF = std::is_same<T, uint16_t>::value;
  constexpr bool FUSE = BF && !MX;
  constexpr int NW = BS / 8;
  using Acc = typename GxAcc<T>::type;
  int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blk >= blocks_per_tensor) return;
  int64_t g = (int64_t)blockIdx.y * blocks_per_tensor + blk;
  uint32_t raw[BF ? BS / 2 : 1];
  float v[BS];
  float amax;
  // The same block of tensor blockIdx.y of the next chunk, for its tensor
  // amax: each workgroup stores its partial max at next_part[y * part_stride
  // + x] (NVFP4 from bf16 only; the host launches this only when every lane
  // of every workgroup holds a block, with next_tensors <= gridDim.y and
  // gridDim.x <= part_stride).
  const bool fuse = FUSE && (int)blockIdx.y < next_tensors;
  uint32_t nraw[FUSE ? BS / 2 : 1];
  if constexpr (BF) {
    const uint4* q = reinterpret_cast<const uint4*>(x + g * BS);
#pragma unroll
    for (int i = 0; i < BS / 8; ++i) {
      const uint4 w = q[i];
      raw[4 * i] = w.x; raw[4 * i + 1] = w.y; raw[4 * i + 2] = w.z; raw[4 * i + 3] = w.w;
    }
    if constexpr (FUSE) {
      if (fuse) {
        const uint4* nq = reinterpret_cast<const uint4*>(next_x + g * BS);
#pragma unroll
        for (int i = 0; i < BS / 8; ++i) {
          const uint4 w = nq[i];
          nraw[4 * i] = w.x; nraw[4 * i + 1] = w.y; nraw[4 * i + 2] = w.z; nraw[4 * i + 3] = w.w;
        }
      }
    }
    // |x| bit patterns order like |x|: a packed 16-bit max over the pairs
    u16x2_t m = {0, 0};
#pragma unroll
    for (int i = 0; i < BS / 2; ++i) {
      v[2 * i] = __uint_as_float(raw[i] << 16);
      v[2 * i + 1] = __uint_as_float(raw[i] & 0xFFFF0000u);
      m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, raw[i] & 0x7FFF7FFFu));
    }
    amax = __uint_as_float((uint32_t)max(m.x, m.y) << 16);
  } else {
    load_vals<BS>(x + g * BS, v);
    amax = 0.0f;
#pragma unroll
    for (int i = 0; i < BS; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }

  double S = 1.0, s6, s4 = 0.0;
  uint32_t code6, code4 = 0;
  int e6 = 0, e4 = 0;
  if (MX) {
    e6 = mx_exponent(amax, 6.0f);
    code6 = (uint32_t)(e6 + 127);
    s6 = ldexp(1.0, e6);
    if (FOUR_SIX) {
      e4 = mx_exponent(amax, 4.0f);
      code4 = (uint32_t)(e4 + 127);
      s4 = ldexp(1.0, e4);
    }
  } else {
    const float Sf = tensor_scale[blockIdx.y];
    S = (double)Sf;
    const bool s_ok = Sf >= 0x1p-100f && Sf <= 0x1p100f;
    const float R6 = s_ok ? __builtin_amdgcn_rcpf(6.0f * Sf) : 0.0f;  // ~1/(6S) within 2^-21
    code6 = e4m3_of_quotient(amax, amax * R6, 6.0f, Sf);
    if (FOUR_SIX) code4 = e4m3_of_quotient(amax, amax * (1.5f * R6), 4.0f, Sf);
    if (!s_ok || code6 == 0xFFu || code4 == 0xFFu) {  // extreme S or a block in the E4M3 subnormal range
      code6 = S > 0.0 ? e4m3_rne_sat_f64((double)amax / (6.0 * S)) : 0u;
      if (FOUR_SIX) code4 = S > 0.0 ? e4m3_rne_sat_f64((double)amax / (4.0 * S)) : 0u;
    }
    s6 = (double)e4m3_to_f32(code6);
    if (FOUR_SIX) s4 = (double)e4m3_to_f32(code4);
  }

  // codes and sums of one plan (scale s, or 2^e for MX)
  auto plan = [&](double s, int e, uint32_t (&pk)[NW], float& g2, Acc& gx) __attribute__((always_inline)) {
    bool exact = true;
    if constexpr (MX) {
      exact = e >= -100 || amax == 0.0f;  // a zero block gives signed zeros either way
      const float p2 = __uint_as_float((uint32_t)(max(e, -126) + 127) << 23);
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        if constexpr (BF) pk[w] = fp4x8_scaled(&raw[4 * w], p2);
        else pk[w] = fp4x8_scaled(&v[8 * w], p2);
      }
    } else {
      const float sf = (float)s, uf = sf * (float)S;  // one rounding of the exact s*S
      const bool zero = sf == 0.0f;
      const bool in_range = uf >= 0x1p-100f && uf <= 0x1p100f;
      const float r0 = in_range ? __builtin_amdgcn_rcpf(uf) : 0.0f;
      const float r = fmaf(r0, fmaf(-uf, r0, 1.0f), r0);  // one Newton step: |r*u - 1| < 2^-23
      const float rl = r * 0x1.ffffe0p-1f, rh = r * 0x1.000010p+0f;  // r (1 -/+ 2^-20)
      uint32_t hi[NW], diff = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        pk[w] = fp4x8_of_product(&v[8 * w], rl);
        hi[w] = fp4x8_of_product(&v[8 * w], rh);
        diff |= pk[w] ^ hi[w];
      }
      exact = zero || in_range;
      // A value whose bracket straddles an E2M1 midpoint m (adjacent codes
      // k, k+1) is decided by the sign of |x| - (m s) S, which one fma gives
      // exactly (m s has at most 7 significant bits).  Such values are rare
      // but not negligible: with S = amax/2688 and 2688 = 21 * 2^7, a
      // threshold m s S with m s = 21 * 2^j sits within S's rounding error of
      // the bf16 values that share the tensor amax's significand.
      if (exact && diff) {
        const float sq = 0.25f * sf;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          uint32_t dw = pk[w] ^ hi[w];
          while (dw) {
            const uint32_t sh = (uint32_t)__builtin_ctz(dw) & ~3u;  // 4 * nibble index
            const uint32_t k = min((pk[w] >> sh) & 7u, (hi[w] >> sh) & 7u);
            const uint32_t m4 = (uint32_t)(kE2M1Mid4 >> (5u * k)) & 31u;  // 4 * midpoint(k, k+1)
            float ax;
            if constexpr (BF) {
              const uint32_t p = sh >> 3;
              const uint32_t a = (p & 1u) ? raw[4 * w + 1] : raw[4 * w];
              const uint32_t b = (p & 1u) ? raw[4 * w + 3] : raw[4 * w + 2];
              const uint32_t r2 = (p & 2u) ? b : a;
              ax = __uint_as_float(((sh & 4u) ? (r2 & 0xFFFF0000u) : (r2 << 16)) & 0x7FFFFFFFu);
            } else {
              ax = fabsf(load_val(x + g * BS + 8 * w + (sh >> 2)));
            }
            const float d = fmaf(-((float)m4 * sq), (float)S, ax);
            const uint32_t up = (uint32_t)(d > 0.0f) | ((uint32_t)(d == 0.0f) & k);
            pk[w] = (pk[w] & ~(7u << sh)) | ((k + (up & 1u)) << sh);
            dw &= ~(15u << sh);
          }
        }
      }
    }
    g2 = 0.0f;
    gx = 0;
    if constexpr (FOUR_SIX) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        if constexpr (BF) fp4x8_sums(pk[w], &raw[4 * w], g2, gx);
        else fp4x8_sums(pk[w], &v[8 * w], g2, gx);
      }
    }
    if (!exact) exact_plan<BS, Acc>(v, s * S, pk, g2, gx);
  };

  uint32_t p6[NW], p4[NW];
  float g2_6, g2_4 = 0.0f;
  Acc gx_6, gx_4 = 0;
  plan(s6, e6, p6, g2_6, gx_6);
  bool use4 = false;
  if (FOUR_SIX) {
    plan(s4, e4, p4, g2_4, gx_4);
    double A = s6 * s6 * (double)g2_6 - s4 * s4 * (double)g2_4;
    double B = s6 * (double)gx_6 - s4 * (double)gx_4;
    use4 = (S * A - 2.0 * B) > 0.0;
  }

  uint32_t packed[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) packed[w] = (FOUR_SIX && use4) ? p4[w] : p6[w];
  uint32_t code = (FOUR_SIX && use4) ? code4 : code6;
  uint32_t flag = use4 ? 1u : 0u;
  if constexpr (SWEEP) {
    // NVFP4 scale sweep: every E4M3 code strictly between the two plans'
    // against the better of those two, by the same exact identity; ties keep
    // the earlier (smaller) code, so the first minimum over the codes from
    // code6 up wins
    static_assert(!MX && FOUR_SIX, "the sweep extends the NVFP4 4/6 kernel");
    double sb = use4 ? s4 : s6;
    float g2b = use4 ? g2_4 : g2_6;
    Acc gxb = use4 ? gx_4 : gx_6;
    for (uint32_t c = code6 + 1; c < code4; ++c) {
      const double sc = (double)e4m3_to_f32(c);
      uint32_t pc[NW];
      float g2c;
      Acc gxc;
      plan(sc, 0, pc, g2c, gxc);
      const double A = sb * sb * (double)g2b - sc * sc * (double)g2c;
      const double B = sb * (double)gxb - sc * (double)gxc;
      // the best so far is code6 or an interior code (smaller than c) unless
      // it is code4, which c < code4 may tie: then c, the smaller code, wins
      const bool take = (S * A - 2.0 * B) > 0.0 || ((S * A - 2.0 * B) == 0.0 && code == code4 && use4);
      if (take) {
#pragma unroll
        for (int w = 0; w < NW; ++w) packed[w] = pc[w];
        sb = sc;
        g2b = g2c;
        gxb = gxc;
        code = c;
      }
    }
    flag = code - code6;
  }
  if (BS == 16) {
    reinterpret_cast<uint2*>(codes)[g] = make_uint2(packed[0], packed[1 % NW]);
  } else {
    reinterpret_cast<uint4*>(codes)[g] = make_uint4(packed[0], packed[1 % NW], packed[2 % NW], packed[3 % NW]);
  }
  scales[g] = (uint8_t)code;
  if (m4_flags) m4_flags[g] = (uint8_t)flag;
  if constexpr (FUSE) {
    if (fuse) {
      u16x2_t m = {0, 0};
#pragma unroll
      for (int i = 0; i < BS / 2; ++i)
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, nraw[i] & 0x7FFF7FFFu));
      const float a = wave_max(__uint_as_float((uint32_t)max(m.x, m.y) << 16));
      __shared__ float red[4];
      if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
      __syncthreads();
      if (threadIdx.x == 0)
        next_part[(int64_t)blockIdx.y * part_stride + blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    }
  }
}

// MXFP8: one thread per block of 32; e = min{e : 448 * 2^e >= amax}.
template <typename T>
__device__ __forceinline__ int mxfp8_block(const T* __restrict__ x, int64_t g, uint8_t* __restrict__ codes,
                                           uint8_t* __restrict__ scales, uint32_t (&out)[8]) {
  float v[32];
  load_vals<32>(x + g * 32, v);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int e = mx_exponent(amax, kE4M3Max);
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t d = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float a = v[4 * w + j];
      // the power-of-two scaling is exact, so the convert rounds exactly
      uint32_t c = e4m3_hw(fminf(ldexpf(fabsf(a), -e), kE4M3Max)) | ((__float_as_uint(a) >> 24) & 0x80u);
      d |= c << (8 * j);
    }
    out[w] = d;
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + g * 32);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  scales[g] = (uint8_t)(e + 127);
  return e;
}

template <typename T>
__global__ void __launch_bounds__(256) quant_mxfp8_kernel(const T* __restrict__ x, int64_t nblocks,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= nblocks) return;
  uint32_t out[8];
  (void)mxfp8_block<T>(x, g, codes, scales, out);
}

// FP8 with one fp32 scale per (row, 128 columns): 4 lanes per group of 128.
template <typename T>
__global__ void __launch_bounds__(256) quant_fp8_row_kernel(const T* __restrict__ x, int64_t ngroups,
                                                            uint8_t* __restrict__ codes,
                                                            float* __restrict__ scales) {
  int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t g = t >> 2;
  bool active = g < ngroups;
  float v[32];
  if (active) {
    load_vals<32>(x + t * 32, v);
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  if (!active) return;
  float sigma = (float)((double)amax / 448.0);
  // all 32 codes from the float quotients; the rare exact midpoints are
  // corrected in one branch taken by the whole lane at most once
  const float sg = sigma > 0.0f ? sigma : 1.0f;
  float q[32];
  uint32_t cm[32];
  bool anymid = false;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    q[i] = fminf(fabsf(v[i]) / sg, kE4M3Max);
    cm[i] = e4m3_hw(q[i]);
    anymid |= e4m3_is_midpoint(q[i]);
  }
  if (anymid) {
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if (e4m3_is_midpoint(q[i])) cm[i] = e4m3_fix_midpoint(cm[i], q[i], fabsf(v[i]), sg);
  }
  uint32_t out[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t d = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = v[4 * w + j];
      const uint32_t c = (sigma > 0.0f ? cm[4 * w + j] : 0u) | ((__float_as_uint(a) >> 24) & 0x80u);
      d |= c << (8 * j);
    }
    out[w] = d;
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + t * 32);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  if ((t & 3) == 0) scales[g] = sigma;
}

// Block FP8 weights: amax of each 128 x 128 tile (one workgroup per tile).
template <typename T>
__global__ void __launch_bounds__(256) fp8_tile_amax_kernel(const T* __restrict__ x, int64_t rows,
                                                            int64_t cols, float* __restrict__ sigma) {
  int64_t tiles_c = cols / 128, tiles_r = rows / 128;
  int64_t tile = blockIdx.x;
  int64_t b = blockIdx.y;
  int64_t tr = tile / tiles_c, tc = tile % tiles_c;
  const T* base = x + b * rows * cols + tr * 128 * cols + tc * 128;
  float m = 0.0f;
  // 256 threads: 16 threads per row (8 values each), 16 rows per pass
  int r0 = threadIdx.x >> 4, c0 = (threadIdx.x & 15) * 8;
  for (int r = r0; r < 128; r += 16) {
    float v[8];
    load_vals<8>(base + (int64_t)r * cols + c0, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
  }
  m = wave_max(m);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    sigma[b * tiles_r * tiles_c + tile] = (float)((double)a / 448.0);
  }
}

// Block FP8 weights: one thread per 32 consecutive values of a row.
template <typename T>
__global__ void __launch_bounds__(256) quant_fp8_tile_kernel(const T* __restrict__ x, int64_t rows,
                                                             int64_t cols, int64_t nchunks,
                                                             const float* __restrict__ sigma,
                                                             uint8_t* __restrict__ codes) {
  int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= nchunks) return;
  int64_t e0 = t * 32;
  int64_t per = rows * cols;
  int64_t b = e0 / per, rem = e0 % per;
  int64_t r = rem / cols, c = rem % cols;
  float sg = sigma[(b * (rows / 128) + r / 128) * (cols / 128) + c / 128];
  float v[32];
  load_vals<32>(x + e0, v);
  uint32_t out[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t d = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float a = v[4 * w + j];
      uint32_t cc = sg > 0.0f ? e4m3_exact_quotient(fabsf(a), sg) : 0u;
      cc |= (__float_as_uint(a) >> 24) & 0x80u;
      d |= cc << (8 * j);
    }
    out[w] = d;
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + e0);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
}

// ---------------------------------------------------------------- dequantize

template <typename OutT>
__device__ __forceinline__ void store8(OutT* out, int64_t i, const float (&f)[8]);

template <>
__device__ __forceinline__ void store8<float>(float* out, int64_t i, const float (&f)[8]) {
  float4* d = reinterpret_cast<float4*>(out + i);
  d[0] = make_float4(f[0], f[1], f[2], f[3]);
  d[1] = make_float4(f[4], f[5], f[6], f[7]);
}

template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t* out, int64_t i, const float (&f)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = f32_to_bf16_bits(f[2 * j]) | (f32_to_bf16_bits(f[2 * j + 1]) << 16);
  *reinterpret_cast<uint4*>(out + i) = make_uint4(w[0], w[1], w[2], w[3]);
}

// MXFP8 quantization that also writes the exact values of the codes, e4m3(c)
// * 2^e: four significant bits, so exact in f32 and in bf16 (both outputs keep
// every finite result of an f32 or bf16 input's block).
template <typename T, typename OutT>
__global__ void __launch_bounds__(256) quant_mxfp8_deq_kernel(const T* __restrict__ x, int64_t nblocks,
                                                              uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales,
                                                              OutT* __restrict__ deq) {
  int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= nblocks) return;
  uint32_t out[8];
  const int e = mxfp8_block<T>(x, g, codes, scales, out);
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    float f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t c = (out[2 * h + j / 4] >> (8 * (j % 4))) & 0xFFu;
      const float m = ldexpf(e4m3_to_f32(c & 0x7Fu), e);
      f[j] = (c & 0x80u) ? -m : m;
    }
    store8<OutT>(deq, g * 32 + 8 * h, f);
  }
}

// fmt: 0 NVFP4, 1 MXFP4, 2 MXFP8, 3 FP8_BLOCK, 4 FP8_ROW.  One thread per 8 values.
// Squared quantization error of each NVFP4 (FMT 0, 16 values) or MXFP4 (FMT 1,
// 32 values) block: err[g] = sum over the block of (x - xhat)^2, xhat the
// dequantized value exactly as dequant_kernel produces it, each difference,
// square and sum rounded to f32.  One lane per block.
template <int FMT, typename T>
__global__ void __launch_bounds__(256) block_err_kernel(const T* __restrict__ x, const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales,
                                                        const float* __restrict__ tensor_scale, int64_t per,
                                                        int64_t nblocks, float* __restrict__ err) {
  constexpr int BS = FMT == 0 ? 16 : 32;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= nblocks) return;
  const int64_t e0 = g * BS;
  float v[BS];
  load_vals<BS>(x + e0, v);
  float sb = 0.0f, S = 0.0f;
  int e = 0;
  if (FMT == 0) {
    sb = e4m3_to_f32(scales[g]);
    S = tensor_scale[e0 / per];
  } else {
    e = (int)scales[g] - 127;
  }
  const uint32_t* cw = reinterpret_cast<const uint32_t*>(codes + e0 / 2);
  float acc = 0.0f;
#pragma unroll
  for (int w = 0; w < BS / 8; ++w) {
    const uint32_t d = cw[w];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t c = (d >> (4 * j)) & 15u;
      const float mag = FMT == 0 ? (e2m1_mag_to_f32(c & 7u) * sb) * S : ldexpf(e2m1_mag_to_f32(c & 7u), e);
      const float diff = v[8 * w + j] - ((c & 8u) ? -mag : mag);
      acc = fmaf(diff, diff, acc);
    }
  }
  err[g] = acc;
}

template <int FMT, typename OutT>
__global__ void __launch_bounds__(256) dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const void* __restrict__ scales,
                                                      const float* __restrict__ tensor_scale,
                                                      int64_t rows, int64_t cols, int64_t n8,
                                                      OutT* __restrict__ out) {
  int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n8) return;
  int64_t e0 = t * 8;
  float f[8];
  if (FMT == 0 || FMT == 1) {
    uint32_t d = reinterpret_cast<const uint32_t*>(codes)[t];
    float s;
    if (FMT == 0) {
      int64_t b = e0 / (rows * cols);
      float sb = e4m3_to_f32(reinterpret_cast<const uint8_t*>(scales)[e0 / 16]);
      float S = tensor_scale[b];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t c = (d >> (4 * j)) & 15u;
        float gs = e2m1_mag_to_f32(c & 7u) * sb;   // exact (<= 6 significant bits)
        float val = gs * S;                          // the one rounding
        f[j] = (c & 8u) ? -val : val;
      }
    } else {
      int e = (int)reinterpret_cast<const uint8_t*>(scales)[e0 / 32] - 127;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t c = (d >> (4 * j)) & 15u;
        float val = ldexpf(e2m1_mag_to_f32(c & 7u), e);
        f[j] = (c & 8u) ? -val : val;
      }
    }
    (void)s;
  } else {
    uint2 d2 = reinterpret_cast<const uint2*>(codes)[t];
    uint32_t dd[2] = {d2.x, d2.y};
    if (FMT == 2) {
      int e = (int)reinterpret_cast<const uint8_t*>(scales)[e0 / 32] - 127;
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = ldexpf(e4m3_to_f32((dd[j >> 2] >> (8 * (j & 3))) & 0xFFu), e);
    } else {
      float sg;
      if (FMT == 3) {
        int64_t per = rows * cols;
        int64_t b = e0 / per, rem = e0 % per;
        int64_t r = rem / cols, c = rem % cols;
        sg = reinterpret_cast<const float*>(scales)[(b * (rows / 128) + r / 128) * (cols / 128) + c / 128];
      } else {
        sg = reinterpret_cast<const float*>(scales)[e0 / 128];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = e4m3_to_f32((dd[j >> 2] >> (8 * (j & 3))) & 0xFFu) * sg;
    }
  }
  store8<OutT>(out, e0, f);
}

}  // namespace fp4

using namespace fp4;

// ---------------------------------------------------------------- host side

namespace {

int launch_fill(uint32_t* p, uint32_t v, int64_t n, hipStream_t st) {
  if (n <= 0) return FP4_OK;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_1d(n, 256)), dim3(256), 0, st, p, v, n);
  return check_launch("fill");
}

// Number of chunks a dynamic-scale NVFP4 batch from bf16 is cut into, so
// that the amax of one chunk is taken while the previous one is quantized
// (1: a separate amax pass first).  Each chunk must still fill the chip, and
// every lane of every quantization workgroup must hold a block.  Eight
// measured best on 512-tensor batches (four and sixteen within 2 %; smaller
// chunks lose more to launch ramps than the fused amax saves).
template <typename T>
int amax_chunks(int64_t batch, int64_t per) {
  if (!std::is_same<T, uint16_t>::value || batch < 16 || per < (1 << 20) || (per / 16) % 256 != 0) return 1;
  int64_t n = std::max<int64_t>(1, std::min<int64_t>(8, batch / 8));
  while ((batch + n - 1) / n > 65535) ++n;
  return (int)n;
}

template <typename T>
int quantize_typed(int fmt, int rule, int ts_mode, const T* x, int64_t batch, int64_t rows,
                   int64_t cols, uint8_t* codes, void* scales, float* tensor_scale,
                   uint8_t* m4, hipStream_t st) {
  const int64_t per = rows * cols;
  if (fmt == FP4_FMT_NVFP4 || fmt == FP4_FMT_MXFP4) {
    const bool mx = fmt == FP4_FMT_MXFP4;
    const int bs = mx ? 32 : 16;
    const int64_t bpt = per / bs;
    // tensor amax of tensors [b0, b0 + nb), then their scales amax / 2688
    auto amax_range = [&](int64_t b0, int64_t nb, hipStream_t sx) -> int {
      // about 4 workgroups per CU in total, at least one per tensor
      int64_t chunks = (per / 8 + 255) / 256;
      int64_t target = 4LL * device_cu_count() / nb;
      unsigned gx = (unsigned)std::max<int64_t>(1, std::min<int64_t>(chunks, std::max<int64_t>(target, 1)));
      for (int64_t c0 = 0; c0 < nb; c0 += 65535) {
        unsigned gy = (unsigned)std::min<int64_t>(65535, nb - c0);
        hipLaunchKernelGGL(tensor_amax_kernel<T>, dim3(gx, gy), dim3(256), 0, sx, x + (b0 + c0) * per, per,
                           reinterpret_cast<uint32_t*>(tensor_scale) + b0 + c0);
        FP4_CHECK(check_launch("tensor_amax"));
      }
      hipLaunchKernelGGL(nv_tensor_scale_kernel, dim3(grid_1d(nb, 256)), dim3(256), 0, sx, tensor_scale + b0, nb);
      return check_launch("tensor_scale");
    };
    // quantization of tensors [b0, b0 + nb); with nn > 0 the same launch also
    // takes partial maxima of the nn <= nb tensors that follow (bf16 NVFP4
    // only), stored in the code bytes of those tensors, which are written
    // only later, by their own quantization
    auto quant_range = [&](int64_t b0, int64_t nb, hipStream_t sx, int64_t nn = 0) -> int {
      unsigned gx = grid_1d(bpt, 256);
      const T* nx = nn > 0 ? x + (b0 + nb) * per : nullptr;
      float* np_ = nn > 0 ? reinterpret_cast<float*>(codes + (b0 + nb) * per / 2) : nullptr;
      for (int64_t c0 = b0; c0 < b0 + nb; c0 += 65535) {
        unsigned gy = (unsigned)std::min<int64_t>(65535, b0 + nb - c0);
        const T* xb = x + c0 * per;
        uint8_t* cb = codes + c0 * per / 2;
        uint8_t* sb = reinterpret_cast<uint8_t*>(scales) + c0 * bpt;
        const float* tb = tensor_scale ? tensor_scale + c0 : nullptr;
        uint8_t* mb = m4 ? m4 + c0 * bpt : nullptr;
        dim3 grid(gx, gy);
        if (!mx && rule == FP4_RULE_SWEEP)
          hipLaunchKernelGGL((quant_fp4_kernel<16, false, true, T, true>), grid, dim3(256), 0, sx, xb, bpt, cb, sb, tb, mb, nx, np_, per / 8, (int)nn);
        else if (!mx && rule == FP4_RULE_4OVER6)
          hipLaunchKernelGGL((quant_fp4_kernel<16, false, true, T>), grid, dim3(256), 0, sx, xb, bpt, cb, sb, tb, mb, nx, np_, per / 8, (int)nn);
        else if (!mx)
          hipLaunchKernelGGL((quant_fp4_kernel<16, false, false, T>), grid, dim3(256), 0, sx, xb, bpt, cb, sb, tb, mb, nx, np_, per / 8, (int)nn);
        else if (rule == FP4_RULE_4OVER6 || rule == FP4_RULE_SWEEP)  // MX: the sweep's candidates are the two plans
          hipLaunchKernelGGL((quant_fp4_kernel<32, true, true, T>), grid, dim3(256), 0, sx, xb, bpt, cb, sb, tb, mb, nx, np_, per / 8, (int)nn);
        else
          hipLaunchKernelGGL((quant_fp4_kernel<32, true, false, T>), grid, dim3(256), 0, sx, xb, bpt, cb, sb, tb, mb, nx, np_, per / 8, (int)nn);
        FP4_CHECK(check_launch("quant_fp4"));
      }
      return FP4_OK;
    };
    if (mx || ts_mode != FP4_TS_DYNAMIC) return quant_range(0, batch, st);
    if (batch == 1 && reinterpret_cast<uintptr_t>(codes) % 4 == 0) {
      // One tensor: the workgroups' maxima are parked in its code bytes,
      // which only the quantization below writes (per / 2 bytes hold the
      // at most per / 2048 + 1 floats), and one small kernel turns them into
      // the scale; no fill and no atomics.
      const int64_t gx = std::max<int64_t>(1, std::min<int64_t>((per / 8 + 255) / 256, 8LL * device_cu_count()));
      float* part = reinterpret_cast<float*>(codes);
      hipLaunchKernelGGL(amax_parts_kernel<T>, dim3((unsigned)gx), dim3(256), 0, st, x, per, part);
      FP4_CHECK(check_launch("amax_parts"));
      hipLaunchKernelGGL(nv_scale_from_parts_kernel, dim3(1), dim3(256), 0, st, part, (int64_t)0, (int)gx,
                         tensor_scale);
      FP4_CHECK(check_launch("tensor_scale"));
      return quant_range(0, 1, st);
    }
    FP4_CHECK(launch_fill(reinterpret_cast<uint32_t*>(tensor_scale), 0u, batch, st));
    const int nch = amax_chunks<T>(batch, per);
    if (nch <= 1) {
      FP4_CHECK(amax_range(0, batch, st));
      return quant_range(0, batch, st);
    }
    // The amax pass only streams from HBM while the quantization pass is
    // bound by vector ALU work, so the batch is cut into chunks and the amax
    // of chunk c+1 is taken inside the quantization launch of chunk c, from
    // loads that hide under its arithmetic.  Stream order alone sequences
    // the chunks: amax(c+1) lands before the scale kernel of c+1, which
    // runs before the quantization of c+1.
    const int64_t per_chunk = (batch + nch - 1) / nch;
    FP4_CHECK(amax_range(0, std::min<int64_t>(per_chunk, batch), st));
    for (int64_t b0 = 0; b0 < batch; b0 += per_chunk) {
      const int64_t nb = std::min<int64_t>(per_chunk, batch - b0);
      const int64_t nn = std::min<int64_t>(per_chunk, std::max<int64_t>(0, batch - b0 - nb));
      FP4_CHECK(quant_range(b0, nb, st, nn));
      if (nn > 0) {
        hipLaunchKernelGGL(nv_scale_from_parts_kernel, dim3((unsigned)nn), dim3(256), 0, st,
                           reinterpret_cast<const float*>(codes + (b0 + nb) * per / 2), per / 8,
                           (int)grid_1d(bpt, 256), tensor_scale + b0 + nb);
        FP4_CHECK(check_launch("tensor_scale"));
      }
    }
    return FP4_OK;
  }
  if (fmt == FP4_FMT_MXFP8) {
    int64_t nb = batch * per / 32;
    hipLaunchKernelGGL(quant_mxfp8_kernel<T>, dim3(grid_1d(nb, 256)), dim3(256), 0, st, x, nb, codes,
                       reinterpret_cast<uint8_t*>(scales));
    return check_launch("quant_mxfp8");
  }
  if (fmt == FP4_FMT_FP8_ROW) {
    int64_t ng = batch * per / 128;
    hipLaunchKernelGGL(quant_fp8_row_kernel<T>, dim3(grid_1d(ng * 4, 256)), dim3(256), 0, st, x, ng,
                       codes, reinterpret_cast<float*>(scales));
    return check_launch("quant_fp8_row");
  }
  if (fmt == FP4_FMT_FP8_BLOCK) {
    int64_t tiles = (rows / 128) * (cols / 128);
    for (int64_t b0 = 0; b0 < batch; b0 += 65535) {
      unsigned gy = (unsigned)std::min<int64_t>(65535, batch - b0);
      hipLaunchKernelGGL(fp8_tile_amax_kernel<T>, dim3((unsigned)tiles, gy), dim3(256), 0, st,
                         x + b0 * per, rows, cols, reinterpret_cast<float*>(scales) + b0 * tiles);
      FP4_CHECK(check_launch("fp8_tile_amax"));
    }
    int64_t nchunks = batch * per / 32;
    hipLaunchKernelGGL(quant_fp8_tile_kernel<T>, dim3(grid_1d(nchunks, 256)), dim3(256), 0, st, x, rows,
                       cols, nchunks, reinterpret_cast<const float*>(scales), codes);
    return check_launch("quant_fp8_tile");
  }
  return fail(FP4_ERR_INVALID_ARG, "unknown format %d", fmt);
}

template <typename T>
int tensor_scales_typed(const T* x, int64_t batch, int64_t per, float* tensor_scale, hipStream_t st) {
  FP4_CHECK(launch_fill(reinterpret_cast<uint32_t*>(tensor_scale), 0u, batch, st));
  const int64_t chunks = (per / 8 + 255) / 256;
  for (int64_t b0 = 0; b0 < batch; b0 += 65535) {
    const int64_t nb = std::min<int64_t>(65535, batch - b0);
    const int64_t target = 4LL * device_cu_count() / nb;
    const unsigned gx = (unsigned)std::max<int64_t>(1, std::min<int64_t>(chunks, std::max<int64_t>(target, 1)));
    hipLaunchKernelGGL(tensor_amax_kernel<T>, dim3(gx, (unsigned)nb), dim3(256), 0, st, x + b0 * per, per,
                       reinterpret_cast<uint32_t*>(tensor_scale) + b0);
    FP4_CHECK(check_launch("tensor_amax"));
  }
  hipLaunchKernelGGL(nv_tensor_scale_kernel, dim3(grid_1d(batch, 256)), dim3(256), 0, st, tensor_scale, batch);
  return check_launch("tensor_scale");
}

int block_of(int fmt) {
  switch (fmt) {
    case FP4_FMT_NVFP4: return 16;
    case FP4_FMT_MXFP4:
    case FP4_FMT_MXFP8: return 32;
    case FP4_FMT_FP8_BLOCK:
    case FP4_FMT_FP8_ROW: return 128;
    default: return 0;
  }
}

}  // namespace

namespace fp4 {
int mxfp8_quantize_dequant(const void* x, int x_dtype, int64_t rows, int64_t cols, uint8_t* codes,
                           uint8_t* scales, void* deq, int deq_dtype, hipStream_t st) {
  if (cols % 32) return fail(FP4_ERR_SHAPE, "MXFP8 needs cols %% 32 == 0");
  const int64_t nb = rows * cols / 32;
  if (nb == 0) return FP4_OK;
  const dim3 grid(grid_1d(nb, 256));
  if (x_dtype == FP4_DT_BF16 && deq_dtype == FP4_DT_BF16)
    hipLaunchKernelGGL((quant_mxfp8_deq_kernel<uint16_t, uint16_t>), grid, dim3(256), 0, st,
                       reinterpret_cast<const uint16_t*>(x), nb, codes, scales, reinterpret_cast<uint16_t*>(deq));
  else if (x_dtype == FP4_DT_F32 && deq_dtype == FP4_DT_F32)
    hipLaunchKernelGGL((quant_mxfp8_deq_kernel<float, float>), grid, dim3(256), 0, st,
                       reinterpret_cast<const float*>(x), nb, codes, scales, reinterpret_cast<float*>(deq));
  else
    return fail(FP4_ERR_UNSUPPORTED, "MXFP8 quantize-dequantize: bf16->bf16 or f32->f32 only");
  return check_launch("quant_mxfp8_deq");
}

int nv_tensor_scales(const void* x, int x_dtype, int64_t batch, int64_t per, float* tensor_scale,
                     hipStream_t st) {
  if (batch <= 0) return FP4_OK;
  if (x_dtype == FP4_DT_BF16)
    return tensor_scales_typed(reinterpret_cast<const uint16_t*>(x), batch, per, tensor_scale, st);
  return tensor_scales_typed(reinterpret_cast<const float*>(x), batch, per, tensor_scale, st);
}

int nv_tensor_scale_from_parts(const float* part, int64_t nparts, float* s, hipStream_t st) {
  if (nparts < 1 || nparts > INT32_MAX) return fail(FP4_ERR_INVALID_ARG, "tensor scale from %lld partial maxima",
                                                    (long long)nparts);
  hipLaunchKernelGGL(nv_scale_from_parts_kernel, dim3(1), dim3(256), 0, st, part, (int64_t)0, (int)nparts, s);
  return check_launch("nv_scale_from_parts");
}
}  // namespace fp4

extern "C" {

const char* fp4_status_string(int status) {
  switch (status) {
    case FP4_OK: return "FP4_OK";
    case FP4_ERR_INVALID_ARG: return "FP4_ERR_INVALID_ARG";
    case FP4_ERR_SHAPE: return "FP4_ERR_SHAPE";
    case FP4_ERR_UNSUPPORTED: return "FP4_ERR_UNSUPPORTED";
    case FP4_ERR_WORKSPACE: return "FP4_ERR_WORKSPACE";
    case FP4_ERR_HIP: return "FP4_ERR_HIP";
    default: return "FP4_ERR_UNKNOWN";
  }
}

const char* fp4_last_error(void) { return fp4::g_last_error.c_str(); }

int fp4_quantize(int fmt, int rule, int ts_mode, const void* x, int x_dtype, int64_t batch,
                 int64_t rows, int64_t cols, uint8_t* codes, void* scales, float* tensor_scale,
                 uint8_t* m4_flags, void* stream) {
  int bs = block_of(fmt);
  if (bs == 0) return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: unknown format %d", fmt);
  if (rule != FP4_RULE_RTN && rule != FP4_RULE_4OVER6 && rule != FP4_RULE_SWEEP)
    return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: unknown rule %d", rule);
  if (ts_mode != FP4_TS_DYNAMIC && ts_mode != FP4_TS_STATIC)
    return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: unknown tensor-scale mode %d", ts_mode);
  if (x_dtype != FP4_DT_BF16 && x_dtype != FP4_DT_F32)
    return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: unknown dtype %d", x_dtype);
  if (batch < 0 || rows < 0 || cols < 0)
    return fail(FP4_ERR_SHAPE, "fp4_quantize: negative dimension");
  if (cols % bs) return fail(FP4_ERR_SHAPE, "fp4_quantize: cols %lld not a multiple of %d", (long long)cols, bs);
  if (fmt == FP4_FMT_FP8_BLOCK && rows % 128)
    return fail(FP4_ERR_SHAPE, "fp4_quantize: rows %lld not a multiple of 128", (long long)rows);
  if (batch == 0 || rows == 0 || cols == 0) return FP4_OK;
  if (!x || !codes || !scales) return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: null pointer");
  if (fmt == FP4_FMT_NVFP4 && !tensor_scale)
    return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: NVFP4 needs tensor_scale");
  if (fmt != FP4_FMT_NVFP4 && fmt != FP4_FMT_MXFP4) m4_flags = nullptr;
  hipStream_t st = as_stream(stream);
  if (x_dtype == FP4_DT_BF16)
    return quantize_typed<uint16_t>(fmt, rule, ts_mode, reinterpret_cast<const uint16_t*>(x), batch,
                                    rows, cols, codes, scales, tensor_scale, m4_flags, st);
  return quantize_typed<float>(fmt, rule, ts_mode, reinterpret_cast<const float*>(x), batch, rows,
                               cols, codes, scales, tensor_scale, m4_flags, st);
}

int fp4_dequantize(int fmt, const uint8_t* codes, const void* scales, const float* tensor_scale,
                   int64_t batch, int64_t rows, int64_t cols, void* out, int out_dtype,
                   void* stream) {
  int bs = block_of(fmt);
  if (bs == 0) return fail(FP4_ERR_INVALID_ARG, "fp4_dequantize: unknown format %d", fmt);
  if (out_dtype != FP4_DT_BF16 && out_dtype != FP4_DT_F32)
    return fail(FP4_ERR_INVALID_ARG, "fp4_dequantize: unknown dtype %d", out_dtype);
  if (batch < 0 || rows < 0 || cols < 0) return fail(FP4_ERR_SHAPE, "fp4_dequantize: negative dimension");
  if (cols % bs) return fail(FP4_ERR_SHAPE, "fp4_dequantize: cols %lld not a multiple of %d", (long long)cols, bs);
  if (fmt == FP4_FMT_FP8_BLOCK && rows % 128)
    return fail(FP4_ERR_SHAPE, "fp4_dequantize: rows %lld not a multiple of 128", (long long)rows);
  if (batch == 0 || rows == 0 || cols == 0) return FP4_OK;
  if (!codes || !scales || !out) return fail(FP4_ERR_INVALID_ARG, "fp4_dequantize: null pointer");
  if (fmt == FP4_FMT_NVFP4 && !tensor_scale)
    return fail(FP4_ERR_INVALID_ARG, "fp4_dequantize: NVFP4 needs tensor_scale");
  hipStream_t st = as_stream(stream);
  int64_t n8 = batch * rows * cols / 8;
  dim3 grid(grid_1d(n8, 256));
#define FP4_DQ(F)                                                                                  \
  if (out_dtype == FP4_DT_F32)                                                                     \
    hipLaunchKernelGGL((dequant_kernel<F, float>), grid, dim3(256), 0, st, codes, scales,          \
                       tensor_scale, rows, cols, n8, reinterpret_cast<float*>(out));               \
  else                                                                                             \
    hipLaunchKernelGGL((dequant_kernel<F, uint16_t>), grid, dim3(256), 0, st, codes, scales,       \
                       tensor_scale, rows, cols, n8, reinterpret_cast<uint16_t*>(out));
  switch (fmt) {
    case FP4_FMT_NVFP4: FP4_DQ(0) break;
    case FP4_FMT_MXFP4: FP4_DQ(1) break;
    case FP4_FMT_MXFP8: FP4_DQ(2) break;
    case FP4_FMT_FP8_BLOCK: FP4_DQ(3) break;
    case FP4_FMT_FP8_ROW: FP4_DQ(4) break;
  }
#undef FP4_DQ
  return check_launch("dequant");
}

int fp4_block_error(int fmt, const void* x, int x_dtype, int64_t batch, int64_t rows, int64_t cols,
                    const uint8_t* codes, const void* scales, const float* tensor_scale, float* err,
                    void* stream) {
  using namespace fp4;
  if (fmt != FP4_FMT_NVFP4 && fmt != FP4_FMT_MXFP4)
    return fail(FP4_ERR_UNSUPPORTED, "fp4_block_error: NVFP4 or MXFP4 only (got %d)", fmt);
  if (x_dtype != FP4_DT_BF16 && x_dtype != FP4_DT_F32)
    return fail(FP4_ERR_INVALID_ARG, "fp4_block_error: unknown dtype %d", x_dtype);
  if (batch < 0 || rows < 0 || cols < 0) return fail(FP4_ERR_SHAPE, "fp4_block_error: negative dimension");
  const int bs = fmt == FP4_FMT_NVFP4 ? 16 : 32;
  if (cols % bs) return fail(FP4_ERR_SHAPE, "fp4_block_error: cols %lld not a multiple of %d", (long long)cols, bs);
  if (batch == 0 || rows == 0 || cols == 0) return FP4_OK;
  if (!x || !codes || !scales || !err || (fmt == FP4_FMT_NVFP4 && !tensor_scale))
    return fail(FP4_ERR_INVALID_ARG, "fp4_block_error: null pointer");
  if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(codes) % 4)
    return fail(FP4_ERR_INVALID_ARG, "fp4_block_error: x needs 16-byte and codes 4-byte alignment");
  const int64_t per = rows * cols, nb = batch * per / bs;
  const dim3 grid(grid_1d(nb, 256));
  hipStream_t st = as_stream(stream);
  const uint8_t* sc = reinterpret_cast<const uint8_t*>(scales);
  if (fmt == FP4_FMT_NVFP4 && x_dtype == FP4_DT_BF16)
    hipLaunchKernelGGL((block_err_kernel<0, uint16_t>), grid, dim3(256), 0, st,
                       reinterpret_cast<const uint16_t*>(x), codes, sc, tensor_scale, per, nb, err);
  else if (fmt == FP4_FMT_NVFP4)
    hipLaunchKernelGGL((block_err_kernel<0, float>), grid, dim3(256), 0, st, reinterpret_cast<const float*>(x),
                       codes, sc, tensor_scale, per, nb, err);
  else if (x_dtype == FP4_DT_BF16)
    hipLaunchKernelGGL((block_err_kernel<1, uint16_t>), grid, dim3(256), 0, st,
                       reinterpret_cast<const uint16_t*>(x), codes, sc, tensor_scale, per, nb, err);
  else
    hipLaunchKernelGGL((block_err_kernel<1, float>), grid, dim3(256), 0, st, reinterpret_cast<const float*>(x),
                       codes, sc, tensor_scale, per, nb, err);
  return check_launch("block_err");
}

}  // extern "C"
