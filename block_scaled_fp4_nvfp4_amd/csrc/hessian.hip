// Hessian-weighted NVFP4 block-scale search behind fp4_quantize_hessian (gfx950).
//
// The Local-Hessian NVFP4 card ("What is different about it") chooses each
// group's weight scale by a Hessian-weighted search instead of the plain
// amax / MSE sweep; only the weight_scale values change (same format, same
// tensor scale), and experts with fewer than 64 routed calibration rows keep
// plain max ("Results").  Reading taken here (the search is only named):
//  * candidates: every E4M3 scale code from the amax/6 plan's to the
//    block-max-to-4 plan's (the sweep's window), codes E2M1 round-to-nearest-
//    even of x / (s S);
//  * error of a candidate: err = d^T H_b d, d = x - xhat (signed), H_b the
//    16 x 16 diagonal block of the expert's input Hessian for the block's
//    columns; the first candidate with the smallest exact error is kept.
//
// Exactness.  d is exact in double (x has at most 24 significant bits,
// xhat = g s S at most 31, and where g > 0 the two lie within a factor of a
// few of each other; where g = 0, d = x).  err is evaluated in double from
// the upper triangle T of H + H^T (T_ii = H_ii, T_ij = H_ij + H_ji for j > i,
// exact in double from f32 H) with fma chains, t_i = sum_{j>=i} T_ij d_j then
// sum_i d_i t_i (d^T H d equals d^T T d for any H; 152 fmas against 272 for
// the full product), whose rounding error is below 2 * 16 * 2^-53 * M with
// M = sum_ij |T_ij| |d_i| |d_j| <= sum_ij |H_ij| |d_i| |d_j|; M is bounded
// by B = (sum_i |d_i|)^2 max |H|.  Two candidates whose double errors differ
// by more than 2^-46 (B_a + B_b) are therefore ordered correctly; closer
// ones are compared exactly: every term H_ij d_i d_j is split into four
// doubles by error-free products (two_prod through fma) and accumulated into
// a 1024-bit fixed-point integer whose least significant bit is 2^-576
// (every term is a multiple of 2^-467: x and S are multiples of 2^-149, g s
// of 2^-10; and below 2^420 in magnitude), and the sign of the difference
// decides.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "fp4_device.h"
#include "host_common.h"

#pragma clang fp contract(off)

namespace fp4 {

constexpr int kHessMinRows = 64;  // calibration rows for a full Hessian
constexpr int kAccLimbs = 16;     // 1024-bit accumulator
constexpr int kAccLsb = -576;     // weight of its least significant bit: 2^-576

// acc += sgn * v for a double v that is a multiple of 2^-519 with |v| < 2^447
// (two's complement over kAccLimbs limbs).
__device__ __noinline__ void acc_add(uint64_t* acc, double v, bool neg) {
  if (v == 0.0) return;
  const uint64_t bits = (uint64_t)__double_as_longlong(v);
  const int ex = (int)((bits >> 52) & 0x7FF);
  uint64_t m = bits & 0xFFFFFFFFFFFFFull;
  int k;  // v = +-m * 2^k
  if (ex == 0) {
    k = -1074;
  } else {
    m |= 1ull << 52;
    k = ex - 1075;
  }
  if ((bits >> 63) != 0) neg = !neg;
  const int pos = k - kAccLsb;  // in [57, 960) for finite inputs (the range above)
  if (pos < 0 || pos >= 64 * (kAccLimbs - 1)) return;  // non-finite input: never out of the array
  const int li = pos >> 6, sh = pos & 63;
  const uint64_t lo = m << sh;
  const uint64_t hi = sh ? (m >> (64 - sh)) : 0ull;
  if (!neg) {
    uint64_t s = acc[li] + lo;
    uint64_t c = s < lo;
    acc[li] = s;
    uint64_t t = acc[li + 1] + hi;
    uint64_t c2 = t < hi;
    t += c;
    c2 |= (t < c);
    acc[li + 1] = t;
    for (int i = li + 2; c2 && i < kAccLimbs; ++i) {
      acc[i] += 1ull;
      c2 = acc[i] == 0ull;
    }
  } else {
    uint64_t a = acc[li];
    uint64_t b = a < lo;
    acc[li] = a - lo;
    uint64_t a1 = acc[li + 1];
    uint64_t d1 = a1 - hi;
    uint64_t b2 = a1 < hi;
    b2 |= d1 < b;
    acc[li + 1] = d1 - b;
    for (int i = li + 2; b2 && i < kAccLimbs; ++i) {
      b2 = acc[i] == 0ull;
      acc[i] -= 1ull;
    }
  }
}

// acc += sgn * h * a * b exactly (four doubles from error-free products).
__device__ __forceinline__ void acc_add_prod3(uint64_t* acc, double h, double a, double b, bool neg) {
  const double p = a * b;
  const double e = fma(a, b, -p);
  const double p1 = h * p;
  const double e1 = fma(h, p, -p1);
  const double p2 = h * e;
  const double e2 = fma(h, e, -p2);
  acc_add(acc, p1, neg);
  acc_add(acc, e1, neg);
  acc_add(acc, p2, neg);
  acc_add(acc, e2, neg);
}

// True iff d_a^T H d_a < d_b^T H d_b exactly (H: 16 x 16 doubles in LDS).
__device__ __noinline__ bool exact_less(const double* da, const double* db, const double* H) {
  uint64_t acc[kAccLimbs];
  for (int i = 0; i < kAccLimbs; ++i) acc[i] = 0ull;
  for (int i = 0; i < 16; ++i)
    for (int j = 0; j < 16; ++j) {
      const double h = H[16 * i + j];
      acc_add_prod3(acc, h, da[i], da[j], false);
      acc_add_prod3(acc, h, db[i], db[j], true);
    }
  // err_a - err_b < 0 iff the top bit is set
  return (acc[kAccLimbs - 1] >> 63) != 0ull;
}

// One candidate: E2M1 magnitudes (nibbles, sign clear) and signed residuals
// d = x - xhat, exact in double.
__device__ __forceinline__ void candidate_residuals(const float (&v)[16], double unit, uint64_t& mags,
                                                    double (&d)[16]) {
  const E2M1Thresholds th = e2m1_thresholds(unit);
  mags = 0ull;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t m = e2m1_code(fabsf(v[i]), th);
    mags |= (uint64_t)m << (4 * i);
    const double q = (double)e2m1_mag_to_f32(m) * unit;  // <= 31 significant bits: exact
    d[i] = (double)v[i] - (signbit(v[i]) ? -q : q);
  }
}

// Row i of the packed upper triangle starts at tri_row(i) (16 - i entries).
constexpr int kTriSize = 136;
__host__ __device__ constexpr int tri_row(int i) { return 16 * i - i * (i - 1) / 2; }

// d^T T d by fma chains (T rows from LDS, broadcast reads) and the bound
// (sum |d|)^2 * max |H| of its rounding error's scale.
// The LDS offset passes through an empty asm statement on every call, so the
// 136 reads of T stay inside the candidate loop (hoisted out of it, they
// would hold 272 registers).
__device__ __forceinline__ void weighted_error(const double (&d)[16], const double* T, double hmax, double& err,
                                               double& bound) {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  const double* Tz = T + z;
  double e = 0.0, s = 0.0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    double t = 0.0;
#pragma unroll
    for (int j = i; j < 16; ++j) t = fma(Tz[tri_row(i) + j - i], d[j], t);
    e = fma(d[i], t, e);
    s += fabs(d[i]);
  }
  err = e;
  bound = s * s * hmax;
}

template <typename T>
__device__ __forceinline__ void load16(const T* p, float (&v)[16]);
template <>
__device__ __forceinline__ void load16<uint16_t>(const uint16_t* p, float (&v)[16]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint4 w = q[i];
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = __uint_as_float(d[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(d[j] & 0xFFFF0000u);
    }
  }
}
template <>
__device__ __forceinline__ void load16<float>(const float* p, float (&v)[16]) {
  const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 w = q[i];
    v[4 * i] = w.x; v[4 * i + 1] = w.y; v[4 * i + 2] = w.z; v[4 * i + 3] = w.w;
  }
}

// Grid: (ceil(rows / 256), cols / 16, experts in this launch).  Workgroup =
// 256 rows of one 16-column block of one expert; each thread one block.
template <typename T>
__global__ void __launch_bounds__(256) hessian_quant_kernel(const T* __restrict__ x, int64_t rows, int64_t cols,
                                                            const float* __restrict__ hess,
                                                            const int32_t* __restrict__ calib_rows,
                                                            const float* __restrict__ tensor_scale,
                                                            uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                            uint8_t* __restrict__ choice) {
  __shared__ double Hs[256];        // H_b, for the exact comparison
  __shared__ double Ts[kTriSize];   // upper triangle of H_b + H_b^T, for the double errors
  __shared__ float red[4];
  const int64_t e = blockIdx.z;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t nb = cols / 16;
  const bool full = calib_rows[e] >= kHessMinRows;
  double hmax = 0.0;
  if (full) {  // uniform per workgroup
    const float h = hess[(e * nb + b) * 256 + tid];
    Hs[tid] = (double)h;
    float m = fabsf(h);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    hmax = (double)fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const int i = tid >> 4, j = tid & 15;
    if (j >= i) Ts[tri_row(i) + j - i] = j == i ? Hs[tid] : Hs[16 * i + j] + Hs[16 * j + i];
    __syncthreads();
  }
  const int64_t r = (int64_t)blockIdx.x * 256 + tid;
  if (r >= rows) return;
  const int64_t blk = (e * rows + r) * nb + b;
  float v[16];
  load16<T>(x + blk * 16, v);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const float S = tensor_scale[e];
  uint32_t c6 = 0u, c4 = 0u;
  if (S > 0.0f && amax > 0.0f) {
    // E4M3 of the double quotient: exact (it cannot lie within double
    // rounding of an E4M3 decision point unless it is on one)
    c6 = e4m3_rne_sat_f64((double)amax / (6.0 * (double)S));
    c4 = full ? e4m3_rne_sat_f64((double)amax / (4.0 * (double)S)) : c6;
  }
  const double Sd = (double)S;
  uint32_t best = c6;
  uint64_t best_mags;
  double d[16];
  candidate_residuals(v, (double)e4m3_to_f32(c6) * Sd, best_mags, d);
  if (c4 > c6) {
    double best_err, best_bound;
    weighted_error(d, Ts, hmax, best_err, best_bound);
    for (uint32_t c = c6 + 1; c <= c4; ++c) {
      uint64_t mags;
      double dc[16];
      candidate_residuals(v, (double)e4m3_to_f32(c) * Sd, mags, dc);
      double err, bound;
      weighted_error(dc, Ts, hmax, err, bound);
      const double margin = 0x1p-46 * (bound + best_bound);
      bool take;
      if (fabs(err - best_err) > margin) {
        take = err < best_err;
      } else if (bound + best_bound == 0.0) {
        take = false;  // both residuals zero: equal errors, the first stays
      } else {
        // the exact comparison takes its residuals through memory: copies
        // made here, so that dc (written for every candidate) stays in
        // registers instead of living in scratch for the whole loop
        double da[16], db[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) da[i] = dc[i];
        uint64_t bm;
        candidate_residuals(v, (double)e4m3_to_f32(best) * Sd, bm, db);
        take = exact_less(da, db, Hs);
      }
      if (take) {
        best = c;
        best_mags = mags;
        best_err = err;
        best_bound = bound;
      }
    }
  }
  uint64_t packed = best_mags;
#pragma unroll
  for (int i = 0; i < 16; ++i) packed |= (uint64_t)(signbit(v[i]) ? 1u : 0u) << (4 * i + 3);
  *reinterpret_cast<uint2*>(codes + blk * 8) = make_uint2((uint32_t)packed, (uint32_t)(packed >> 32));
  scales[blk] = (uint8_t)best;
  if (choice) choice[blk] = (uint8_t)(best - c6);
}

}  // namespace fp4

using namespace fp4;

extern "C" int fp4_quantize_hessian(const void* x, int x_dtype, int64_t experts, int64_t rows, int64_t cols,
                                    const float* hessian, const int32_t* calib_rows, uint8_t* codes,
                                    uint8_t* scales, float* tensor_scale, uint8_t* choice, void* stream) {
  if (x_dtype != FP4_DT_BF16 && x_dtype != FP4_DT_F32)
    return fail(FP4_ERR_INVALID_ARG, "quantize_hessian: x must be bf16 or f32 (got %d)", x_dtype);
  if (experts < 0 || rows < 0 || cols < 0) return fail(FP4_ERR_SHAPE, "quantize_hessian: negative dimension");
  if (cols % 16) return fail(FP4_ERR_SHAPE, "quantize_hessian: cols %lld is not a multiple of 16", (long long)cols);
  if (experts == 0 || rows == 0 || cols == 0) return FP4_OK;
  if (!x || !hessian || !calib_rows || !codes || !scales || !tensor_scale)
    return fail(FP4_ERR_INVALID_ARG, "quantize_hessian: null pointer");
  if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(codes) % 8 ||
      reinterpret_cast<uintptr_t>(hessian) % 4 || reinterpret_cast<uintptr_t>(calib_rows) % 4 ||
      reinterpret_cast<uintptr_t>(tensor_scale) % 4)
    return fail(FP4_ERR_INVALID_ARG, "quantize_hessian: x needs 16-byte, codes 8-byte alignment");
  if (cols / 16 > 65535) return fail(FP4_ERR_UNSUPPORTED, "quantize_hessian: more than 65535 blocks per row");
  if ((rows + 255) / 256 > INT32_MAX) return fail(FP4_ERR_UNSUPPORTED, "quantize_hessian: too many rows");
  hipStream_t st = as_stream(stream);
  FP4_CHECK(nv_tensor_scales(x, x_dtype, experts, rows * cols, tensor_scale, st));
  const int64_t nb = cols / 16;
  for (int64_t e0 = 0; e0 < experts; e0 += 65535) {
    const int64_t ne = std::min<int64_t>(65535, experts - e0);
    const dim3 grid((unsigned)((rows + 255) / 256), (unsigned)nb, (unsigned)ne);
    const int64_t off = e0 * rows * cols;
    const float* h = hessian + e0 * nb * 256;
    if (x_dtype == FP4_DT_BF16)
      hipLaunchKernelGGL(hessian_quant_kernel<uint16_t>, grid, dim3(256), 0, st,
                         reinterpret_cast<const uint16_t*>(x) + off, rows, cols, h, calib_rows + e0,
                         tensor_scale + e0, codes + off / 2, scales + off / 16, choice ? choice + off / 16 : nullptr);
    else
      hipLaunchKernelGGL(hessian_quant_kernel<float>, grid, dim3(256), 0, st,
                         reinterpret_cast<const float*>(x) + off, rows, cols, h, calib_rows + e0,
                         tensor_scale + e0, codes + off / 2, scales + off / 16, choice ? choice + off / 16 : nullptr);
    FP4_CHECK(check_launch("hessian_quant"));
  }
  return FP4_OK;
}
