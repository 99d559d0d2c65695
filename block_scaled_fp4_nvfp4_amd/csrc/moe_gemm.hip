// Grouped MFMA GEMMs of the MoE forward for quantized activations, and the
// shared expert (gfx950).
//
// Modes (model cards on block_scaled_fp4_nvfp4):
//  * NVFP4 x NVFP4 (W4A4; Local-Hessian NVFP4 card, opening section: activation
//    tensor scale amax/2688).  Both operands are decoded exactly to fp16
//    (g * s has at most 6 significant bits and lies in [2^-10, 2688]) and
//    multiplied on the fp16 MFMA with fp32 accumulation; the two tensor
//    scales multiply the result.  The E4M3 block scale per 16 values has a
//    mantissa, so it cannot ride in the MFMA's power-of-two scale operand.
//  * MXFP4 weights x MXFP8 activations (MXFP4-FP8-R12 card, runtime contract
//    table): the block-scaled f8f6f4 MFMA consumes E2M1 / E4M3 codes and the
//    UE8M0 scales per 32 directly.
//  * Block FP8 (same card: retained block-FP8 experts, dynamic FP8
//    activations): E4M3 x E4M3 MFMA with unit scales per 128-wide K step,
//    each partial multiplied by the activation row's and the weight tile's
//    fp32 scales.
//  * Shared expert (FP4-Local AZ card, "The shared expert"): MXFP8 weights and
//    dynamic MXFP8 activations through the same block-scaled MFMA, output
//    scaled by sigmoid(x . gate).
//
// Operand lane layouts (gfx950, measured): v_mfma_scale_f32_16x16x128_f8f6f4
// takes, in lane l (g = l / 16), row l % 16 of A (column l % 16 of B) with
// FP8 codes for K in [16g, 16g+16) and [64+16g, 64+16g+16), or FP4 codes for K
// in [32g, 32g+32); the lane's scale byte belongs to row (column) l % 16 and
// K block l / 16 of 32.  v_mfma_f32_16x16x32_f16 takes K in [8g, 8g+8).  Both
// leave C[4g + r][l % 16] in accumulator r of lane l.
//
// Work decomposition: one workgroup (4 waves, 2 x 2) owns a 64-row x 64-output
// tile of one expert (for gate_up: 64 gate and the matching 64 up rows).  The
// permutation kernel provides each expert's first tile; workgroups are
// remapped so that consecutive tiles (same expert) run on the same XCD and
// share its L2.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "fp4_device.h"
#include "host_common.h"
#include "moe_common.h"
#include "moe_internal.h"

extern "C" int fp4_quantize(int fmt, int rule, int ts_mode, const void* x, int x_dtype, int64_t batch,
                            int64_t rows, int64_t cols, uint8_t* codes, void* scales, float* tensor_scale,
                            uint8_t* m4_flags, void* stream);

namespace fp4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));

enum { GK_NV = 0, GK_MX = 1, GK_FP8 = 2 };
enum { EPI_GATEUP = 0, EPI_DOWN = 1 };

constexpr int kBM = kGemmTileM;  // 64 rows per tile
constexpr int kBN = 64;          // outputs per tile
constexpr int kBK = 128;         // K per step

struct GemmArgs {
  // A operand: quantized activations, one row per token (gather) or per sorted row
  const uint8_t* a_codes;
  const void* a_scales;
  const float* a_tensor_scale;  // NVFP4
  int a_gather;                 // 1: A row = token of pair_of_row[row] / k; 0: A row = sorted row
  // B operand: weights [E][N_rows][K]
  const uint8_t* w_codes;
  const void* w_scales;
  const float* w_tensor_scale;  // NVFP4: [E]
  int w_fp8;                    // MX mode: weights are E4M3 codes (shared expert) instead of E2M1
  // routing
  const int32_t* offsets;       // [E+1] (dense: nullptr)
  const int32_t* pair_of_row;
  const int32_t* tile_offsets;  // [E+1]
  int E, k, dense_rows;         // dense_rows > 0: one expert with that many rows, no routing
  int K, N;                     // reduction size; outputs (gate_up: I; down: H)
  float* out;                   // gate_up: h [rows][N]; down: o [rows][N]
  const float* row_scale;       // down epilogue: per-row multiplier (shared-expert gate), may be null
};

// ---------------------------------------------------------------- operands

// NVFP4 16 bytes (32 values) + their two E4M3 scales -> 16 dwords of fp16 pairs.
__device__ __forceinline__ void nv_decode32(uint4 c, uint32_t s2, uint32_t (&o)[16]) {
  const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)s2, 0);
  const float s1 = __builtin_amdgcn_cvt_f32_fp8((int)s2, 1);
  const half2_t h0 = {(_Float16)s0, (_Float16)s0};
  const half2_t h1 = {(_Float16)s1, (_Float16)s1};
  const uint32_t d[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const half2_t sc = w < 2 ? h0 : h1;
#pragma unroll
    for (int sel = 0; sel < 4; ++sel) {
      half2_t p;
      if (sel == 0) p = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d[w], 1.0f, 0);
      if (sel == 1) p = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d[w], 1.0f, 1);
      if (sel == 2) p = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d[w], 1.0f, 2);
      if (sel == 3) p = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d[w], 1.0f, 3);
      p = p * sc;  // exact: <= 6 significant bits, in fp16's normal range
      o[4 * w + sel] = __builtin_bit_cast(uint32_t, p);
    }
  }
}

__device__ __forceinline__ half8_t as_half8(const uint32_t* p) {
  uint4 v = make_uint4(p[0], p[1], p[2], p[3]);
  return __builtin_bit_cast(half8_t, v);
}

// ------------------------------------------------------------------ kernel

template <int GK, int EPI>
__global__ void __launch_bounds__(256) grouped_gemm_kernel(GemmArgs g) {
  extern __shared__ int s_toff[];  // [E + 1] tile offsets (routed mode)
  const int NT = g.N / kBN;
  // XCD-aware order: hardware places workgroup i on XCD i % 8; give each XCD
  // a contiguous range of logical tiles.
  const int G = gridDim.x;
  const int per_xcd = G / 8;
  const int L = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;

  int e, mt, nt;
  int r_begin, n_rows;
  if (g.dense_rows > 0) {
    e = 0;
    nt = L % NT;
    mt = L / NT;
    if (mt * kBM >= g.dense_rows) return;
    r_begin = 0;
    n_rows = g.dense_rows;
  } else {
    for (int i = threadIdx.x; i <= g.E; i += 256) s_toff[i] = g.tile_offsets[i];
    __syncthreads();
    nt = L % NT;
    const int mg = L / NT;
    if (mg >= s_toff[g.E]) return;
    int lo = 0, hi = g.E;
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (s_toff[mid] <= mg) lo = mid; else hi = mid;
    }
    e = lo;
    mt = mg - s_toff[e];
    r_begin = g.offsets[e];
    n_rows = g.offsets[e + 1] - r_begin;
  }

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int lr = lane & 15, lg = lane >> 4;
  const int K = g.K;
  const int NW = EPI == EPI_GATEUP ? 2 * g.N : g.N;  // weight rows per expert

  // A rows handled by this lane (two 16-row subtiles)
  const uint8_t* a_ptr[2];
  bool a_ok[2];
  int a_row[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int rr = mt * kBM + wm * 32 + i * 16 + lr;  // row within the expert
    a_ok[i] = rr < n_rows;
    int R = r_begin + (a_ok[i] ? rr : 0);
    int arow = g.a_gather ? g.pair_of_row[R] / g.k : R;
    a_row[i] = arow;
    int64_t rb = GK == GK_NV ? (int64_t)K / 2 : (int64_t)K;
    a_ptr[i] = g.a_codes + (int64_t)arow * rb;
  }
  // weight rows handled by this lane: [n-subtile j][gate/up u]
  constexpr int NU = EPI == EPI_GATEUP ? 2 : 1;
  int w_row[2][NU];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int u = 0; u < NU; ++u) w_row[j][u] = u * g.N + nt * kBN + wn * 32 + j * 16 + lr;
  const int64_t w_rb = (GK == GK_NV || (GK == GK_MX && !g.w_fp8)) ? (int64_t)K / 2 : (int64_t)K;
  const uint8_t* w_base = g.w_codes + (int64_t)e * NW * w_rb;

  floatx4 acc[2][2][NU];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int u = 0; u < NU; ++u) acc[i][j][u] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += kBK) {
    if (GK == GK_NV) {
      // A: 16 B of E2M1 at K [k0 + 32 lg, +32), scales 2 bytes
      uint32_t ad[2][16];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint4 c = make_uint4(0u, 0u, 0u, 0u);
        uint32_t s2 = 0;
        if (a_ok[i]) {
          c = *reinterpret_cast<const uint4*>(a_ptr[i] + (k0 + 32 * lg) / 2);
          s2 = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(g.a_scales) +
                                                  (int64_t)a_row[i] * (K / 16) + (k0 + 32 * lg) / 16);
        }
        nv_decode32(c, s2, ad[i]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int wr = w_row[j][u];
          uint4 c = *reinterpret_cast<const uint4*>(w_base + (int64_t)wr * w_rb + (k0 + 32 * lg) / 2);
          uint32_t s2 = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(g.w_scales) +
                                                           ((int64_t)e * NW + wr) * (K / 16) + (k0 + 32 * lg) / 16);
          uint32_t wd[16];
          nv_decode32(c, s2, wd);
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int m = 0; m < 4; ++m)
              acc[i][j][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(&ad[i][4 * m]),
                                                                    as_half8(&wd[4 * m]), acc[i][j][u], 0, 0, 0);
        }
    } else {
      // A: E4M3 codes, K [k0+16lg, +16) and [k0+64+16lg, +16)
      intx8 av[2];
      int asc[2];
      float afs[2][4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint4 lo = make_uint4(0u, 0u, 0u, 0u), hi = make_uint4(0u, 0u, 0u, 0u);
        if (a_ok[i]) {
          lo = *reinterpret_cast<const uint4*>(a_ptr[i] + k0 + 16 * lg);
          hi = *reinterpret_cast<const uint4*>(a_ptr[i] + k0 + 64 + 16 * lg);
        }
        av[i] = intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        if (GK == GK_MX) {
          asc[i] = a_ok[i] ? reinterpret_cast<const uint8_t*>(g.a_scales)[(int64_t)a_row[i] * (K / 32) + k0 / 32 + lg] : 0;
        } else {
          asc[i] = 127;
        }
      }
      if (GK == GK_FP8) {
        // activation scale of the C rows this lane accumulates: rows 4 lg + r of subtile i
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            int rr = mt * kBM + wm * 32 + i * 16 + 4 * lg + r;
            float sa = 0.0f;
            if (rr < n_rows) {
              int R = r_begin + rr;
              int arow = g.a_gather ? g.pair_of_row[R] / g.k : R;
              sa = reinterpret_cast<const float*>(g.a_scales)[(int64_t)arow * (K / 128) + k0 / 128];
            }
            afs[i][r] = sa;
          }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int wr = w_row[j][u];
          const uint8_t* wp = w_base + (int64_t)wr * w_rb;
          intx8 bv;
          int bsc = 127;
          float wfs = 1.0f;
          if (GK == GK_MX && !g.w_fp8) {
            uint4 c = *reinterpret_cast<const uint4*>(wp + (k0 + 32 * lg) / 2);
            bv = intx8{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
          } else {
            uint4 lo = *reinterpret_cast<const uint4*>(wp + k0 + 16 * lg);
            uint4 hi = *reinterpret_cast<const uint4*>(wp + k0 + 64 + 16 * lg);
            bv = intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          }
          if (GK == GK_MX) {
            bsc = reinterpret_cast<const uint8_t*>(g.w_scales)[((int64_t)e * NW + wr) * (K / 32) + k0 / 32 + lg];
          } else {
            // one fp32 scale per 128 x 128 weight tile; the 16 rows of this subtile share it
            wfs = reinterpret_cast<const float*>(g.w_scales)[((int64_t)e * (NW / 128) + wr / 128) * (K / 128) + k0 / 128];
          }
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            if (GK == GK_MX) {
              if (g.w_fp8)
                acc[i][j][u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av[i], bv, acc[i][j][u], 0, 0, 0,
                                                                                asc[i], 0, bsc);
              else
                acc[i][j][u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av[i], bv, acc[i][j][u], 0, 4, 0,
                                                                                asc[i], 0, bsc);
            } else {
              floatx4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av[i], bv, floatx4{0.f, 0.f, 0.f, 0.f},
                                                                           0, 0, 0, 127, 0, 127);
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[i][j][u][r] = fmaf(p[r], afs[i][r] * wfs, acc[i][j][u][r]);
            }
          }
        }
    }
  }

  // epilogue
  float scale = 1.0f;
  if (GK == GK_NV) scale = g.a_tensor_scale[0] * g.w_tensor_scale[e];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = nt * kBN + wn * 32 + j * 16 + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = mt * kBM + wm * 32 + i * 16 + 4 * lg + r;
        if (rr >= n_rows) continue;
        const int64_t R = r_begin + rr;
        float v;
        if (EPI == EPI_GATEUP) {
          const float gt = acc[i][j][0][r] * scale;
          const float up = acc[i][j][NU - 1][r] * scale;
          v = silu_f32(gt) * up;
        } else {
          v = acc[i][j][0][r] * scale;
          if (g.row_scale) v *= g.row_scale[R];
        }
        g.out[R * g.N + n] = v;
      }
    }
}

// Zero rows [n_valid, P) of a [P, cols] f32 buffer (n_valid read on the device).
__global__ void zero_rows_tail_kernel(float* __restrict__ buf, const int32_t* __restrict__ n_valid, int64_t P,
                                      int cols) {
  const int64_t begin = (int64_t)n_valid[0] * cols, end = P * cols;
  for (int64_t i = begin + (int64_t)blockIdx.x * 256 + threadIdx.x; i < end; i += (int64_t)gridDim.x * 256)
    buf[i] = 0.0f;
}

// sigmoid(x_t . gate) for every token (one wave per token), bf16 x and gate.
__global__ void __launch_bounds__(256) shared_gate_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ gate, int64_t T, int H,
                                                          float* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  float acc = 0.0f;
  for (int c = lane * 8; c < H; c += 512) {
    uint4 a = *reinterpret_cast<const uint4*>(x + t * H + c);
    uint4 b = *reinterpret_cast<const uint4*>(gate + c);
    acc = dot2_bf16(a.x, b.x, acc);
    acc = dot2_bf16(a.y, b.y, acc);
    acc = dot2_bf16(a.z, b.z, acc);
    acc = dot2_bf16(a.w, b.w, acc);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) out[t] = 1.0f / (1.0f + __expf(-acc));
}

// ------------------------------------------------------------------- host

template <int GK, int EPI>
static int launch_gemm(const GemmArgs& a, int64_t tiles_m_bound, hipStream_t st) {
  const int NT = a.N / kBN;
  int64_t G = tiles_m_bound * NT;
  G = (G + 7) / 8 * 8;
  if (G <= 0) return FP4_OK;
  if (G > INT32_MAX) return fail(FP4_ERR_UNSUPPORTED, "grouped GEMM grid too large");
  const size_t lds = a.dense_rows > 0 ? 0 : sizeof(int) * ((size_t)a.E + 1);
  hipLaunchKernelGGL((grouped_gemm_kernel<GK, EPI>), dim3((unsigned)G), dim3(256), lds, st, a);
  return check_launch("grouped_gemm");
}

static int act_fmt_to_gk(int a_fmt) {
  return a_fmt == FP4_FMT_NVFP4 ? GK_NV : (a_fmt == FP4_FMT_MXFP8 ? GK_MX : GK_FP8);
}

int launch_grouped(const moe_fp4_layer* L, const uint16_t* x, int64_t T, const WsPtrs& w, int max_active,
                   hipStream_t st, const Marker& mark) {
  (void)max_active;
  const int E = L->num_experts, H = L->hidden, I = L->inter, k = L->top_k;
  const int64_t P = T * k;
  if (H % kBK || I % kBK || I % kBN || H % kBN)
    return fail(FP4_ERR_SHAPE, "grouped GEMM needs hidden and inter multiples of 128");
  const int gk = act_fmt_to_gk(L->a_fmt);
  // 2. dynamic quantization of x (NVFP4: tensor scale amax/2688 over all of x,
  //    or the caller's static scale, which the quantizer then only reads)
  const bool static_x = L->a_fmt == FP4_FMT_NVFP4 && L->input_scale;
  float* x_ts = static_x ? const_cast<float*>(L->input_scale) : w.x_ts;
  FP4_CHECK(fp4_quantize(L->a_fmt, FP4_RULE_RTN, static_x ? FP4_TS_STATIC : FP4_TS_DYNAMIC, x, FP4_DT_BF16, 1,
                         T, H, w.xq_codes, w.xq_scales, x_ts, nullptr, st));
  FP4_CHECK(mark(2));
  const int64_t tiles_bound = (P + kBM - 1) / kBM + std::min<int64_t>(E, P);
  // 3. gate_up + SiLU * up -> h
  GemmArgs a{};
  a.a_codes = w.xq_codes;
  a.a_scales = w.xq_scales;
  a.a_tensor_scale = x_ts;
  a.a_gather = 1;
  a.w_codes = L->w13;
  a.w_scales = L->w13_scale;
  a.w_tensor_scale = L->w13_scale_2;
  a.w_fp8 = 0;
  a.offsets = w.offsets;
  a.pair_of_row = w.pair_of_row;
  a.tile_offsets = w.tile_offsets;
  a.E = E;
  a.k = k;
  a.dense_rows = 0;
  a.K = H;
  a.N = I;
  a.out = w.h;
  a.row_scale = nullptr;
  if (gk == GK_NV) FP4_CHECK((launch_gemm<GK_NV, EPI_GATEUP>(a, tiles_bound, st)));
  else if (gk == GK_MX) FP4_CHECK((launch_gemm<GK_MX, EPI_GATEUP>(a, tiles_bound, st)));
  else FP4_CHECK((launch_gemm<GK_FP8, EPI_GATEUP>(a, tiles_bound, st)));
  FP4_CHECK(mark(3));
  // 4. quantization of h (sorted rows; NVFP4 tensor scale over all of h).
  //    Rows of skipped pairs (invalid expert ids) hold no h: zero them first.
  hipLaunchKernelGGL(zero_rows_tail_kernel, dim3(64), dim3(256), 0, st, w.h, w.offsets + E, P, I);
  FP4_CHECK(check_launch("zero_rows_tail"));
  const bool static_h = L->a_fmt == FP4_FMT_NVFP4 && L->inter_scale;
  float* h_ts = static_h ? const_cast<float*>(L->inter_scale) : w.h_ts;
  FP4_CHECK(fp4_quantize(L->a_fmt, FP4_RULE_RTN, static_h ? FP4_TS_STATIC : FP4_TS_DYNAMIC, w.h, FP4_DT_F32, 1,
                         P, I, w.hq_codes, w.hq_scales, h_ts, nullptr, st));
  FP4_CHECK(mark(4));
  // 5. down -> o
  GemmArgs d = a;
  d.a_codes = w.hq_codes;
  d.a_scales = w.hq_scales;
  d.a_tensor_scale = h_ts;
  d.a_gather = 0;
  d.w_codes = L->w2;
  d.w_scales = L->w2_scale;
  d.w_tensor_scale = L->w2_scale_2;
  d.K = I;
  d.N = H;
  d.out = w.o;
  if (gk == GK_NV) FP4_CHECK((launch_gemm<GK_NV, EPI_DOWN>(d, tiles_bound, st)));
  else if (gk == GK_MX) FP4_CHECK((launch_gemm<GK_MX, EPI_DOWN>(d, tiles_bound, st)));
  else FP4_CHECK((launch_gemm<GK_FP8, EPI_DOWN>(d, tiles_bound, st)));
  return mark(5);
}

int launch_shared_expert(const moe_fp4_layer* L, const uint16_t* x, int64_t T, const WsPtrs& w,
                         hipStream_t st) {
  const int H = L->hidden, S = L->shared_inter;
  if (H % kBK || S % kBK || S % kBN || H % kBN)
    return fail(FP4_ERR_SHAPE, "shared expert needs widths that are multiples of 128");
  FP4_CHECK(fp4_quantize(FP4_FMT_MXFP8, FP4_RULE_RTN, FP4_TS_DYNAMIC, x, FP4_DT_BF16, 1, T, H, w.sx_codes,
                         w.sx_scales, nullptr, nullptr, st));
  const int64_t tiles = (T + kBM - 1) / kBM;
  GemmArgs a{};
  a.a_codes = w.sx_codes;
  a.a_scales = w.sx_scales;
  a.a_gather = 0;
  a.w_codes = L->ws13;
  a.w_scales = L->ws13_scale;
  a.w_fp8 = 1;
  a.E = 1;
  a.k = 1;
  a.dense_rows = (int)T;
  a.K = H;
  a.N = S;
  a.out = w.sh;
  FP4_CHECK((launch_gemm<GK_MX, EPI_GATEUP>(a, tiles, st)));
  FP4_CHECK(fp4_quantize(FP4_FMT_MXFP8, FP4_RULE_RTN, FP4_TS_DYNAMIC, w.sh, FP4_DT_F32, 1, T, S, w.sh_codes,
                         w.sh_scales, nullptr, nullptr, st));
  // per-token gate into the (now free) f32 h region of the shared expert
  float* g_t = w.sh;
  hipLaunchKernelGGL(shared_gate_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, x, L->shared_gate, T, H,
                     g_t);
  FP4_CHECK(check_launch("shared_gate"));
  GemmArgs d{};
  d.a_codes = w.sh_codes;
  d.a_scales = w.sh_scales;
  d.a_gather = 0;
  d.w_codes = L->ws2;
  d.w_scales = L->ws2_scale;
  d.w_fp8 = 1;
  d.E = 1;
  d.k = 1;
  d.dense_rows = (int)T;
  d.K = S;
  d.N = H;
  d.out = w.s_out;
  d.row_scale = g_t;
  FP4_CHECK((launch_gemm<GK_MX, EPI_DOWN>(d, tiles, st)));
  return FP4_OK;
}

}  // namespace fp4
