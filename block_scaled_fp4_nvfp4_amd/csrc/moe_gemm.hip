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
// share its L2.  The register-fed down projections of large batches give a
// workgroup several consecutive output tiles of its rows: their activation
// tile (K = inter, short) is loaded into LDS once for all of them.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <utility>

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

// LDS rows hold 16-byte chunks in XOR-swizzled order so that the MFMA
// fragment reads (16 lanes read the same chunk of 16 consecutive rows) and
// the staging writes (consecutive lanes write consecutive chunks of a few
// rows) touch distinct 16-byte bank groups within every 8 lanes and within
// every 16 lanes.  Row widths: 64 B (4 chunks), 128 B (8), 256 B (16).
template <int ROW_BYTES>
__device__ __forceinline__ int swz(int row, int chunk) {
  if (ROW_BYTES == 64) return row * 64 + 16 * (chunk ^ (((row >> 1) ^ (row >> 3)) & 3));
  if (ROW_BYTES == 128) return row * 128 + 16 * (chunk ^ ((row ^ (row >> 3)) & 7));
  return row * 256 + 16 * (chunk ^ (row & 15));
}

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
  // down: when set, o leaves the epilogue here as fp16 (rounded to nearest
  // even from the f32 accumulator) and `out` is not written
  _Float16* out_f16;
  const float* row_scale;       // down epilogue: per-row multiplier (shared-expert gate), may be null
  // MX gate_up on 128-output tiles only (grouped_gemm_mx_kernel<EPI_GATEUP, 2>):
  // when set, h leaves the epilogue as MXFP8 (E4M3 codes [rows][N], UE8M0
  // scales [rows][N/32]) and `out` is not written
  uint8_t* q_codes;
  uint8_t* q_scales;
  // NVFP4 gate_up: when set, workgroup i of the amax_nparts launched writes
  // max |h| over the h values it stores to amax_part[i] (0 if it has no
  // tile), for the tensor scale of h
  float* amax_part;
  int64_t amax_nparts;
  // MX gate_up (grouped_gemm_mx_kernel): w_codes / w_scales are in the tiled
  // order of moe_fp4_tile_weights
  int w_tiled;
};

// One value of an epilogue: h or o in f32, or o in fp16 where the caller
// asked for it.
template <int EPI>
__device__ __forceinline__ void store_out(const GemmArgs& g, int64_t idx, float v) {
  if (EPI == EPI_DOWN && g.out_f16) g.out_f16[idx] = (_Float16)v;
  else g.out[idx] = v;
}

// Tile of this workgroup among n_tiles real (row block, output group) tiles.
// Workgroups are dispatched to the 8 XCDs in turn (workgroup i to XCD i % 8);
// XCD x takes the contiguous range [x per, (x + 1) per), per = ceil(n_tiles /
// 8), so an expert's consecutive tiles share that XCD's L2, and the
// workgroups beyond the real tiles (the grid is sized by a bound on the tile
// count) are spread over all XCDs instead of leaving the last ones idle.
// -1: no tile.
__device__ __forceinline__ int xcd_tile(int n_tiles) {
  const int per = (n_tiles + 7) / 8;
  const int k = blockIdx.x / 8;
  const int L = (blockIdx.x % 8) * per + k;
  return k < per && L < n_tiles ? L : -1;
}

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
//
// One workgroup = 4 waves computes a 64-row x (64 * NSUB)-output tile of one
// expert.  All waves share the tile's 64 activation rows; wave w owns outputs
// [16 NSUB w, 16 NSUB (w+1)) of the tile (for gate_up: those gate rows and the
// matching up rows).  Per 128-wide K step the workgroup stages the packed
// operands and their scales in LDS (double buffered: the next step's global
// loads are in flight while the current step's MFMAs run); NVFP4 activations
// are decoded to fp16 once, on their way into LDS.

template <int GK, int EPI, int NSUB, bool WFP8>
struct TileCfg {
  static constexpr int BM = kBM;
  static constexpr int BN = 64 * NSUB;                              // outputs per tile
  static constexpr int NU = EPI == EPI_GATEUP ? 2 : 1;
  static constexpr int WROWS = NU * BN;                             // weight rows per tile
  static constexpr int W_STRIDE = WFP8 ? 128 : 64;                 // weight row in LDS (bytes)
  static constexpr int W_CPR = WFP8 ? 8 : 4;                        // 16-byte chunks per row per K step
  static constexpr int A_BYTES = GK == GK_NV ? 256 : 128;           // per row per K step in LDS
  static constexpr int A_STRIDE = A_BYTES;
  static constexpr int W_SCALE_BYTES = GK == GK_NV ? 8 : 4;        // per row per K step
  static constexpr int A_SCALE_BYTES = 4;
  static constexpr size_t STAGE =
      ((size_t)BM * A_STRIDE + (size_t)BM * A_SCALE_BYTES + (size_t)WROWS * W_STRIDE + (size_t)WROWS * W_SCALE_BYTES +
       15) / 16 * 16;
};

template <int GK, int EPI, int NSUB, bool WFP8, bool WT>
__global__ void __launch_bounds__(256) grouped_gemm_kernel(GemmArgs g) {
  static_assert(!WT || (GK == GK_NV && !WFP8), "tiled weights on this kernel: NVFP4");
  using C = TileCfg<GK, EPI, NSUB, WFP8>;
  constexpr int BM = C::BM, BN = C::BN, NU = C::NU, WROWS = C::WROWS;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr bool w_fp8 = WFP8;
  constexpr int w_stride = C::W_STRIDE;
  constexpr int w_cpr = C::W_CPR;
  constexpr size_t stage = C::STAGE;
  int* s_toff = reinterpret_cast<int*>(lds + 2 * stage);

  const int NT = g.N / BN;

  int L, e, mt, nt, r_begin, n_rows;
  if (g.dense_rows > 0) {
    e = 0;
    L = xcd_tile((g.dense_rows + BM - 1) / BM * NT);
    if (L < 0) return;
    nt = L % NT;
    mt = L / NT;
    r_begin = 0;
    n_rows = g.dense_rows;
  } else {
    for (int i = threadIdx.x; i <= g.E; i += 256) s_toff[i] = g.tile_offsets[i];
    __syncthreads();
    L = xcd_tile(s_toff[g.E] * NT);
    if (L < 0) {
      if (GK == GK_NV && EPI == EPI_GATEUP && g.amax_part && threadIdx.x == 0) g.amax_part[blockIdx.x] = 0.0f;
      return;
    }
    nt = L % NT;
    const int mg = L / NT;
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

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int K = g.K;
  const int KS = K / kBK;
  const int NW = NU * g.N;  // weight rows per expert
  const int64_t a_rb = GK == GK_NV ? (int64_t)K / 2 : (int64_t)K;
  const int64_t w_rb = w_fp8 ? (int64_t)K : (int64_t)K / 2;
  const uint8_t* w_base = g.w_codes + (int64_t)e * NW * w_rb;

  auto a_row_of = [&](int r, bool& ok) __attribute__((always_inline)) -> int {
    const int rr = mt * BM + r;
    ok = rr < n_rows;
    const int R = r_begin + (ok ? rr : 0);
    return g.a_gather ? g.pair_of_row[R] / g.k : R;
  };
  auto w_grow = [&](int i) __attribute__((always_inline)) -> int { return (i / BN) * g.N + nt * BN + (i % BN); };

  // ---- per-thread global load assignments (fixed across K steps).  Rows
  // past the expert's end load row 0 of the expert instead: MFMA rows are
  // independent and those rows are never stored, so no load is predicated
  // and the K loop body stays one basic block.
  // A: MX/FP8 2 chunks of 16 B (rows tid/8 and 32 + tid/8); NV 1 chunk (row tid/4)
  constexpr int A_CH = GK == GK_NV ? 1 : 2;
  const uint8_t* a_src[A_CH];
  const uint8_t* an_src[A_CH];
  int a_lrow[A_CH], a_part[A_CH];
#pragma unroll
  for (int c = 0; c < A_CH; ++c) {
    const int ch = tid + 256 * c;
    const int r = GK == GK_NV ? ch / 4 : ch / 8;
    a_lrow[c] = r;
    a_part[c] = GK == GK_NV ? ch % 4 : ch % 8;
    bool ok;
    const int64_t arow = a_row_of(r, ok);
    a_src[c] = g.a_codes + arow * a_rb + (GK == GK_NV ? 16 * a_part[c] : 16 * a_part[c]);
    an_src[c] = reinterpret_cast<const uint8_t*>(g.a_scales) + arow * (K / 16) + 2 * a_part[c];
  }
  // A scales (MX: 4 bytes, FP8: one float per row per K step): every thread
  // loads the scale of row tid % 64 (the four waves store identical values)
  const int as_lrow = tid & (BM - 1);
  int64_t as_row = 0;
  {
    bool ok;
    as_row = a_row_of(as_lrow, ok);
  }
  // W: WROWS * w_cpr chunks of 16 B, a multiple of 256
  constexpr int W_CH = WROWS * w_cpr / 256;
  static_assert(WROWS * w_cpr % 256 == 0, "weight tile must split evenly over 256 threads");
  const uint8_t* w_src[W_CH];
  int w_soff[W_CH];
#pragma unroll
  for (int c = 0; c < W_CH; ++c) {
    const int ch = tid + 256 * c;
    const int row = ch / w_cpr, part = ch % w_cpr;
    const int gr = w_grow(row);
    // tiled (moe_fp4_tile_weights): a wave's 16 rows (aligned) of a step are one kilobyte
    w_src[c] = WT ? w_base + (int64_t)(gr >> 4) * (KS * 1024) + (gr & 15) * 64 + 16 * part
                  : w_base + (int64_t)gr * w_rb + 16 * part;
    w_soff[c] = swz<w_stride>(row, part);
  }
  // W scales: row tid % WROWS (WROWS <= 256; duplicates store identical values)
  static_assert(WROWS <= 256 && (WROWS & (WROWS - 1)) == 0, "weight rows per tile");
  const int ws_lrow = tid & (WROWS - 1);
  const int64_t ws_grow = w_grow(ws_lrow);

  // One K step's operands on their way from global memory to LDS.
  struct Stage {
    u32x4 pa[A_CH];
    uint32_t pas;            // A scales (MX dword / FP8 float bits)
    uint32_t pan[A_CH];      // NV A scale pairs
    u32x4 pw[W_CH];
    u32x2 pws;
  };

  auto load_step = [&](Stage& R, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < A_CH; ++c) {
      if (GK == GK_NV) {
        R.pa[c] = ld16(a_src[c] + k0 / 2);
        R.pan[c] = *reinterpret_cast<const uint16_t*>(an_src[c] + k0 / 16);
      } else {
        R.pa[c] = ld16(a_src[c] + k0);
      }
    }
    if (GK == GK_MX)
      R.pas = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(g.a_scales) + as_row * (K / 32) +
                                                 k0 / 32);
    if (GK == GK_FP8)
      R.pas = __float_as_uint(reinterpret_cast<const float*>(g.a_scales)[as_row * (K / 128) + k0 / 128]);
#pragma unroll
    for (int c = 0; c < W_CH; ++c) R.pw[c] = ld16(w_src[c] + (WT ? k0 * 8 : (WFP8 ? k0 : k0 / 2)));
    if (GK == GK_NV && WT) {  // tiled: 16 rows' 8 scale bytes of a step as 128 bytes
      R.pws = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(g.w_scales) +
                                              (int64_t)e * NW * (K / 16) + (int64_t)(ws_grow >> 4) * (KS * 128) +
                                              k0 + (ws_grow & 15) * 8);
    } else if (GK == GK_NV) {
      R.pws = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(g.w_scales) +
                                              ((int64_t)e * NW + ws_grow) * (K / 16) + k0 / 16);
    } else if (GK == GK_MX) {
      R.pws.x = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(g.w_scales) +
                                                   ((int64_t)e * NW + ws_grow) * (K / 32) + k0 / 32);
    } else {
      R.pws.x = __float_as_uint(reinterpret_cast<const float*>(g.w_scales)[
          ((int64_t)e * (NW / 128) + ws_grow / 128) * (K / 128) + k0 / 128]);
    }
  };

  auto store_step = [&](const Stage& R, int buf) __attribute__((always_inline)) {
    uint8_t* sb = lds + buf * stage;
    uint8_t* s_a = sb;
    uint8_t* s_as = sb + BM * C::A_STRIDE;
    uint8_t* s_w = s_as + BM * C::A_SCALE_BYTES;
    uint8_t* s_ws = s_w + WROWS * w_stride;
#pragma unroll
    for (int c = 0; c < A_CH; ++c) {
      if (GK == GK_NV) {
        uint32_t d[16];
        nv_decode32(make_uint4(R.pa[c].x, R.pa[c].y, R.pa[c].z, R.pa[c].w), R.pan[c], d);
        const int r = a_lrow[c], c0 = 4 * a_part[c];
        st16(s_a + swz<256>(r, c0), u32x4{d[0], d[1], d[2], d[3]});
        st16(s_a + swz<256>(r, c0 + 1), u32x4{d[4], d[5], d[6], d[7]});
        st16(s_a + swz<256>(r, c0 + 2), u32x4{d[8], d[9], d[10], d[11]});
        st16(s_a + swz<256>(r, c0 + 3), u32x4{d[12], d[13], d[14], d[15]});
      } else {
        st16(s_a + swz<128>(a_lrow[c], a_part[c]), R.pa[c]);
      }
    }
    if (GK != GK_NV) reinterpret_cast<uint32_t*>(s_as)[as_lrow] = R.pas;
#pragma unroll
    for (int c = 0; c < W_CH; ++c) st16(s_w + w_soff[c], R.pw[c]);
    if (GK == GK_NV) reinterpret_cast<u32x2*>(s_ws)[ws_lrow] = R.pws;
    else reinterpret_cast<uint32_t*>(s_ws)[ws_lrow] = R.pws.x;
  };

  floatx4 acc[4][NU * NSUB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int s = 0; s < NU * NSUB; ++s) acc[i][s] = floatx4{0.f, 0.f, 0.f, 0.f};

  // LDS row (within the tile's weight rows) of this wave's subtile s
  auto w_lrow = [&](int s) __attribute__((always_inline)) -> int {
    const int u = s / NSUB, j = s % NSUB;
    return u * BN + wave * 16 * NSUB + j * 16 + lr;
  };

  auto compute_step = [&](int buf) __attribute__((always_inline)) {
    const uint8_t* sb = lds + buf * stage;
    const uint8_t* s_a = sb;
    const uint8_t* s_as = sb + BM * C::A_STRIDE;
    const uint8_t* s_w = s_as + BM * C::A_SCALE_BYTES;
    const uint8_t* s_ws = s_w + WROWS * w_stride;
    if (GK == GK_NV) {
      uint32_t af[4][16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 v = ld16(s_a + swz<256>(16 * i + lr, 4 * lg + q));
          af[i][4 * q] = v.x; af[i][4 * q + 1] = v.y; af[i][4 * q + 2] = v.z; af[i][4 * q + 3] = v.w;
        }
      }
      // all of this step's fragments are read before the first MFMA, so the
      // LDS latency is paid once per step
      u32x4 wc[NU * NSUB];
      uint32_t ws2[NU * NSUB];
#pragma unroll
      for (int s = 0; s < NU * NSUB; ++s) {
        const int wr = w_lrow(s);
        wc[s] = ld16(s_w + swz<w_stride>(wr, lg));
        ws2[s] = *reinterpret_cast<const uint16_t*>(s_ws + wr * 8 + 2 * lg);
      }
#pragma unroll
      for (int s = 0; s < NU * NSUB; ++s) {
        uint32_t wd[16];
        nv_decode32(make_uint4(wc[s].x, wc[s].y, wc[s].z, wc[s].w), ws2[s], wd);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int m = 0; m < 4; ++m)
            acc[i][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(&af[i][4 * m]), as_half8(&wd[4 * m]),
                                                               acc[i][s], 0, 0, 0);
      }
    } else {
      intx8 af[4];
      int asc[4];
      float afs[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 lo = ld16(s_a + swz<128>(16 * i + lr, lg));
        const u32x4 hi = ld16(s_a + swz<128>(16 * i + lr, 4 + lg));
        af[i] = intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        if (GK == GK_MX) asc[i] = s_as[(16 * i + lr) * 4 + lg];
        if (GK == GK_FP8) {
#pragma unroll
          for (int r = 0; r < 4; ++r) afs[i][r] = reinterpret_cast<const float*>(s_as)[16 * i + 4 * lg + r];
        }
      }
      intx8 bv[NU * NSUB];
      int bsc[NU * NSUB];
      float wfs[NU * NSUB];
#pragma unroll
      for (int s = 0; s < NU * NSUB; ++s) {
        const int wr = w_lrow(s);
        if (w_fp8) {
          const u32x4 lo = ld16(s_w + swz<w_stride>(wr, lg));
          const u32x4 hi = ld16(s_w + swz<w_stride>(wr, 4 + lg));
          bv[s] = intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        } else {
          const u32x4 c = ld16(s_w + swz<w_stride>(wr, lg));
          bv[s] = intx8{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
        }
        if (GK == GK_MX) bsc[s] = s_ws[wr * 4 + lg];
        else wfs[s] = reinterpret_cast<const float*>(s_ws)[wave * 16 * NSUB + (s % NSUB) * 16 + (s / NSUB) * BN];
      }
      // all of this step's fragments are read before the first MFMA, so the
      // LDS latency is paid once per step
#pragma unroll
      for (int s = 0; s < NU * NSUB; ++s) {
        if (GK == GK_MX) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (w_fp8)
              acc[i][s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bv[s], acc[i][s], 0, 0, 0, asc[i],
                                                                           0, bsc[s]);
            else
              acc[i][s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bv[s], acc[i][s], 0, 4, 0, asc[i],
                                                                           0, bsc[s]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const floatx4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                af[i], bv[s], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][s][r] = fmaf(p[r], afs[i][r] * wfs[s], acc[i][s][r]);
          }
        }
      }
    }
  };

  // Pin this step's accumulators before the LDS stores that follow: without
  // the empty asm uses the compiler sinks the MFMAs below the stores (and
  // their vmcnt wait), and every step then exposes the full load latency.
  // Accumulators live in AGPRs except on the FP8 path, which rescales them
  // with VALU FMAs.
  auto pin_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int s = 0; s < NU * NSUB; ++s) {
        if (GK == GK_FP8) asm volatile("" ::"v"(acc[i][s]));
        else asm volatile("" ::"a"(acc[i][s]));
      }
    __builtin_amdgcn_sched_barrier(0);
  };

  // K loop over two LDS buffers: step ks is computed from buffer ks&1 while
  // the global loads of step ks+1 (issued at the end of the previous step)
  // are in flight; they are stored to the other buffer once this step's
  // MFMAs have been issued.  (A second register stage, to issue loads two
  // steps ahead, measured no faster and costs occupancy.)
  Stage R;
  load_step(R, 0);
  store_step(R, 0);
  __syncthreads();
  if (KS > 1) load_step(R, kBK);
  for (int ks = 0; ks < KS; ++ks) {
    compute_step(ks & 1);
    if (ks + 1 < KS) {
      pin_acc();
      store_step(R, (ks + 1) & 1);
      __syncthreads();
      if (ks + 2 < KS) load_step(R, (ks + 2) * kBK);
    }
  }

  // ---- epilogue
  float scale = 1.0f;
  if (GK == GK_NV) scale = g.a_tensor_scale[0] * g.w_tensor_scale[e];
  float vmax = 0.0f;  // max |h| stored by this lane (NVFP4 gate_up)
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
      const int n = nt * BN + wave * 16 * NSUB + j * 16 + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = mt * BM + 16 * i + 4 * lg + r;
        if (rr >= n_rows) continue;
        const int64_t R = r_begin + rr;
        float v;
        if (EPI == EPI_GATEUP) {
          v = silu_f32(acc[i][j][r] * scale) * (acc[i][NSUB + j][r] * scale);
          vmax = fmaxf(vmax, fabsf(v));
        } else {
          v = acc[i][j][r] * scale;
          if (g.row_scale) v *= g.row_scale[R];
        }
        store_out<EPI>(g, R * g.N + n, v);
      }
    }
  if constexpr (GK == GK_NV && EPI == EPI_GATEUP) {
    if (g.amax_part) {
      // max is exact in any order, so the tensor amax is the one a separate
      // pass over h would find
      __shared__ float red[4];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, off));
      if (lane == 0) red[wave] = vmax;
      __syncthreads();
      if (tid == 0) g.amax_part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    }
  }
}

// h of an MX gate_up tile straight to MXFP8.  With 128-output tiles a wave's
// 32 outputs of a row are one block of 32 (two 16-column subtiles), so the
// block amax is a max over the lane's two values and its 15 partner lanes;
// exponent and codes as the standalone MXFP8 quantizer takes them (the max
// is exact in any order, and the power-of-two scaling makes each convert
// exact).  acc[i][j] holds gate and acc[i][2 + j] up of subtile j for rows
// row0 + 16 i + 4 lg + r (r the accumulator element), column 16 j + lr of
// the block; blk is the block's index within the row.
__device__ __forceinline__ void store_h_mxfp8(const GemmArgs& g, const floatx4 (&acc)[4][4], int blk, int row0,
                                              int n_rows, int64_t r_begin, int lg, int lr) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) v[j] = silu_f32(acc[i][j][r]) * acc[i][2 + j][r];
      float amax = fmaxf(fabsf(v[0]), fabsf(v[1]));
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
      const int ex = mx_exponent(amax, kE4M3Max);
      const int rr = row0 + 16 * i + 4 * lg + r;
      if (rr >= n_rows) continue;
      const int64_t R = r_begin + rr;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t c = e4m3_hw(fminf(ldexpf(fabsf(v[j]), -ex), kE4M3Max)) |
                           ((__float_as_uint(v[j]) >> 24) & 0x80u);
        g.q_codes[R * g.N + 32 * blk + 16 * j + lr] = (uint8_t)c;
      }
      if (lr == 0) g.q_scales[R * (g.N / 32) + blk] = (uint8_t)(ex + 127);
    }
}

// h of a block-FP8 gate_up tile (128 outputs: 4 waves x 2 subtiles x 16)
// straight to FP8 with one f32 scale per (row, 128 outputs), as
// quant_fp8_row_kernel takes them from the f32 h: the row's amax over the
// tile's 128 values (16-lane shuffles within a wave, then the four waves
// through LDS; max is exact in any order), sigma = fp32(amax / 448), the
// exact E4M3 code of |v| / sigma and the sign of v (sigma 0: signed zeros).
// acc[i][j] holds gate and acc[i][2 + j] up of subtile j for rows
// row0 + 16 i + 4 lg + r, column 16 j + lr of the wave's 32; nt is the tile's
// 128-output block.
__device__ __forceinline__ void store_h_fp8row(const GemmArgs& g, const floatx4 (&acc)[4][4], int nt, int row0,
                                               int n_rows, int64_t r_begin, int wave, int lg, int lr) {
  __shared__ float s_amax[4][64];
  float v[4][4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int j = 0; j < 2; ++j) v[i][r][j] = silu_f32(acc[i][j][r]) * acc[i][2 + j][r];
      float m = fmaxf(fabsf(v[i][r][0]), fabsf(v[i][r][1]));
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 16));
      if (lr == 0) s_amax[wave][16 * i + 4 * lg + r] = m;
    }
  __syncthreads();
  const int64_t N = g.N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * i + 4 * lg + r;
      const float amax = fmaxf(fmaxf(s_amax[0][row], s_amax[1][row]), fmaxf(s_amax[2][row], s_amax[3][row]));
      const float sigma = (float)((double)amax / 448.0);
      const float sg = sigma > 0.0f ? sigma : 1.0f;
      const int rr = row0 + row;
      if (rr >= n_rows) continue;
      const int64_t R = r_begin + rr;
      // codes of |v| r (1 -/+ 2^-20) with r ~ 1/sigma within 2^-23 bracket
      // the code of the exact quotient; where they agree it is that code,
      // else the exact quotient decides (as in the standalone quantizer)
      // (sigma below 2^-120, where 1/sigma nears the float range, always exact)
      const bool rok = sg >= 0x1p-120f;
      const float r0 = rok ? __builtin_amdgcn_rcpf(sg) : 0.0f;
      const float rc = fmaf(r0, fmaf(-sg, r0, 1.0f), r0);
      const float rl = rc * 0x1.ffffe0p-1f, rh = rc * 0x1.000010p+0f;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float a = fabsf(v[i][r][j]);
        uint32_t c = e4m3_hw(fminf(a * rl, kE4M3Max));
        if (!rok || c != e4m3_hw(fminf(a * rh, kE4M3Max))) c = e4m3_exact_quotient(a, sg);
        c = (sigma > 0.0f ? c : 0u) | ((__float_as_uint(v[i][r][j]) >> 24) & 0x80u);
        g.q_codes[R * N + 128 * nt + 32 * wave + 16 * j + lr] = (uint8_t)c;
      }
      if (wave == 0 && lr == 0) reinterpret_cast<float*>(g.q_scales)[R * (N / 128) + nt] = sigma;
    }
}

// ------------------------------------------- MX path with LDS-DMA staging
//
// MXFP4 weights x MXFP8 activations.  Same tile as above (64 rows x 64*NSUB
// outputs, 4 waves, 16 MFMAs of 16x16x128 per wave and step), but the
// operands go from global memory straight into LDS (global_load_lds: lane l
// of a DMA instruction writes LDS bytes base + 16 l .. + 15) through a ring
// of three stages, so the loads of step ks+2 are in flight while step ks is
// computed and no registers are spent on staging.  Each stage holds
// [A 64 x 128 B | W WROWS x 64 B | A scales 64 dwords | W scales WROWS
// dwords]; A and W rows keep the XOR-swizzled chunk order (a lane fetches
// the global chunk that belongs in the LDS slot its lane number selects).
// Every thread issues the same number of DMA instructions per step, so one
// wait for vmcnt <= N_INS before the step's barrier completes its own
// instructions for the step about to be read; the barrier then covers the
// other waves' instructions.  With WT the weights are in the tiled order of
// moe_fp4_tile_weights: a W instruction, which covers 16 consecutive rows of
// one K step, then reads one contiguous kilobyte (row-major: sixteen 64-byte
// pieces 2 KB apart at the model's hidden size), and the 64 W scale lanes
// read four 64-byte runs.
template <int EPI, int NSUB>
struct MxCfg {
  static constexpr int BM = kBM;
  static constexpr int BN = 64 * NSUB;
  static constexpr int NU = EPI == EPI_GATEUP ? 2 : 1;
  static constexpr int WROWS = NU * BN;
  static constexpr int A_BYTES = BM * 128;
  static constexpr int W_BYTES = WROWS * 64;
  static constexpr int A_INS = A_BYTES / 4096;  // 16-byte DMA instructions per thread per step
  static constexpr int W_INS = W_BYTES / 4096;
  static constexpr int SC_DW = BM + WROWS;      // scale dwords per step
  static constexpr int S_INS = (SC_DW + 255) / 256;  // 4-byte DMA instructions per thread per step
  static constexpr int N_INS = A_INS + W_INS + S_INS;
  static constexpr int STAGE = A_BYTES + W_BYTES + SC_DW * 4;
  static_assert(A_BYTES % 4096 == 0 && W_BYTES % 4096 == 0 && SC_DW % 64 == 0, "DMA tiling");
};

// One DMA instruction: lane l copies 16 (4) bytes from its global address to
// LDS address lds + 16 l (lds + 4 l).
__device__ __forceinline__ void dma16_to_lds(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4_to_lds(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}


template <int EPI, int NSUB, bool WT>
__global__ void __launch_bounds__(256, 2) grouped_gemm_mx_kernel(GemmArgs g) {
  using C = MxCfg<EPI, NSUB>;
  constexpr int BM = C::BM, BN = C::BN, NU = C::NU, WROWS = C::WROWS;
  __shared__ __attribute__((aligned(16))) uint8_t st0[C::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[C::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st2[C::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t dummy[256];  // target of the unused scale DMA lanes
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
  int* s_toff = reinterpret_cast<int*>(lds_dyn);

  const int NT = g.N / BN;

  int L, e, mt, nt, r_begin, n_rows;
  if (g.dense_rows > 0) {
    e = 0;
    L = xcd_tile((g.dense_rows + BM - 1) / BM * NT);
    if (L < 0) return;
    nt = L % NT;
    mt = L / NT;
    r_begin = 0;
    n_rows = g.dense_rows;
  } else {
    for (int i = threadIdx.x; i <= g.E; i += 256) s_toff[i] = g.tile_offsets[i];
    __syncthreads();
    L = xcd_tile(s_toff[g.E] * NT);
    if (L < 0) return;
    nt = L % NT;
    const int mg = L / NT;
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

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int K = g.K;
  const int KS = K / kBK;
  const int NW = NU * g.N;
  const int SKB = K / 32;  // scale bytes per row (one UE8M0 per 32)
  const uint8_t* w_base = g.w_codes + (int64_t)e * NW * (K / 2);

  // rows past the expert's end fetch row 0 of the expert (never stored)
  auto a_row_of = [&](int r) __attribute__((always_inline)) -> int64_t {
    const int rr = mt * BM + r;
    const int R = r_begin + (rr < n_rows ? rr : 0);
    return g.a_gather ? g.pair_of_row[R] / g.k : R;
  };
  auto w_grow = [&](int i) __attribute__((always_inline)) -> int { return (i / BN) * g.N + nt * BN + (i % BN); };
  // offsets within the expert of weight row gr's K-step-0 code piece and
  // scale dword, and what one K step adds to them
  constexpr int W_STEP = WT ? 1024 : 64, WS_STEP = WT ? 64 : 4;
  auto w_code_at = [&](int gr) __attribute__((always_inline)) -> int64_t {
    return WT ? (int64_t)(gr >> 4) * (KS * 1024) + (gr & 15) * 64 : (int64_t)gr * (K / 2);
  };
  auto w_scale_at = [&](int gr) __attribute__((always_inline)) -> int64_t {
    return WT ? (int64_t)(gr >> 4) * (KS * 64) + (gr & 15) * 4 : (int64_t)gr * SKB;
  };

  // global source of this lane for each DMA instruction (K step 0); the step
  // advances A by 128 bytes, W by W_STEP bytes, the A scales by 4 bytes and
  // the W scales by WS_STEP bytes
  const uint8_t* a_src[C::A_INS];
  const uint8_t* w_src[C::W_INS];
  const uint8_t* s_src[C::S_INS];
#pragma unroll
  for (int q = 0; q < C::A_INS; ++q) {
    const int row = (q * 4 + wave) * 8 + (lane >> 3), slot = lane & 7;
    const int chunk = slot ^ ((row ^ (row >> 3)) & 7);  // inverse of swz<128>
    a_src[q] = g.a_codes + a_row_of(row) * K + 16 * chunk;
  }
#pragma unroll
  for (int q = 0; q < C::W_INS; ++q) {
    const int row = (q * 4 + wave) * 16 + (lane >> 2), slot = lane & 3;
    const int chunk = slot ^ (((row >> 1) ^ (row >> 3)) & 3);  // inverse of swz<64>
    w_src[q] = w_base + w_code_at(w_grow(row)) + 16 * chunk;
  }
#pragma unroll
  for (int q = 0; q < C::S_INS; ++q) {
    const int d = (q * 4 + wave) * 64 + lane;
    if (d < BM)
      s_src[q] = reinterpret_cast<const uint8_t*>(g.a_scales) + a_row_of(d) * SKB;
    else if (d < C::SC_DW)
      s_src[q] = reinterpret_cast<const uint8_t*>(g.w_scales) + (int64_t)e * NW * SKB + w_scale_at(w_grow(d - BM));
    else
      s_src[q] = reinterpret_cast<const uint8_t*>(g.a_scales) + a_row_of(0) * SKB;
  }
  // K-step advance of scale lane (q, lane): W scale lanes move WS_STEP bytes
  auto s_step = [&](int q) __attribute__((always_inline)) -> int {
    if constexpr (!WT) return 4;
    const int d = (q * 4 + wave) * 64 + lane;
    return d >= BM && d < C::SC_DW ? WS_STEP : 4;
  };

  // ks < 0: the same instructions all read one 16-byte line (a stage that is
  // never read again is refilled with it), so every step issues N_INS DMA
  // instructions without moving data
  auto dma_step = [&](uint8_t* st, int ks) __attribute__((always_inline)) {
    const bool real = ks >= 0;
#pragma unroll
    for (int q = 0; q < C::A_INS; ++q)
      dma16_to_lds(real ? a_src[q] + ks * 128 : g.a_codes, st + (q * 4 + wave) * 1024);
#pragma unroll
    for (int q = 0; q < C::W_INS; ++q)
      dma16_to_lds(real ? w_src[q] + ks * W_STEP : g.a_codes, st + C::A_BYTES + (q * 4 + wave) * 1024);
#pragma unroll
    for (int q = 0; q < C::S_INS; ++q) {
      const int d0 = (q * 4 + wave) * 64;
      uint8_t* dst = d0 < C::SC_DW ? st + C::A_BYTES + C::W_BYTES + d0 * 4 : dummy;
      dma4_to_lds(real ? s_src[q] + ks * s_step(q) : g.a_codes, dst);
    }
  };

  floatx4 acc[4][NU * NSUB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int s = 0; s < NU * NSUB; ++s) acc[i][s] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto compute_step = [&](const uint8_t* st) __attribute__((always_inline)) {
    const uint8_t* s_a = st;
    const uint8_t* s_w = st + C::A_BYTES;
    const uint8_t* s_as = st + C::A_BYTES + C::W_BYTES;
    const uint8_t* s_ws = s_as + BM * 4;
    intx8 af[4];
    int asc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 lo = ld16(s_a + swz<128>(16 * i + lr, lg));
      const u32x4 hi = ld16(s_a + swz<128>(16 * i + lr, 4 + lg));
      af[i] = intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      asc[i] = s_as[(16 * i + lr) * 4 + lg];
    }
#pragma unroll
    for (int s = 0; s < NU * NSUB; ++s) {
      const int wr = (s / NSUB) * BN + wave * 16 * NSUB + (s % NSUB) * 16 + lr;
      const u32x4 c = ld16(s_w + swz<64>(wr, lg));
      const intx8 bv = intx8{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
      const int bsc = s_ws[wr * 4 + lg];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[i][s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bv, acc[i][s], 0, 4, 0, asc[i], 0, bsc);
    }
  };

  // one step: wait for this thread's DMAs of the stage to be read (the
  // next step's DMAs may stay in flight), barrier
  // (everyone's DMAs done, everyone done reading the stage about to be
  // refilled), refill the stage two steps ahead, compute
  auto step = [&](const uint8_t* cur, uint8_t* refill, int ks) __attribute__((always_inline)) {
    // own DMAs done; own LDS reads of the previous step done
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(C::N_INS));
    // a bare barrier that the compiler cannot move memory operations across
    // (a fenced __syncthreads would also wait for every DMA in flight)
    asm volatile("s_barrier" ::: "memory");
    dma_step(refill, ks + 2 < KS ? ks + 2 : -1);
    compute_step(cur);
  };

  dma_step(st0, 0);
  dma_step(st1, KS > 1 ? 1 : -1);
  int ks = 0;
  for (; ks + 3 <= KS; ks += 3) {
    step(st0, st2, ks);
    step(st1, st0, ks + 1);
    step(st2, st1, ks + 2);
  }
  if (ks < KS) step(st0, st2, ks);
  if (ks + 1 < KS) step(st1, st0, ks + 1);
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));  // no DMA outstanding at exit

  // ---- epilogue
  if constexpr (EPI == EPI_GATEUP && NSUB == 2) {
    if (g.q_codes) {
      store_h_mxfp8(g, acc, (nt * BN) / 32 + wave, mt * BM, n_rows, r_begin, lg, lr);
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
      const int n = nt * BN + wave * 16 * NSUB + j * 16 + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = mt * BM + 16 * i + 4 * lg + r;
        if (rr >= n_rows) continue;
        const int64_t R = r_begin + rr;
        float v;
        if (EPI == EPI_GATEUP) {
          v = silu_f32(acc[i][j][r]) * acc[i][NSUB + j][r];
        } else {
          v = acc[i][j][r];
          if (g.row_scale) v *= g.row_scale[R];
        }
        store_out<EPI>(g, R * g.N + n, v);
      }
    }
}

// MXFP4 weights x MXFP8 activations for a reduction size fixed at compile
// time (KS steps of 128).  The tile and MFMA layout are those of the kernel
// above, but each wave fetches its own weight fragments straight into
// registers D steps ahead (the 4 waves split the outputs, so no weight byte
// is shared between waves and none goes through LDS), and only the
// activation tile, which all 4 waves read, is staged by DMA through a ring of
// RS LDS stages.  With the K loop fully unrolled, the compiler places exact
// waits for the register loads, and the wait for a stage's DMA is a
// compile-time count of the memory instructions issued after it
// (mx2_wait_count); about 2.5x the bytes of the DMA-only kernel are in flight.
template <int GK, int EPI, int NSUB, int KS>
struct Mx2Cfg {
  static constexpr int BM = kBM;
  static constexpr int BN = 64 * NSUB;
  static constexpr int NU = EPI == EPI_GATEUP ? 2 : 1;
  static constexpr int NS = NU * NSUB;          // 16-column weight subtiles per wave
  static constexpr int RS = KS < 8 ? KS : 8;    // activation stages in the LDS ring
  // steps of weight fragments in flight per wave (2 for the 128-output
  // gate_up tiles, whose 4 weight subtiles per wave would spill more)
  static constexpr int D = KS < 3 ? KS : (NS >= 4 ? 2 : 3);
  static constexpr int A_BYTES = BM * 128;
  static constexpr int STAGE = A_BYTES;
  // per row and step one scale dword: 4 UE8M0 block scales (MX) or the f32
  // scale of the 128-block (FP8); either way K/32 bytes per row.  The tile's
  // scales of all KS steps sit in one LDS table [step][row], copied once.
  static constexpr int TAB = KS * BM * 4;
  static constexpr int A_INS = A_BYTES / 4096;    // 16-byte DMA instructions per thread and stage
  static constexpr int OPS_A = A_INS;
  static constexpr int W_LD = GK == GK_FP8 ? 2 : 1;  // 16-byte code loads per subtile and step
  static constexpr int OPS_W = (W_LD + 1) * NS;   // + one scale dword per subtile
};

// Memory instructions a thread issues between the DMA of stage ks (or the
// weight loads of step ks) and the wait at the top of step ks.  The prologue
// issues W(0..D-1) then A(0..RS-2); step j issues A(j+RS-1) after its barrier
// and W(j+D) after its MFMAs.  The wait covers both, so the compiler never
// adds its own (it would wait for every load in flight).
// VS >= KS: steps that load weight fragments (a workgroup looping over
// several output tiles keeps loading weights after its KS activation stages).
template <int KS, int RS, int D, int OA, int OW, int VS = KS>
constexpr int mx2_ops_between_steps(int j0, int ks) {  // steps j0+1 .. ks-1
  int n = 0;
  for (int j = j0 + 1; j < ks; ++j) {
    if (j + RS - 1 < KS) n += OA;
    if (j + D < VS) n += OW;
  }
  return n;
}
template <int KS, int RS, int D, int OA, int OW, int VS = KS>
constexpr int mx2_wait_count(int ks) {
  const int last = (KS < RS - 1 ? KS : RS - 1) - 1;  // last stage of the prologue
  int na = 0, nw = 0;
  if (ks <= RS - 2) {
    na = (last - ks) * OA + mx2_ops_between_steps<KS, RS, D, OA, OW, VS>(-1, ks);
  } else {
    const int j0 = ks - RS + 1;
    na = (j0 + D < VS ? OW : 0) + mx2_ops_between_steps<KS, RS, D, OA, OW, VS>(j0, ks);
  }
  if (ks < D) {
    nw = (D - 1 - ks) * OW + (last + 1) * OA + mx2_ops_between_steps<KS, RS, D, OA, OW, VS>(-1, ks);
  } else {
    nw = mx2_ops_between_steps<KS, RS, D, OA, OW, VS>(ks - D, ks);
  }
  const int n = na < nw ? na : nw;
  return n < 63 ? n : 63;  // 63 outstanding is the counter's limit
}

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>): a loop
// whose index is a constant expression in its body
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(N));
}

// NTW > 1 (down projection): a workgroup computes NTW consecutive output
// tiles of its rows.  Its activation tile stays in the LDS ring (RS = KS
// stages, loaded once); the weight fragments of the next tile load under the
// current tile's last steps (the lead of D steps runs on across tiles); each
// tile's o rows are stored as soon as its KS steps are done.
template <int GK, int EPI, int NSUB, int KS, bool WT, int NTW = 1>
__global__ void __launch_bounds__(256, 2) grouped_gemm_mx2_kernel(GemmArgs g) {
  static_assert(GK == GK_MX || GK == GK_FP8, "MX or block-FP8 operands");
  using C = Mx2Cfg<GK, EPI, NSUB, KS>;
  constexpr int BM = C::BM, BN = C::BN, NU = C::NU, NS = C::NS, RS = C::RS, D = C::D;
  static_assert(RS <= 8, "ring of at most 8 stages");
  static_assert(NTW == 1 || (EPI == EPI_DOWN && RS == KS), "several tiles per workgroup: down, resident activations");
  static_assert(NTW == 1 || GK == GK_MX || BN % 128 == 0, "block-FP8 weight scales per 128 outputs");
  constexpr int VS = KS * NTW;  // steps of the workgroup
  // one array per stage: the compiler then sees that reading a stage does
  // not alias the DMAs into the others (one array would make it wait for
  // every DMA in flight before each read)
  __shared__ __attribute__((aligned(16))) uint8_t r0[C::STAGE], r1[RS > 1 ? C::STAGE : 16],
      r2[RS > 2 ? C::STAGE : 16], r3[RS > 3 ? C::STAGE : 16], r4[RS > 4 ? C::STAGE : 16],
      r5[RS > 5 ? C::STAGE : 16], r6[RS > 6 ? C::STAGE : 16], r7[RS > 7 ? C::STAGE : 16];
  auto stage = [&](auto sc) __attribute__((always_inline)) -> uint8_t* {
    constexpr int S = decltype(sc)::value;
    if constexpr (S == 0) return r0;
    else if constexpr (S == 1) return r1;
    else if constexpr (S == 2) return r2;
    else if constexpr (S == 3) return r3;
    else if constexpr (S == 4) return r4;
    else if constexpr (S == 5) return r5;
    else if constexpr (S == 6) return r6;
    else return r7;
  };
  __shared__ __attribute__((aligned(16))) uint8_t s_tab[C::TAB];  // activation scales [step][row]
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
  int* s_toff = reinterpret_cast<int*>(lds_dyn);

  const int NT = g.N / (BN * NTW);  // groups of NTW output tiles

  int L, e, mt, nt, r_begin, n_rows;
  if (g.dense_rows > 0) {
    e = 0;
    L = xcd_tile((g.dense_rows + BM - 1) / BM * NT);
    if (L < 0) return;
    nt = (L % NT) * NTW;
    mt = L / NT;
    r_begin = 0;
    n_rows = g.dense_rows;
  } else {
    for (int i = threadIdx.x; i <= g.E; i += 256) s_toff[i] = g.tile_offsets[i];
    __syncthreads();
    L = xcd_tile(s_toff[g.E] * NT);
    if (L < 0) return;
    nt = (L % NT) * NTW;
    const int mg = L / NT;
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

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  constexpr int K = KS * kBK;
  constexpr int SKB = K / 32;  // scale bytes per row
  const int NW = NU * g.N;
  constexpr int W_ROW = GK == GK_FP8 ? K : K / 2;      // weight bytes per row
  // A row holds PH 64-byte pieces per K step.  What one K step adds to a
  // lane's weight address and (MX) scale address: row-major, the row's next
  // PH pieces and its next scale dword; tiled (moe_fp4_tile_weights), the
  // next PH kilobytes and 64 bytes.  W_HALF: offset of a row's second piece.
  constexpr int PH = GK == GK_FP8 ? 2 : 1;
  constexpr int W_STEP = WT ? PH * 1024 : PH * 64;
  constexpr int W_HALF = WT ? 1024 : 64;
  constexpr int WS_STEP = WT && GK == GK_MX ? 64 : 4;
  const uint8_t* w_base = g.w_codes + (int64_t)e * NW * W_ROW;
  const uint8_t* ws_base = reinterpret_cast<const uint8_t*>(g.w_scales);

  auto a_row_of = [&](int r) __attribute__((always_inline)) -> int64_t {
    const int rr = mt * BM + r;
    const int R = r_begin + (rr < n_rows ? rr : 0);  // rows past the expert's end fetch row 0 (never stored)
    return g.a_gather ? g.pair_of_row[R] / g.k : R;
  };
  auto w_grow = [&](int i) __attribute__((always_inline)) -> int { return (i / BN) * g.N + nt * BN + (i % BN); };

  // activation DMA sources (step 0; a step advances codes by 128 B, scales by 4 B)
  const uint8_t* a_src[C::A_INS];
#pragma unroll
  for (int q = 0; q < C::A_INS; ++q) {
    const int row = (q * 4 + wave) * 8 + (lane >> 3), slot = lane & 7;
    const int chunk = slot ^ ((row ^ (row >> 3)) & 7);  // inverse of swz<128>
    a_src[q] = g.a_codes + a_row_of(row) * K + 16 * chunk;
  }
  // this lane's row of the scale table (row = lane; each wave copies steps w, w + 4, ...)
  const uint8_t* as_src = reinterpret_cast<const uint8_t*>(g.a_scales) + a_row_of(lane) * SKB;
  // this lane's weight rows: column lr of subtile s, K block lg of each step
  const uint8_t* w_src[NS];
  const uint8_t* ws_src[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int wr = (s / NSUB) * BN + wave * 16 * NSUB + (s % NSUB) * 16 + lr;
    const int gr = w_grow(wr);
    if constexpr (WT)  // 16 consecutive rows (gr % 16 == lr): PH kilobytes per K step
      w_src[s] = w_base + (int64_t)(gr >> 4) * (KS * PH * 1024) + (gr & 15) * 64 + 16 * lg;
    else
      w_src[s] = w_base + (int64_t)gr * W_ROW + 16 * lg;
    if (GK == GK_MX && WT)
      ws_src[s] = ws_base + (int64_t)e * NW * SKB + (int64_t)(gr >> 4) * (KS * 64) + (gr & 15) * 4;
    else if (GK == GK_MX)  // the step's 4 UE8M0 block scales of the row as one dword
      ws_src[s] = ws_base + ((int64_t)e * NW + gr) * SKB;
    else  // the f32 scale of the row's 128 x 128 block
      ws_src[s] = ws_base + (((int64_t)e * (NW / 128) + w_grow(wr) / 128) * KS) * 4;
  }

  auto dma_a = [&](int ks, uint8_t* st) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < C::A_INS; ++q) dma16_to_lds(a_src[q] + ks * 128, st + (q * 4 + wave) * 1024);
  };
  u32x4 wq[D][NS][C::W_LD];
  int wsq[D][NS];
  // step v = (tile v / KS of the workgroup, K step v % KS); the next output
  // tile is BN weight rows further: whole 16-row groups when tiled, whole
  // 128 x 128 scale blocks for block FP8 (BN % 128 == 0)
  constexpr int64_t W_NT = WT ? (int64_t)(BN / 16) * KS * PH * 1024 : (int64_t)BN * W_ROW;
  constexpr int64_t WS_NT = GK == GK_MX ? (WT ? (int64_t)(BN / 16) * KS * 64 : (int64_t)BN * SKB)
                                        : (int64_t)(BN / 128) * KS * 4;
  auto load_w = [&](int v, u32x4 (&q)[NS][C::W_LD], int (&sc)[NS]) __attribute__((always_inline)) {
    const int nv = v / KS, ks = v % KS;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint8_t* wp = w_src[s] + W_NT * nv + W_STEP * ks;
      q[s][0] = ld16(wp);
      if constexpr (GK == GK_FP8) q[s][C::W_LD - 1] = ld16(wp + W_HALF);
      sc[s] = (int)*reinterpret_cast<const uint32_t*>(ws_src[s] + WS_NT * nv + WS_STEP * ks);  // MX: byte lg is this lane's
    }
  };

  floatx4 acc[4][NS];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[i][s] = floatx4{0.f, 0.f, 0.f, 0.f};

  // prologue: the scale table (older than every later load, so the waits
  // below cover it), weights of steps 0..D-1, then activation stages 0..RS-2
  for (int ks = __builtin_amdgcn_readfirstlane(wave); ks < KS; ks += 4) dma4_to_lds(as_src + 4 * ks, s_tab + ks * BM * 4);
#pragma unroll
  for (int j = 0; j < D; ++j) load_w(j, wq[j], wsq[j]);
  static_for<RS - 1>([&](auto jc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    if constexpr (j < KS) dma_a(j, stage(std::integral_constant<int, j>{}));
  });
  __builtin_amdgcn_sched_barrier(0);

  // epilogue of one output tile (its index arithmetic starts from an opaque
  // zero so that none of it is hoisted into the unrolled K loop, where it
  // would hold registers through every step)
  auto store_tile = [&](int ntile) __attribute__((always_inline)) {
    int z0;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z0));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NSUB; ++j) {
        const int n = ntile * BN + wave * 16 * NSUB + j * 16 + lr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rr = mt * BM + 16 * i + 4 * lg + r + z0;
          if (rr >= n_rows) continue;
          const int64_t R = r_begin + rr;
          float v;
          if (EPI == EPI_GATEUP) {
            v = silu_f32(acc[i][j][r]) * acc[i][NSUB + j][r];
          } else {
            v = acc[i][j][r];
            if (g.row_scale) v *= g.row_scale[R];
          }
          store_out<EPI>(g, R * g.N + n, v);
        }
      }
  };

  static_for<VS>([&](auto vc) __attribute__((always_inline)) {
    constexpr int v = decltype(vc)::value, ks = v % KS;
    if constexpr (v < KS) {
      // own DMAs of stage ks done (later ones may stay in flight); own LDS
      // reads of the previous step done; then everyone's.  Later tiles read
      // the same stages, which no DMA overwrites.
      wait_vm_lgkm0<mx2_wait_count<KS, RS, D, C::OPS_A, C::OPS_W, VS>(ks)>();
      asm volatile("s_barrier" ::: "memory");
      if constexpr (ks + RS - 1 < KS) dma_a(ks + RS - 1, stage(std::integral_constant<int, (ks + RS - 1) % RS>{}));
    }
    __builtin_amdgcn_sched_barrier(0);
    {
      // with several tiles, an opaque zero keeps the compiler from holding
      // every stage's fragments in registers from one tile to the next
      int zo = 0;
      if constexpr (NTW > 1) asm volatile("s_mov_b32 %0, 0" : "=s"(zo));
      const uint8_t* s_a = stage(std::integral_constant<int, ks % RS>{}) + zo;
      const uint8_t* s_as = s_tab + ks * BM * 4 + zo;
      intx8 af[4];
      int asc[4];
      float afs[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 lo = ld16(s_a + swz<128>(16 * i + lr, lg));
        const u32x4 hi = ld16(s_a + swz<128>(16 * i + lr, 4 + lg));
        af[i] = intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        if constexpr (GK == GK_MX) {
          asc[i] = s_as[(16 * i + lr) * 4 + lg];
        } else {  // f32 scales of the accumulator rows 16 i + 4 lg + r
          const u32x4 v = ld16(s_as + (16 * i + 4 * lg) * 4);
          afs[i][0] = __uint_as_float(v.x); afs[i][1] = __uint_as_float(v.y);
          afs[i][2] = __uint_as_float(v.z); afs[i][3] = __uint_as_float(v.w);
        }
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if constexpr (GK == GK_MX) {
          const u32x4 c = wq[v % D][s][0];
          const intx8 bv = intx8{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
          const int bsc = (int)(((uint32_t)wsq[v % D][s] >> (8 * lg)) & 0xFFu);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[i][s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bv, acc[i][s], 0, 4, 0, asc[i], 0, bsc);
        } else {
          // unit-scale E4M3 products of the 128-block, then the block's
          // activation-row and weight scales in f32
          const u32x4 lo = wq[v % D][s][0], hi = wq[v % D][s][C::W_LD - 1];
          const intx8 bv = intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          const float ws = __uint_as_float((uint32_t)wsq[v % D][s]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const floatx4 pp = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                af[i], bv, floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][s][r] = fmaf(pp[r], afs[i][r] * ws, acc[i][s][r]);
          }
        }
      }
    }
    // the accumulators are used here, so the step's MFMAs are not sunk
    // towards the epilogue (which would keep every step's operands live)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int s = 0; s < NS; ++s) asm volatile("" ::"v"(acc[i][s]));
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (v + D < VS) load_w(v + D, wq[v % D], wsq[v % D]);
    if constexpr (NTW > 1 && ks == KS - 1) {
      store_tile(nt + v / KS);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[i][s] = floatx4{0.f, 0.f, 0.f, 0.f};
      __builtin_amdgcn_sched_barrier(0);
    }
  });
  if constexpr (NTW > 1) return;

  if constexpr (GK == GK_MX && EPI == EPI_GATEUP && NSUB == 2) {
    if (g.q_codes) {
      int z0;
      asm volatile("v_mov_b32 %0, 0" : "=v"(z0));
      store_h_mxfp8(g, acc, (nt * BN) / 32 + wave, mt * BM + z0, n_rows, r_begin, lg, lr);
      return;
    }
  }
  if constexpr (GK == GK_FP8 && EPI == EPI_GATEUP && NSUB == 2) {
    if (g.q_codes) {
      int z0;
      asm volatile("v_mov_b32 %0, 0" : "=v"(z0));
      store_h_fp8row(g, acc, nt, mt * BM + z0, n_rows, r_begin, wave, lg, lr);
      return;
    }
  }
  store_tile(nt);
}

// NVFP4 x NVFP4 on the same plan: each wave's weight fragments (E2M1 codes
// and the two E4M3 scales of its 32 values) go straight into VGPRs D steps
// ahead and are decoded to fp16 per MFMA fragment; the activation codes and
// scales arrive by DMA in an LDS ring, and during step ks the workgroup
// decodes step ks+1's tile once into one of two fp16 LDS buffers (one barrier
// per step).  Waits are compile-time counts as in the kernel above.
template <int EPI, int NSUB, int KS>
struct Nv2Cfg {
  static constexpr int BM = kBM;
  static constexpr int BN = 64 * NSUB;
  static constexpr int NU = EPI == EPI_GATEUP ? 2 : 1;
  static constexpr int NS = NU * NSUB;
  static constexpr int RS = KS < 6 ? KS : 6;         // raw activation stages
  static constexpr int D = KS < 2 ? KS : 2;          // steps of weight fragments in flight per wave
  static constexpr int RAW_A = BM * 64;              // E2M1 codes: 64 rows x 128 values
  static constexpr int RAW = RAW_A + BM * 8;         // + 8 E4M3 scales per row
  static constexpr int DEC = BM * 256;               // fp16 tile, 64 rows x 128 values
  static constexpr int OPS_A = 2;                    // one 16-byte and one 4-byte DMA per thread
  static constexpr int OPS_W = 2 * NS;               // per subtile: codes (16 B) + the row's 8 scales
};

// Memory instructions issued by a thread between a given raw stage's DMA (or
// a step's weight loads) and the wait at the top of step ks.  Prologue:
// W(0..D-1), raw(0..RS-2); step j: raw(j+RS-1) after the barrier, W(j+D)
// after the MFMAs.
// VS >= KS: steps that load weight fragments (several output tiles per
// workgroup); raw stages are loaded during the first KS steps only.
template <int KS, int RS, int D, int OA, int OW, int VS = KS>
constexpr int nv2_ops_steps(int j0, int ks) {  // ops of steps j0+1 .. ks-1
  int n = 0;
  for (int j = j0 + 1; j < ks; ++j) {
    if (j + RS - 1 < KS) n += OA;
    if (j + D < VS) n += OW;
  }
  return n;
}
template <int KS, int RS, int D, int OA, int OW, int VS = KS>
constexpr int nv2_after_raw(int s, int ks) {  // raw stage s, wait of step ks
  const int last = (KS < RS - 1 ? KS : RS - 1) - 1;
  if (s <= RS - 2) return (last - s) * OA + nv2_ops_steps<KS, RS, D, OA, OW, VS>(-1, ks);
  const int j0 = s - RS + 1;
  return (j0 + D < VS ? OW : 0) + nv2_ops_steps<KS, RS, D, OA, OW, VS>(j0, ks);
}
template <int KS, int RS, int D, int OA, int OW, int VS = KS>
constexpr int nv2_wait_count(int ks) {  // raw(ks+1) and W(ks) done
  const int last = (KS < RS - 1 ? KS : RS - 1) - 1;
  const int nw = ks < D ? (D - 1 - ks) * OW + (last + 1) * OA + nv2_ops_steps<KS, RS, D, OA, OW, VS>(-1, ks)
                        : nv2_ops_steps<KS, RS, D, OA, OW, VS>(ks - D, ks);
  int n = nw;
  if (ks + 1 < KS) {
    const int na = nv2_after_raw<KS, RS, D, OA, OW, VS>(ks + 1, ks);
    n = na < n ? na : n;
  }
  return n < 63 ? n : 63;
}

// NTW > 1 (down projection): a workgroup computes NTW consecutive output
// tiles of its rows.  The raw activation stages stay in LDS (RS = KS, loaded
// once) and every tile decodes them again, one step ahead as in the first;
// the weight lead of D steps runs on across tiles; each tile's o rows are
// stored as soon as its KS steps are done.
template <int EPI, int NSUB, int KS, bool WT, int NTW = 1>
__global__ void __launch_bounds__(256, 2) grouped_gemm_nv2_kernel(GemmArgs g) {
  using C = Nv2Cfg<EPI, NSUB, KS>;
  constexpr int BM = C::BM, BN = C::BN, NU = C::NU, NS = C::NS, RS = C::RS, D = C::D;
  static_assert(RS <= 6, "ring of at most 6 raw stages");
  static_assert(NTW == 1 || (EPI == EPI_DOWN && RS == KS), "several tiles per workgroup: down, resident activations");
  constexpr int VS = KS * NTW;  // steps of the workgroup
  __shared__ __attribute__((aligned(16))) uint8_t q0[C::RAW], q1[RS > 1 ? C::RAW : 16], q2[RS > 2 ? C::RAW : 16],
      q3[RS > 3 ? C::RAW : 16], q4[RS > 4 ? C::RAW : 16], q5[RS > 5 ? C::RAW : 16];
  __shared__ __attribute__((aligned(16))) uint8_t d0[C::DEC], d1[C::DEC];
  __shared__ __attribute__((aligned(16))) uint8_t dummy[512];
  auto raw = [&](auto sc) __attribute__((always_inline)) -> uint8_t* {
    constexpr int S = decltype(sc)::value;
    if constexpr (S == 0) return q0;
    else if constexpr (S == 1) return q1;
    else if constexpr (S == 2) return q2;
    else if constexpr (S == 3) return q3;
    else if constexpr (S == 4) return q4;
    else return q5;
  };
  auto dec = [&](auto sc) __attribute__((always_inline)) -> uint8_t* {
    if constexpr (decltype(sc)::value == 0) return d0;
    else return d1;
  };
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
  int* s_toff = reinterpret_cast<int*>(lds_dyn);

  const int NT = g.N / (BN * NTW);  // groups of NTW output tiles
  int L, e, mt, nt, r_begin, n_rows;
  if (g.dense_rows > 0) {
    e = 0;
    L = xcd_tile((g.dense_rows + BM - 1) / BM * NT);
    if (L < 0) return;
    nt = (L % NT) * NTW;
    mt = L / NT;
    r_begin = 0;
    n_rows = g.dense_rows;
  } else {
    for (int i = threadIdx.x; i <= g.E; i += 256) s_toff[i] = g.tile_offsets[i];
    __syncthreads();
    L = xcd_tile(s_toff[g.E] * NT);
    if (L < 0) {
      if (EPI == EPI_GATEUP && g.amax_part && threadIdx.x == 0) g.amax_part[blockIdx.x] = 0.0f;
      return;
    }
    nt = (L % NT) * NTW;
    const int mg = L / NT;
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

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  // 16-row groups of the tile that hold rows (an expert's last tile is
  // partial): the MFMAs and fragment reads of the others are skipped (C3:
  // gate_up 554 -> 529 us; the same branches in the MX kernel measured slower)
  const int rgv = __builtin_amdgcn_readfirstlane(min(4, (n_rows - mt * BM + 15) >> 4));
  constexpr int K = KS * kBK;
  const int NW = NU * g.N;
  auto a_row_of = [&](int r) __attribute__((always_inline)) -> int64_t {
    const int rr = mt * BM + r;
    const int R = r_begin + (rr < n_rows ? rr : 0);  // rows past the expert's end fetch row 0 (never stored)
    return g.a_gather ? g.pair_of_row[R] / g.k : R;
  };
  auto w_grow = [&](int i) __attribute__((always_inline)) -> int { return (i / BN) * g.N + nt * BN + (i % BN); };

  // raw activation DMA: thread t moves 16 code bytes of row t/4 (values
  // 32 (t%4) .. +32) and, for t < 128, the 4 scale bytes t%2 of row t/2
  const int arow = tid >> 2, apart = tid & 3;
  const uint8_t* a_src = g.a_codes + a_row_of(arow) * (K / 2) + 16 * apart;
  const uint8_t* as_src = reinterpret_cast<const uint8_t*>(g.a_scales) +
                          a_row_of(tid < 128 ? tid >> 1 : 0) * (K / 16) + 4 * (tid & 1);
  auto dma_raw = [&](int ks, uint8_t* st) __attribute__((always_inline)) {
    dma16_to_lds(a_src + ks * 64, st + wave * 1024);
    dma4_to_lds(as_src + ks * 8, wave < 2 ? st + C::RAW_A + wave * 256 : dummy);
  };
  // decode this thread's 32 raw values into the fp16 tile (swizzled rows of 256 B)
  auto decode_raw = [&](const uint8_t* st, uint8_t* dt) __attribute__((always_inline)) {
    const u32x4 c = ld16(st + 16 * tid);
    const uint32_t s2 = *reinterpret_cast<const uint16_t*>(st + C::RAW_A + arow * 8 + 2 * apart);
    uint32_t d[16];
    nv_decode32(make_uint4(c.x, c.y, c.z, c.w), s2, d);
    st16(dt + swz<256>(arow, 4 * apart), u32x4{d[0], d[1], d[2], d[3]});
    st16(dt + swz<256>(arow, 4 * apart + 1), u32x4{d[4], d[5], d[6], d[7]});
    st16(dt + swz<256>(arow, 4 * apart + 2), u32x4{d[8], d[9], d[10], d[11]});
    st16(dt + swz<256>(arow, 4 * apart + 3), u32x4{d[12], d[13], d[14], d[15]});
  };
  // this lane's weight rows: column lr of subtile s, values 32 lg .. +32 of
  // each step; a step moves row-major codes 64 bytes and scales 8, tiled
  // ones (moe_fp4_tile_weights: 16 rows' step as one kilobyte / 128 bytes)
  // 1024 and 128
  constexpr int W_STEP = WT ? 1024 : 64, WS_STEP = WT ? 128 : 8;
  const uint8_t* w_src[NS];
  const uint8_t* ws_src[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int wr = (s / NSUB) * BN + wave * 16 * NSUB + (s % NSUB) * 16 + lr;
    const int gr = w_grow(wr);
    const int64_t grow = (int64_t)e * NW + gr;
    if constexpr (WT) {  // 16 consecutive rows (gr % 16 == lr)
      w_src[s] = g.w_codes + (int64_t)e * NW * (K / 2) + (int64_t)(gr >> 4) * (KS * 1024) + (gr & 15) * 64 + 16 * lg;
      ws_src[s] = reinterpret_cast<const uint8_t*>(g.w_scales) + (int64_t)e * NW * (K / 16) +
                  (int64_t)(gr >> 4) * (KS * 128) + (gr & 15) * 8;
    } else {
      w_src[s] = g.w_codes + grow * (K / 2) + 16 * lg;
      ws_src[s] = reinterpret_cast<const uint8_t*>(g.w_scales) + grow * (K / 16);
    }
  }
  u32x4 wq[D][NS];
  u32x2 wsq[D][NS];
  // step v = (tile v / KS of the workgroup, K step v % KS); the next output
  // tile is BN weight rows further (whole 16-row groups when tiled)
  constexpr int64_t W_NT = WT ? (int64_t)(BN / 16) * KS * 1024 : (int64_t)BN * (K / 2);
  constexpr int64_t WS_NT = WT ? (int64_t)(BN / 16) * KS * 128 : (int64_t)BN * (K / 16);
  auto load_w = [&](int v, u32x4 (&q)[NS], u32x2 (&sc)[NS]) __attribute__((always_inline)) {
    const int nv = v / KS, ks = v % KS;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      q[s] = ld16(w_src[s] + W_NT * nv + W_STEP * ks);
      sc[s] = *reinterpret_cast<const u32x2*>(ws_src[s] + WS_NT * nv + WS_STEP * ks);  // the row's 8 scales of the step
    }
  };

  floatx4 acc[4][NS];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[i][s] = floatx4{0.f, 0.f, 0.f, 0.f};

  // prologue: weights of steps 0..D-1, raw stages 0..RS-2, then step 0's tile decoded
#pragma unroll
  for (int j = 0; j < D; ++j) load_w(j, wq[j], wsq[j]);
  static_for<RS - 1>([&](auto jc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    if constexpr (j < KS) dma_raw(j, raw(std::integral_constant<int, j>{}));
  });
  __builtin_amdgcn_sched_barrier(0);
  wait_vm_lgkm0<nv2_after_raw<KS, RS, D, C::OPS_A, C::OPS_W>(0, 0)>();
  asm volatile("s_barrier" ::: "memory");
  decode_raw(raw(std::integral_constant<int, 0>{}), dec(std::integral_constant<int, 0>{}));
  __builtin_amdgcn_sched_barrier(0);

  // epilogue of one down tile (index arithmetic from an opaque zero: not
  // hoisted into the K loop)
  auto store_down_tile = [&](int ntile) __attribute__((always_inline)) {
    int z0;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z0));
    const float scale = g.a_tensor_scale[0] * g.w_tensor_scale[e];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NSUB; ++j) {
        const int n = ntile * BN + wave * 16 * NSUB + j * 16 + lr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rr = mt * BM + 16 * i + 4 * lg + r + z0;
          if (rr >= n_rows) continue;
          const int64_t R = r_begin + rr;
          float v = acc[i][j][r] * scale;
          if (g.row_scale) v *= g.row_scale[R];
          store_out<EPI>(g, R * g.N + n, v);
        }
      }
  };

  static_for<VS>([&](auto vc) __attribute__((always_inline)) {
    constexpr int v = decltype(vc)::value, ks = v % KS;
    if constexpr (v < KS) {
      wait_vm_lgkm0<nv2_wait_count<KS, RS, D, C::OPS_A, C::OPS_W, VS>(ks)>();
    } else {
      wait_vm_lgkm0<63>();  // this thread's decode of the step done (the raw stages all arrived in the first tile)
    }
    asm volatile("s_barrier" ::: "memory");
    if constexpr (ks + RS - 1 < KS && v < KS)
      dma_raw(ks + RS - 1, raw(std::integral_constant<int, (ks + RS - 1) % RS>{}));
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (v + 1 < VS)
      decode_raw(raw(std::integral_constant<int, (v + 1) % KS % RS>{}), dec(std::integral_constant<int, (v + 1) % 2>{}));
    __builtin_amdgcn_sched_barrier(0);
    {
      const uint8_t* s_a = dec(std::integral_constant<int, v % 2>{});
      uint32_t af[4][16];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i == 0 || i < rgv) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x4 f = ld16(s_a + swz<256>(16 * i + lr, 4 * lg + q));
            af[i][4 * q] = f.x; af[i][4 * q + 1] = f.y; af[i][4 * q + 2] = f.z; af[i][4 * q + 3] = f.w;
          }
        }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u32x4 c = wq[v % D][s];
        const u32x2 sc = wsq[v % D][s];
        const uint32_t s2 = ((lg < 2 ? sc.x : sc.y) >> (16 * (lg & 1))) & 0xFFFFu;
        uint32_t wd[16];
        nv_decode32(make_uint4(c.x, c.y, c.z, c.w), s2, wd);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i == 0 || i < rgv) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
              acc[i][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(&af[i][4 * m]), as_half8(&wd[4 * m]),
                                                                 acc[i][s], 0, 0, 0);
          }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int s = 0; s < NS; ++s) asm volatile("" ::"v"(acc[i][s]));
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (v + D < VS) load_w(v + D, wq[v % D], wsq[v % D]);
    if constexpr (NTW > 1 && ks == KS - 1) {
      store_down_tile(nt + v / KS);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[i][s] = floatx4{0.f, 0.f, 0.f, 0.f};
      __builtin_amdgcn_sched_barrier(0);
    }
  });
  if constexpr (NTW > 1) return;

  // ---- epilogue (index arithmetic from an opaque zero: not hoisted into the K loop)
  int z0;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z0));
  const float scale = g.a_tensor_scale[0] * g.w_tensor_scale[e];
  float vmax = 0.0f;  // max |h| stored by this lane (gate_up)
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
      const int n = nt * BN + wave * 16 * NSUB + j * 16 + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = mt * BM + 16 * i + 4 * lg + r + z0;
        if (rr >= n_rows) continue;
        const int64_t R = r_begin + rr;
        float v;
        if (EPI == EPI_GATEUP) {
          v = silu_f32(acc[i][j][r] * scale) * (acc[i][NSUB + j][r] * scale);
          vmax = fmaxf(vmax, fabsf(v));
        } else {
          v = acc[i][j][r] * scale;
          if (g.row_scale) v *= g.row_scale[R];
        }
        store_out<EPI>(g, R * g.N + n, v);
      }
    }
  if constexpr (EPI == EPI_GATEUP) {
    if (g.amax_part) {  // as in the register-staged kernel: max |h| of the workgroup
      __shared__ float red[4];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, off));
      if (lane == 0) red[wave] = vmax;
      __syncthreads();
      if (tid == 0) g.amax_part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    }
  }
}

// Output tiles per workgroup of the register-fed down GEMMs (nt tiles of
// output per row block, tiles_m_bound row blocks): 4, else 2, as long as the
// grid keeps 16 workgroups per CU, else 1.  At 8192 tokens x top-10 (1,792
// row blocks, 20 output tiles) 4 measured 345 / 351 / 461 us for the NVFP4 /
// MX / block-FP8 down GEMMs against 404 / 421 / 520 us with one tile (10:
// 355 / 361 / 467); a 16-token batch (163 row blocks) keeps one tile, whose
// grid is then 12.7 workgroups per CU.
static int down_tiles_per_wg(int64_t tiles_m_bound, int nt) {
  const int64_t want = 16LL * device_cu_count();
  if (nt % 4 == 0 && tiles_m_bound * (nt / 4) >= want) return 4;
  if (nt % 2 == 0 && tiles_m_bound * (nt / 2) >= want) return 2;
  return 1;
}

// Workgroups of a grouped GEMM launch: M-tile bound x output tiles, rounded
// up to a multiple of the 8 XCDs (the tile remapping needs whole rounds).
static int64_t gemm_grid(int64_t tiles_m_bound, int N, int BN) {
  return (tiles_m_bound * (N / BN) + 7) / 8 * 8;
}

// Raises a kernel's dynamic-LDS limit on the current device the first time
// it launches there; `raised` holds one bit per device, so concurrent callers
// at worst set the attribute twice.
static int raise_dyn_lds(const void* kernel, int bytes, std::atomic<uint64_t>& raised) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(FP4_ERR_HIP, "hipGetDevice failed");
  const uint64_t bit = 1ull << (dev & 63);
  if (raised.load(std::memory_order_acquire) & bit) return FP4_OK;
  RelaxedCapture relaxed;
  if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
    return fail(FP4_ERR_HIP, "hipFuncSetAttribute failed");
  raised.fetch_or(bit, std::memory_order_acq_rel);
  return FP4_OK;
}

template <int EPI, int NSUB, int KS, bool WT, int NTW = 1>
static int launch_gemm_nv2_t(const GemmArgs& a, int64_t tiles_m_bound, hipStream_t st) {
  using C = Nv2Cfg<EPI, NSUB, KS>;
  if (a.N % (C::BN * NTW)) return fail(FP4_ERR_SHAPE, "grouped GEMM: %d outputs are not whole groups of tiles", a.N);
  const int64_t G = gemm_grid(tiles_m_bound, a.N, C::BN * NTW);
  if (a.amax_part && G != a.amax_nparts)
    return fail(FP4_ERR_UNSUPPORTED, "grouped GEMM: %lld partial maxima expected, %lld workgroups",
                (long long)a.amax_nparts, (long long)G);
  if (G <= 0) return FP4_OK;
  if (G > INT32_MAX) return fail(FP4_ERR_UNSUPPORTED, "grouped GEMM grid too large");
  const size_t lds = a.dense_rows > 0 ? 0 : sizeof(int) * ((size_t)a.E + 1);
  // static LDS: the raw and decoded stages, 512 bytes of other arrays and 64
  // for the gate_up epilogue's reduction
  constexpr size_t fixed = (size_t)C::RS * C::RAW + 2 * (size_t)C::DEC + 512 + 64;
  if (fixed + lds > 160 * 1024) return fail(FP4_ERR_UNSUPPORTED, "grouped GEMM tile needs too much LDS");
  static std::atomic<uint64_t> lds_raised{0};
  FP4_CHECK(raise_dyn_lds(reinterpret_cast<const void*>(&grouped_gemm_nv2_kernel<EPI, NSUB, KS, WT, NTW>),
                            (int)(160 * 1024 - fixed), lds_raised));
  hipLaunchKernelGGL((grouped_gemm_nv2_kernel<EPI, NSUB, KS, WT, NTW>), dim3((unsigned)G), dim3(256), lds, st, a);
  return check_launch("grouped_gemm_nv2");
}

template <int EPI, int NSUB, int KS, int NTW = 1>
static int launch_gemm_nv2(const GemmArgs& a, int64_t tiles_m_bound, hipStream_t st) {
  return a.w_tiled ? launch_gemm_nv2_t<EPI, NSUB, KS, true, NTW>(a, tiles_m_bound, st)
                   : launch_gemm_nv2_t<EPI, NSUB, KS, false, NTW>(a, tiles_m_bound, st);
}
template <int EPI, int NSUB, int KS>
static int launch_gemm_nv2_down(const GemmArgs& a, int64_t tiles_m_bound, hipStream_t st) {
  switch (down_tiles_per_wg(tiles_m_bound, a.N / (64 * NSUB))) {
    case 4: return launch_gemm_nv2<EPI, NSUB, KS, 4>(a, tiles_m_bound, st);
    case 2: return launch_gemm_nv2<EPI, NSUB, KS, 2>(a, tiles_m_bound, st);
    default: return launch_gemm_nv2<EPI, NSUB, KS>(a, tiles_m_bound, st);
  }
}

// Tiled order of moe_fp4_tile_weights.  The E stacked [rows, cols] tensors
// are one run of E * rows rows (rows % 16 == 0, so no 16-row group straddles
// two experts).  A row holds PH 64-byte pieces per 128-wide K step (E2M1 1,
// E4M3 2); piece h of the 16 rows of a group is one kilobyte.  A row's block
// scales of a K step are SB bytes (MXFP4 4, NVFP4 8; block FP8: none).
// Thread i copies 16-byte code chunk i and the scales of (row, step) i.
__global__ void __launch_bounds__(256) tile_weights_kernel(const uint8_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales,
                                                           int64_t rows_total, int KS, int PH, int SB,
                                                           uint8_t* __restrict__ tiled_codes,
                                                           uint8_t* __restrict__ tiled_scales) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cpr = KS * PH * 4;  // 16-byte chunks per row
  if (i < rows_total * cpr) {   // code chunks: row r, K step ks, piece h, 16 bytes u of its 64
    const int64_t r = i / cpr;
    const int c = (int)(i - r * cpr), ks = c / (PH * 4), h = (c >> 2) % PH, u = c & 3;
    const int64_t dst = (r >> 4) * ((int64_t)KS * PH * 1024) + (ks * PH + h) * 1024 + (r & 15) * 64 + u * 16;
    *reinterpret_cast<uint4*>(tiled_codes + dst) = *reinterpret_cast<const uint4*>(codes + i * 16);
  }
  if (tiled_scales && i < rows_total * KS) {  // scales of row r, K step ks
    const int64_t r = i / KS;
    const int ks = (int)(i - r * KS);
    const int64_t dst = (r >> 4) * ((int64_t)KS * 16 * SB) + ks * 16 * SB + (r & 15) * SB;
    if (SB == 8)
      *reinterpret_cast<u32x2*>(tiled_scales + dst) = *reinterpret_cast<const u32x2*>(scales + i * 8);
    else
      *reinterpret_cast<uint32_t*>(tiled_scales + dst) = *reinterpret_cast<const uint32_t*>(scales + i * 4);
  }
}

// Where the register-fed kernel (which can read tiled weights) runs: the MX
// and block-FP8 down projections for 128-multiple outputs over the model's
// inter of 640, and the block-FP8 gate_up over its hidden of 2560.
static bool mx_down_on_mx2(int N, int K) { return N % 128 == 0 && K == 640; }
static bool fp8_gateup_on_mx2(int N, int K) { return N % 64 == 0 && K == 2560; }
// Block-FP8 gate_up on 128-output tiles (tiled weights, and a grid that
// keeps 16 workgroups per CU; decode-size grids, which the wider tiles would
// halve, keep 64): 8192 tokens 750 -> 686 us.  Its epilogue can then hold a
// (row, 128) block of h whole and write h quantized.
static bool fp8_gateup_128(int w_tiled, int N, int K, int64_t tiles_m_bound) {
  return w_tiled && N % 128 == 0 && K == 2560 && tiles_m_bound * (N / 128) >= 16LL * device_cu_count();
}
// the MX gate_up over the model's hidden of 2560 on 128-output tiles, when
// its weights are tiled (then faster than the all-DMA kernel; on row-major
// weights the all-DMA kernel is the faster one)
static bool mx_gateup_on_mx2(int N, int K) { return N % 128 == 0 && K == 2560; }

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

template <int GK, int EPI, int NSUB, bool WFP8, bool WT>
static int launch_gemm_n_t(const GemmArgs& a, int64_t tiles_m_bound, hipStream_t st) {
  using C = TileCfg<GK, EPI, NSUB, WFP8>;
  const int64_t G = gemm_grid(tiles_m_bound, a.N, C::BN);
  if (a.amax_part && G != a.amax_nparts)
    return fail(FP4_ERR_UNSUPPORTED, "grouped GEMM: %lld partial maxima expected, %lld workgroups",
                (long long)a.amax_nparts, (long long)G);
  if (G <= 0) return FP4_OK;
  if (G > INT32_MAX) return fail(FP4_ERR_UNSUPPORTED, "grouped GEMM grid too large");
  // 256 bytes stay for the kernel's static LDS (the epilogue's reduction)
  constexpr size_t dyn_max = 160 * 1024 - 256;
  const size_t lds = 2 * C::STAGE + (a.dense_rows > 0 ? 0 : sizeof(int) * ((size_t)a.E + 1));
  if (lds > dyn_max) return fail(FP4_ERR_UNSUPPORTED, "grouped GEMM tile needs %zu bytes of LDS", lds);
  static std::atomic<uint64_t> lds_raised{0};
  FP4_CHECK(raise_dyn_lds(reinterpret_cast<const void*>(&grouped_gemm_kernel<GK, EPI, NSUB, WFP8, WT>),
                            (int)dyn_max, lds_raised));
  hipLaunchKernelGGL((grouped_gemm_kernel<GK, EPI, NSUB, WFP8, WT>), dim3((unsigned)G), dim3(256), lds, st, a);
  return check_launch("grouped_gemm");
}

template <int GK, int EPI, int NSUB, bool WFP8>
static int launch_gemm_n(const GemmArgs& a, int64_t tiles_m_bound, hipStream_t st) {
  if constexpr (GK == GK_NV && !WFP8) {
    if (a.w_tiled) return launch_gemm_n_t<GK, EPI, NSUB, WFP8, true>(a, tiles_m_bound, st);
  } else {
    if (a.w_tiled) return fail(FP4_ERR_UNSUPPORTED, "tiled weights on a GEMM kernel that reads rows");
  }
  return launch_gemm_n_t<GK, EPI, NSUB, WFP8, false>(a, tiles_m_bound, st);
}

template <int GK, int EPI, int NSUB, int KS, bool WT, int NTW = 1>
static int launch_gemm_mx2_t(const GemmArgs& a, int64_t tiles_m_bound, hipStream_t st) {
  using C = Mx2Cfg<GK, EPI, NSUB, KS>;
  if (a.N % (C::BN * NTW)) return fail(FP4_ERR_SHAPE, "grouped GEMM: %d outputs are not whole groups of tiles", a.N);
  const int NT = a.N / (C::BN * NTW);
  int64_t G = tiles_m_bound * NT;
  G = (G + 7) / 8 * 8;
  if (G <= 0) return FP4_OK;
  if (G > INT32_MAX) return fail(FP4_ERR_UNSUPPORTED, "grouped GEMM grid too large");
  const size_t lds = a.dense_rows > 0 ? 0 : sizeof(int) * ((size_t)a.E + 1);
  // static LDS: the ring, the scale table and 1 KB for the FP8 h epilogue's row maxima
  constexpr size_t fixed = (size_t)C::RS * C::STAGE + C::TAB + 1024;
  if (fixed + lds > 160 * 1024) return fail(FP4_ERR_UNSUPPORTED, "grouped GEMM tile needs too much LDS");
  static std::atomic<uint64_t> lds_raised{0};
  FP4_CHECK(raise_dyn_lds(reinterpret_cast<const void*>(&grouped_gemm_mx2_kernel<GK, EPI, NSUB, KS, WT, NTW>),
                            (int)(160 * 1024 - fixed), lds_raised));
  hipLaunchKernelGGL((grouped_gemm_mx2_kernel<GK, EPI, NSUB, KS, WT, NTW>), dim3((unsigned)G), dim3(256), lds, st, a);
  return check_launch("grouped_gemm_mx2");
}

template <int GK, int EPI, int NSUB, int KS, int NTW = 1>
static int launch_gemm_mx2(const GemmArgs& a, int64_t tiles_m_bound, hipStream_t st) {
  return a.w_tiled ? launch_gemm_mx2_t<GK, EPI, NSUB, KS, true, NTW>(a, tiles_m_bound, st)
                   : launch_gemm_mx2_t<GK, EPI, NSUB, KS, false, NTW>(a, tiles_m_bound, st);
}

template <int GK, int EPI, int NSUB, int KS>
static int launch_gemm_mx2_down(const GemmArgs& a, int64_t tiles_m_bound, hipStream_t st) {
  switch (down_tiles_per_wg(tiles_m_bound, a.N / (64 * NSUB))) {
    case 4: return launch_gemm_mx2<GK, EPI, NSUB, KS, 4>(a, tiles_m_bound, st);
    case 2: return launch_gemm_mx2<GK, EPI, NSUB, KS, 2>(a, tiles_m_bound, st);
    default: return launch_gemm_mx2<GK, EPI, NSUB, KS>(a, tiles_m_bound, st);
  }
}

template <int EPI, int NSUB, bool WT>
static int launch_gemm_mx_t(const GemmArgs& a, int64_t tiles_m_bound, hipStream_t st) {
  using C = MxCfg<EPI, NSUB>;
  const int NT = a.N / C::BN;
  int64_t G = tiles_m_bound * NT;
  G = (G + 7) / 8 * 8;
  if (G <= 0) return FP4_OK;
  if (G > INT32_MAX) return fail(FP4_ERR_UNSUPPORTED, "grouped GEMM grid too large");
  const size_t lds = a.dense_rows > 0 ? 0 : sizeof(int) * ((size_t)a.E + 1);
  if (3 * (size_t)C::STAGE + 256 + lds > 160 * 1024)
    return fail(FP4_ERR_UNSUPPORTED, "grouped GEMM tile needs too much LDS");
  static std::atomic<uint64_t> lds_raised{0};
  FP4_CHECK(raise_dyn_lds(reinterpret_cast<const void*>(&grouped_gemm_mx_kernel<EPI, NSUB, WT>),
                            (int)(160 * 1024 - 3 * C::STAGE - 256), lds_raised));
  hipLaunchKernelGGL((grouped_gemm_mx_kernel<EPI, NSUB, WT>), dim3((unsigned)G), dim3(256), lds, st, a);
  return check_launch("grouped_gemm_mx");
}

template <int EPI, int NSUB>
static int launch_gemm_mx(const GemmArgs& a, int64_t tiles_m_bound, hipStream_t st) {
  return a.w_tiled ? launch_gemm_mx_t<EPI, NSUB, true>(a, tiles_m_bound, st)
                   : launch_gemm_mx_t<EPI, NSUB, false>(a, tiles_m_bound, st);
}

// Widest tile (outputs per tile 64 * NSUB) that divides N and fits LDS.
template <int GK, int EPI, bool WFP8>
static int launch_gemm_w(const GemmArgs& a, int64_t tiles_m_bound, hipStream_t st) {
  if (a.N % 128 == 0) return launch_gemm_n<GK, EPI, 2, WFP8>(a, tiles_m_bound, st);
  if (a.N % 64 == 0) return launch_gemm_n<GK, EPI, 1, WFP8>(a, tiles_m_bound, st);
  return fail(FP4_ERR_SHAPE, "output width %d is not a multiple of 64", a.N);
}

template <int GK, int EPI>
static int launch_gemm(const GemmArgs& a, int64_t tiles_m_bound, hipStream_t st) {
  if (GK == GK_NV) {
    // down over the model's inter 640 on the register-fed kernel (measured
    // faster there; over K = 2560 the register-staged kernel is faster)
    if constexpr (EPI == EPI_DOWN) {
      if (a.N % 128 == 0 && a.K == 640) return launch_gemm_nv2_down<EPI, 2, 5>(a, tiles_m_bound, st);
    } else {
      // gate_up over the model's hidden of 2560 on tiled weights: the
      // register-fed kernel (on row-major weights the register-staged one)
      if (a.w_tiled && a.N % 128 == 0 && a.K == 2560) return launch_gemm_nv2<EPI, 2, 20>(a, tiles_m_bound, st);
    }
    return launch_gemm_w<GK, EPI, false>(a, tiles_m_bound, st);
  }
  if (GK == GK_FP8) {
    // the model's reduction sizes on the register-fed kernel (gate_up with
    // 64-output tiles: 128-output ones spill)
    if constexpr (EPI == EPI_DOWN) {
      if (mx_down_on_mx2(a.N, a.K)) return launch_gemm_mx2_down<GK_FP8, EPI, 2, 5>(a, tiles_m_bound, st);
    } else {
      // 128-output tiles on tiled weights when they still give every CU 16
      // workgroups (8192 tokens: 686 against 750 us); decode batches, whose
      // grid the wider tiles would halve, and row-major weights keep 64
      if (fp8_gateup_128(a.w_tiled, a.N, a.K, tiles_m_bound)) return launch_gemm_mx2<GK_FP8, EPI, 2, 20>(a, tiles_m_bound, st);
      if (a.q_codes) return fail(FP4_ERR_UNSUPPORTED, "FP8 h epilogue needs 128-output gate_up tiles");
      if (fp8_gateup_on_mx2(a.N, a.K)) return launch_gemm_mx2<GK_FP8, EPI, 1, 20>(a, tiles_m_bound, st);
    }
    if (a.w_tiled) return fail(FP4_ERR_UNSUPPORTED, "tiled weights on a GEMM kernel that reads rows");
    // FP8 weight tiles are twice the bytes: 64-output gate_up tiles keep two
    // workgroups per CU in LDS and measure faster; the down tiles do not
    if (EPI == EPI_GATEUP && a.N % 64 == 0) return launch_gemm_n<GK, EPI, 1, true>(a, tiles_m_bound, st);
    return launch_gemm_w<GK, EPI, true>(a, tiles_m_bound, st);
  }
  if (a.w_fp8) return launch_gemm_w<GK, EPI, true>(a, tiles_m_bound, st);
  // the DMA-staged kernel pays off over long K (gate_up, K = hidden); the
  // short-K down projection is faster on the register-staged kernel
  // down projection over the model's inter 640: the register-fed kernel with
  // its K loop unrolled (measured faster than either staging kernel there;
  // over K = 2560 the all-DMA kernel is faster)
  if constexpr (EPI == EPI_DOWN) {
    if (mx_down_on_mx2(a.N, a.K)) return launch_gemm_mx2_down<GK_MX, EPI, 2, 5>(a, tiles_m_bound, st);
  }
  if constexpr (EPI == EPI_GATEUP) {
    if (a.w_tiled && mx_gateup_on_mx2(a.N, a.K)) return launch_gemm_mx2<GK_MX, EPI, 2, 20>(a, tiles_m_bound, st);
    if (a.N % 128 == 0) return launch_gemm_mx<EPI, 2>(a, tiles_m_bound, st);
    if (a.q_codes) return fail(FP4_ERR_UNSUPPORTED, "MXFP8 h epilogue needs 128-output gate_up tiles");
    if (a.N % 64 == 0) return launch_gemm_mx<EPI, 1>(a, tiles_m_bound, st);
  }
  if (a.w_tiled) return fail(FP4_ERR_UNSUPPORTED, "tiled weights on a GEMM kernel that reads rows");
  return launch_gemm_w<GK, EPI, false>(a, tiles_m_bound, st);
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
  // the tiled copy of W13, when the layer has one, where the gate_up kernel
  // reads it (NVFP4 and MXFP4: always; block FP8: on the register-fed
  // kernel, codes only, its block scales stay as they are)
  a.w_tiled = L->w13_tiled && (gk != GK_FP8 || fp8_gateup_on_mx2(I, H)) ? 1 : 0;
  a.w_codes = a.w_tiled ? L->w13_tiled : L->w13;
  a.w_scales = a.w_tiled && gk != GK_FP8 ? static_cast<const void*>(L->w13_scale_tiled) : L->w13_scale;
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
  // MXFP8 h has one scale per 32 outputs, which the MX gate_up kernel's
  // 128-output tiles hold whole: its epilogue writes h quantized (no f32 h);
  // likewise FP8 h (one scale per 128 outputs) on the block-FP8 kernel's
  // 128-output tiles
  const bool h_in_epilogue = (gk == GK_MX && I % 128 == 0) || (gk == GK_FP8 && fp8_gateup_128(a.w_tiled, I, H, tiles_bound));
  a.q_codes = h_in_epilogue ? w.hq_codes : nullptr;
  a.q_scales = h_in_epilogue ? static_cast<uint8_t*>(w.hq_scales) : nullptr;
  // NVFP4 h with a dynamic tensor scale: the gate_up workgroups (register-
  // staged kernel, 128- or 64-output tiles) leave their max |h| behind, so
  // the scale needs no second pass over h
  const bool static_h = L->a_fmt == FP4_FMT_NVFP4 && L->inter_scale;
  const bool h_parts = gk == GK_NV && !static_h;
  a.amax_part = h_parts ? w.h_amax_part : nullptr;
  a.amax_nparts = h_parts ? gemm_grid(tiles_bound, I, I % 128 == 0 ? 128 : 64) : 0;
  if (gk == GK_NV) FP4_CHECK((launch_gemm<GK_NV, EPI_GATEUP>(a, tiles_bound, st)));
  else if (gk == GK_MX) FP4_CHECK((launch_gemm<GK_MX, EPI_GATEUP>(a, tiles_bound, st)));
  else FP4_CHECK((launch_gemm<GK_FP8, EPI_GATEUP>(a, tiles_bound, st)));
  FP4_CHECK(mark(3));
  // 4. quantization of h (sorted rows; NVFP4 tensor scale over all of h).
  //    Rows of skipped pairs (invalid expert ids, sorted last) hold no h and
  //    are quantized as whatever they hold: their codes are never read (a
  //    tile row past its expert's end reads the expert's first row), the
  //    FP8 / MX scales are per row and per block, and S_h comes from the
  //    gate_up workgroups' maxima over the rows they stored.
  float* h_ts = static_h ? const_cast<float*>(L->inter_scale) : w.h_ts;
  if (!h_in_epilogue) {
    if (h_parts) FP4_CHECK(nv_tensor_scale_from_parts(w.h_amax_part, a.amax_nparts, h_ts, st));
    FP4_CHECK(fp4_quantize(L->a_fmt, FP4_RULE_RTN, (static_h || h_parts) ? FP4_TS_STATIC : FP4_TS_DYNAMIC, w.h,
                           FP4_DT_F32, 1, P, I, w.hq_codes, w.hq_scales, h_ts, nullptr, st));
  }
  FP4_CHECK(mark(4));
  // 5. down -> o
  GemmArgs d = a;
  d.a_codes = w.hq_codes;
  d.a_scales = w.hq_scales;
  d.a_tensor_scale = h_ts;
  d.a_gather = 0;
  d.q_codes = nullptr;
  d.q_scales = nullptr;
  d.amax_part = nullptr;
  d.amax_nparts = 0;
  // the tiled copy of W2 where the down kernel reads it (NVFP4: always; MX
  // and block FP8: on the register-fed kernel)
  d.w_tiled = L->w2_tiled && (gk == GK_NV || mx_down_on_mx2(H, I)) ? 1 : 0;
  d.w_codes = d.w_tiled ? L->w2_tiled : L->w2;
  d.w_scales = d.w_tiled && gk != GK_FP8 ? static_cast<const void*>(L->w2_scale_tiled) : L->w2_scale;
  d.w_tensor_scale = L->w2_scale_2;
  d.K = I;
  d.N = H;
  d.out = nullptr;
  d.out_f16 = reinterpret_cast<_Float16*>(w.o);  // o in fp16: half the bytes the combine reads back
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

extern "C" int moe_fp4_tile_weights(int w_fmt, const uint8_t* codes, const uint8_t* scales, int64_t experts,
                                    int64_t rows, int64_t cols, uint8_t* tiled_codes, uint8_t* tiled_scales,
                                    void* stream) {
  using namespace fp4;
  if (w_fmt != FP4_FMT_NVFP4 && w_fmt != FP4_FMT_MXFP4 && w_fmt != FP4_FMT_FP8_BLOCK)
    return fail(FP4_ERR_UNSUPPORTED, "tile_weights: NVFP4, MXFP4 or block-FP8 weights only (got %d)", w_fmt);
  const bool fp4 = w_fmt != FP4_FMT_FP8_BLOCK;  // E2M1 codes with per-row block scales
  const int SB = w_fmt == FP4_FMT_NVFP4 ? 8 : 4;
  if (experts < 0 || rows < 0 || cols < 0) return fail(FP4_ERR_SHAPE, "tile_weights: negative dimension");
  if (rows % 16 || cols % 128)
    return fail(FP4_ERR_SHAPE, "tile_weights: rows %lld must be a multiple of 16, cols %lld of 128", (long long)rows,
                (long long)cols);
  if (experts == 0 || rows == 0 || cols == 0) return FP4_OK;
  if (!codes || !tiled_codes || (fp4 && (!scales || !tiled_scales)))
    return fail(FP4_ERR_INVALID_ARG, "tile_weights: null pointer");
  if (reinterpret_cast<uintptr_t>(codes) % 16 || reinterpret_cast<uintptr_t>(tiled_codes) % 16 ||
      (fp4 && (reinterpret_cast<uintptr_t>(scales) % SB || reinterpret_cast<uintptr_t>(tiled_scales) % SB)))
    return fail(FP4_ERR_INVALID_ARG, "tile_weights: codes need 16-byte and scales %d-byte alignment", SB);
  const int64_t rows_total = experts * rows;
  const int KS = (int)(cols / 128), PH = fp4 ? 1 : 2;
  const int64_t n = rows_total * KS * PH * 4;  // code chunks (at least the scale groups)
  hipLaunchKernelGGL(tile_weights_kernel, dim3(grid_1d(n, 256)), dim3(256), 0, as_stream(stream), codes,
                     fp4 ? scales : nullptr, rows_total, KS, PH, SB, tiled_codes, fp4 ? tiled_scales : nullptr);
  return check_launch("tile_weights");
}
