// Routed-expert MoE forward behind moe_fp4_forward (gfx950).
//
// Steps (model cards on block_scaled_fp4_nvfp4: stacked [E, out, in] experts
// with fused gate_up, dabsLabs NVFP4 card; top-k routing width and shared
// expert width from the configuration, FP4-Local AZ card):
//   1. permute: stable counting sort of the T*k (token, slot) pairs by expert
//   2. dynamic activation quantization of x (W4A4 / MX / FP8 modes)
//   3. gate_up projection of each pair's token, SiLU(gate) * up -> h (f32)
//   4. quantization of h (same modes)
//   5. down projection of each pair -> o (f32, unweighted)
//   6. combine: y[t] = sum_j w[t, j] * o[row(t, j)] in slot order (+ shared expert)
//
// This file holds the workspace plan, the permutation, the weight-only
// (bf16 activation) GEMV path used at decode sizes, the combine and the
// C entry points; the MFMA grouped GEMMs live in moe_gemm.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "fp4_device.h"
#include "host_common.h"
#include "moe_common.h"
#include "moe_internal.h"

namespace fp4 {

// ------------------------------------------------------------ workspace plan

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// MXFP4 weights x MXFP8 activations at decode sizes (at most 1024 pairs, the
// single-workgroup permutation) take the weight-streaming GEMVs on the exactly
// dequantized MXFP8 activations: every MXFP8 value (E4M3 times a power of two)
// is a bf16 value, so the products and the f32 sums are those of the MFMA
// path up to summation order, while each weight is read once per expert
// instead of once per 64-row tile.
bool w4a8_gemv(const moe_fp4_layer* L, int64_t T) {
  return L->w_fmt == FP4_FMT_MXFP4 && L->a_fmt == FP4_FMT_MXFP8 && T * L->top_k <= 1024 &&
         L->hidden <= 4096 && L->inter <= 1024;
}

int plan_workspace(const moe_fp4_layer* L, int64_t T, WsPlan* w) {
  const int64_t E = L->num_experts, H = L->hidden, I = L->inter, k = L->top_k;
  const int64_t P = T * k;
  const int64_t nb = (P + kPermBlock - 1) / kPermBlock;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + std::max<size_t>(bytes, 1), 256);
    return at;
  };
  WsPlan p{};
  p.error_flag = take(sizeof(int32_t) * 4);
  p.counts = take(sizeof(int32_t) * E);
  p.offsets = take(sizeof(int32_t) * (E + 1));
  p.pair_of_row = take(sizeof(int32_t) * P);
  p.row_of_pair = take(sizeof(int32_t) * P);
  p.active = take(sizeof(int32_t) * (E + 1));
  p.tile_offsets = take(sizeof(int32_t) * (E + 1));
  p.block_counts = take(sizeof(int32_t) * nb * E);
  p.block_invalid = take(sizeof(int32_t) * nb);
  p.x_tensor_scale = take(sizeof(float) * 2);
  p.h_tensor_scale = take(sizeof(float) * 2);
  p.h = take(sizeof(float) * P * I);
  // quantized activations (layout of the activation format)
  size_t xq_codes = 0, xq_scales = 0, hq_codes = 0, hq_scales = 0;
  switch (L->a_fmt) {
    case FP4_FMT_NVFP4:
      xq_codes = T * H / 2; xq_scales = T * H / 16;
      hq_codes = P * I / 2; hq_scales = P * I / 16;
      break;
    case FP4_FMT_MXFP8:
      xq_codes = T * H; xq_scales = T * H / 32;
      hq_codes = P * I; hq_scales = P * I / 32;
      break;
    case FP4_FMT_FP8_ROW:
      xq_codes = T * H; xq_scales = T * H / 128 * 4;
      hq_codes = P * I; hq_scales = P * I / 128 * 4;
      break;
    default: break;
  }
  p.xq_codes = take(xq_codes);
  p.xq_scales = take(xq_scales);
  p.hq_codes = take(hq_codes);
  p.hq_scales = take(hq_scales);
  p.o = take(sizeof(float) * P * H);
  if (w4a8_gemv(L, T)) {
    p.x_deq = take(2 * T * H);
    p.h_deq = take(sizeof(float) * P * I);
  }
  if (L->a_fmt == FP4_FMT_NVFP4) {
    // one per gate_up workgroup: M-tile bound x (I / 64) tiles at most, in
    // whole rounds of the 8 XCDs
    const int64_t tiles = (P + kGemmTileM - 1) / kGemmTileM + std::min<int64_t>(E, P);
    p.h_amax_part = take(sizeof(float) * ((tiles * (I / 64) + 7) / 8 * 8));
  }
  if (L->shared_inter > 0) {
    const int64_t S = L->shared_inter;
    p.sx_codes = take(T * H);
    p.sx_scales = take(T * H / 32);
    p.sh = take(sizeof(float) * T * S);
    p.sh_codes = take(T * S);
    p.sh_scales = take(T * S / 32);
    p.s_out = take(sizeof(float) * T * H);
  }
  p.total = off;
  *w = p;
  return FP4_OK;
}

// ----------------------------------------------------------------- permute

// Exclusive scan of up to three ints per thread over the 1024 threads of one
// workgroup: shuffle scans within each wave, then one wave scans the 16 wave
// totals (two barriers).  Returns the exclusive prefixes in v[] and the
// totals in total[].  `tmp` holds 64 ints of LDS.
template <int NV>
__device__ void block_scan_1024(int (&v)[NV], int* tmp, int (&total)[NV]) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int x[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) x[i] = v[i];
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int y = __shfl_up(x[i], d, 64);
      if (lane >= d) x[i] += y;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < NV; ++i) tmp[i * 16 + w] = x[i];
  }
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int t = lane < 16 ? tmp[i * 16 + lane] : 0;
      int s = t;
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) {
        const int y = __shfl_up(s, d, 64);
        if (lane >= d) s += y;
      }
      if (lane < 16) tmp[i * 16 + lane] = s - t;  // exclusive wave prefix
      if (lane == 15) tmp[48 + i] = s;             // total
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int incl = x[i] + tmp[i * 16 + w];
    total[i] = tmp[48 + i];
    v[i] = incl - v[i];
  }
  __syncthreads();
}

// Counts, offsets, active-expert list and GEMM tile offsets from per-expert
// counts held in `cnt` (global, E ints).  One workgroup of 1024 threads.
__device__ void finish_offsets(const int32_t* cnt, int E, int tile_m, int32_t* offsets,
                               int32_t* active, int32_t* tile_offsets, int* tmp, int* s_off = nullptr) {
  int tid = threadIdx.x;
  int per = (E + 1023) / 1024;
  int lo = min(E, tid * per), hi = min(E, lo + per);
  int s_cnt = 0, s_act = 0, s_tile = 0;
  for (int e = lo; e < hi; ++e) {
    int c = cnt[e];
    s_cnt += c;
    s_act += c > 0;
    s_tile += (c + tile_m - 1) / tile_m;
  }
  int b[3] = {s_cnt, s_act, s_tile}, tot[3];
  block_scan_1024<3>(b, tmp, tot);
  int b_cnt = b[0], b_act = b[1], b_tile = b[2];
  const int tot_cnt = tot[0], tot_act = tot[1], tot_tile = tot[2];
  for (int e = lo; e < hi; ++e) {
    int c = cnt[e];
    offsets[e] = b_cnt;
    if (s_off) s_off[e] = b_cnt;
    tile_offsets[e] = b_tile;
    if (c > 0) active[1 + b_act++] = e;
    b_cnt += c;
    b_tile += (c + tile_m - 1) / tile_m;
  }
  if (tid == 0) {
    offsets[E] = tot_cnt;
    tile_offsets[E] = tot_tile;
    active[0] = tot_act;
  }
}

// Whole permutation in one workgroup of 1024 threads for P <= 1024 pairs
// (decode batches): ranks, histogram, scan and scatter all through LDS.
__global__ void __launch_bounds__(1024) perm_small_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                         int tile_m, int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ pair_of_row,
                                                         int32_t* __restrict__ row_of_pair,
                                                         int32_t* __restrict__ active,
                                                         int32_t* __restrict__ tile_offsets,
                                                         int32_t* __restrict__ error_flag) {
  extern __shared__ __attribute__((aligned(16))) int smem[];
  int* s_ids = smem;            // 1024
  int* tmp = smem + 1024;       // 1024
  int* s_hist = smem + 2048;    // E
  int* s_off = s_hist + E;      // E
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 1024) s_hist[e] = 0;
  int my = -1;
  if (tid < P) {
    int v = ids[tid];
    my = (v >= 0 && v < E) ? v : -2;
  }
  s_ids[tid] = my;
  __syncthreads();
  if (my >= 0) atomicAdd(&s_hist[my], 1);
  // rank among the earlier pairs of the same expert: the earlier ids are
  // read four at a time (16-byte LDS reads, several in flight)
  int r = 0;
  if (my >= 0) {
    const int4* ids4 = reinterpret_cast<const int4*>(s_ids);
    const int full = tid >> 2;
#pragma unroll 4
    for (int q = 0; q < full; ++q) {
      const int4 v = ids4[q];
      r += (v.x == my) + (v.y == my) + (v.z == my) + (v.w == my);
    }
    for (int q = full * 4; q < tid; ++q) r += s_ids[q] == my;
  }
  int bad[1] = {my == -2 ? 1 : 0}, bad_tot[1];
  block_scan_1024<1>(bad, tmp, bad_tot);  // also orders the histogram updates
  const int bad_total = bad_tot[0];
  for (int e = tid; e < E; e += 1024) counts[e] = s_hist[e];
  finish_offsets(s_hist, E, tile_m, offsets, active, tile_offsets, tmp, s_off);
  __syncthreads();
  if (tid < P) {
    if (my >= 0) {
      int row = s_off[my] + r;
      row_of_pair[tid] = row;
      pair_of_row[row] = tid;
    } else {
      row_of_pair[tid] = -1;
    }
  }
  if (tid == 0) error_flag[0] = bad_total;
}

// Pass 1 (grid = ceil(P/256)): per block of 256 consecutive pairs, the rank of
// each pair among the earlier pairs of the block with the same expert, and
// the block's per-expert counts.
__global__ void __launch_bounds__(kPermBlock) perm_count_kernel(const int32_t* __restrict__ ids, int64_t P,
                                                                int E, int32_t* __restrict__ rank,
                                                                int32_t* __restrict__ block_counts,
                                                                int32_t* __restrict__ block_invalid,
                                                                int32_t* __restrict__ scan_done) {
  extern __shared__ int smem[];
  int* s_ids = smem;              // kPermBlock
  int* s_hist = smem + kPermBlock;  // E
  int tid = threadIdx.x;
  int64_t p = (int64_t)blockIdx.x * kPermBlock + tid;
  if ((blockIdx.x | tid) == 0) *scan_done = 0;  // arrivals of the next pass's workgroups
  for (int e = tid; e < E; e += kPermBlock) s_hist[e] = 0;
  int my = -1;
  if (p < P) {
    int v = ids[p];
    my = (v >= 0 && v < E) ? v : -2;
  }
  s_ids[tid] = my;
  __syncthreads();
  if (my >= 0) atomicAdd(&s_hist[my], 1);
  // rank among the earlier pairs of the same expert: the earlier ids are
  // read four at a time (16-byte LDS reads, several in flight)
  int r = 0;
  if (my >= 0) {
    const int4* ids4 = reinterpret_cast<const int4*>(s_ids);
    const int full = tid >> 2;
#pragma unroll 4
    for (int q = 0; q < full; ++q) {
      const int4 v = ids4[q];
      r += (v.x == my) + (v.y == my) + (v.z == my) + (v.w == my);
    }
    for (int q = full * 4; q < tid; ++q) r += s_ids[q] == my;
  }
  __syncthreads();
  if (p < P) rank[p] = my >= 0 ? r : -1;
  for (int e = tid; e < E; e += kPermBlock) block_counts[(int64_t)blockIdx.x * E + e] = s_hist[e];
  if (tid == 0) {
    int bad = 0;
    for (int q = 0; q < kPermBlock; ++q) bad += s_ids[q] == -2;
    block_invalid[blockIdx.x] = bad;
  }
}

// Pass 2 (grid = ceil(E/64) workgroups of 1024): per-expert running sums
// over blocks, turning block_counts into block bases.  Lane l of every wave
// takes expert 64 x + l (coalesced rows of block_counts), wave w the w-th
// sixteenth of the blocks; a workgroup adds up its waves' parts in LDS, then
// rewrites its columns.  Each workgroup stores its experts' totals at device
// scope (written through to memory), waits for them, and counts itself in
// scan_done (zeroed by pass 1); the last to arrive reads every total back at
// device scope and writes the offsets, the active list, the tile offsets and
// the error flag.  No workgroup waits for another.
__global__ void __launch_bounds__(1024) perm_scan_kernel(int nb, int E, int tile_m,
                                                         int32_t* __restrict__ block_counts,
                                                         const int32_t* __restrict__ block_invalid,
                                                         int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ active,
                                                         int32_t* __restrict__ tile_offsets,
                                                         int32_t* __restrict__ error_flag,
                                                         int32_t* __restrict__ scan_done) {
  extern __shared__ int s_cnt[];  // E: the last workgroup's copy of the totals
  __shared__ int tmp[64];
  __shared__ int s_part[16][64];
  __shared__ int s_last;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 64 + lane;
  const int per = (nb + 15) / 16;
  const int b0 = min(nb, wave * per), b1 = min(nb, b0 + per);
  int32_t* col = block_counts + e;
  int sum = 0;
  if (e < E) {
    int b = b0;
    for (; b + 8 <= b1; b += 8) {  // 8 independent loads in flight
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = col[(int64_t)(b + u) * E];
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += c[u];
    }
    for (; b < b1; ++b) sum += col[(int64_t)b * E];
  }
  s_part[wave][lane] = sum;
  __syncthreads();
  int run = 0;
  for (int w = 0; w < wave; ++w) run += s_part[w][lane];
  if (e < E) {
    int b = b0;
    for (; b + 8 <= b1; b += 8) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = col[(int64_t)(b + u) * E];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        col[(int64_t)(b + u) * E] = run;
        run += c[u];
      }
    }
    for (; b < b1; ++b) {
      const int c = col[(int64_t)b * E];
      col[(int64_t)b * E] = run;
      run += c;
    }
    if (wave == 15) __hip_atomic_store(counts + e, run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // wave 15 ends at nb
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores acknowledged
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(scan_done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (int)gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  for (int i = threadIdx.x; i < E; i += 1024) s_cnt[i] = __hip_atomic_load(counts + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int bad[1] = {0}, bad_tot[1];
  for (int b = threadIdx.x; b < nb; b += 1024) bad[0] += block_invalid[b];
  block_scan_1024<1>(bad, tmp, bad_tot);
  const int tot_bad = bad_tot[0];
  __syncthreads();
  finish_offsets(s_cnt, E, tile_m, offsets, active, tile_offsets, tmp);
  if (threadIdx.x == 0) error_flag[0] = tot_bad;
}

// Pass 3 (grid = ceil(P/256)): sorted row of every pair.
__global__ void __launch_bounds__(kPermBlock) perm_scatter_kernel(const int32_t* __restrict__ ids, int64_t P,
                                                                  int E, const int32_t* __restrict__ block_base,
                                                                  const int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ row_of_pair,
                                                                  int32_t* __restrict__ pair_of_row) {
  int64_t p = (int64_t)blockIdx.x * kPermBlock + threadIdx.x;
  if (p >= P) return;
  int r = row_of_pair[p];  // rank written by pass 1
  if (r < 0) {
    row_of_pair[p] = -1;
    return;
  }
  int e = ids[p];
  int row = offsets[e] + block_base[(int64_t)blockIdx.x * E + e] + r;
  row_of_pair[p] = row;
  pair_of_row[row] = (int32_t)p;
}

int launch_permute(const int32_t* ids, int64_t P, int E, int tile_m, const WsPtrs& w, hipStream_t st) {
  if (P <= 1024 && E <= 4096) {
    size_t lds = sizeof(int) * (2048 + 2 * (size_t)E);
    hipLaunchKernelGGL(perm_small_kernel, dim3(1), dim3(1024), lds, st, ids, (int)P, E, tile_m, w.counts,
                       w.offsets, w.pair_of_row, w.row_of_pair, w.active, w.tile_offsets, w.error_flag);
    return check_launch("perm_small");
  }
  int64_t nb = (P + kPermBlock - 1) / kPermBlock;
  if (nb == 0) nb = 1;  // still writes counts/offsets for P == 0
  size_t lds = sizeof(int) * (kPermBlock + E);
  int32_t* scan_done = w.error_flag + 1;
  hipLaunchKernelGGL(perm_count_kernel, dim3((unsigned)nb), dim3(kPermBlock), lds, st, ids, P, E,
                     w.row_of_pair, w.block_counts, w.block_invalid, scan_done);
  FP4_CHECK(check_launch("perm_count"));
  hipLaunchKernelGGL(perm_scan_kernel, dim3((unsigned)((E + 63) / 64)), dim3(1024), sizeof(int) * (size_t)E, st,
                     (int)nb, E, tile_m, w.block_counts, w.block_invalid, w.counts, w.offsets, w.active,
                     w.tile_offsets, w.error_flag, scan_done);
  FP4_CHECK(check_launch("perm_scan"));
  if (P > 0) {
    hipLaunchKernelGGL(perm_scatter_kernel, dim3((unsigned)nb), dim3(kPermBlock), 0, st, ids, P, E,
                       w.block_counts, w.offsets, w.row_of_pair, w.pair_of_row);
    FP4_CHECK(check_launch("perm_scatter"));
  }
  return FP4_OK;
}

// --------------------------------------------- weight-only GEMV path (decode)

template <int WFMT>
__device__ __forceinline__ int64_t scale_row_stride(int64_t cols) {
  return WFMT == FP4_FMT_NVFP4 ? cols / 16 : cols / 32;
}

// Scale bytes of 16-byte code chunk c (32 values) of a weight row: NVFP4 has
// two E4M3 scales (bytes 2c, 2c+1), MXFP4 one UE8M0 scale (byte c).
template <int WFMT>
__device__ __forceinline__ uint32_t chunk_scale_bits(const uint8_t* srow, int c) {
  if (WFMT == FP4_FMT_NVFP4) return *reinterpret_cast<const uint16_t*>(srow + 2 * c);
  return srow[c];
}

// Value of scale byte SEL (0 or 1) of a chunk's scale bits.
template <int WFMT, int SEL>
__device__ __forceinline__ float chunk_scale(uint32_t bits) {
  if (WFMT == FP4_FMT_NVFP4) return __builtin_amdgcn_cvt_f32_fp8((int)bits, SEL);
  return bits ? __uint_as_float(bits << 23) : 5.877471754111438e-39f;  // UE8M0 2^(c-127); c = 0: 2^-127
}

// acc + scale-weighted dot product of one 32-value code chunk with 32 bf16
// activations (x[q] holds the pair (2q, 2q+1)).  NVFP4: two 16-value blocks,
// each partial sum scaled by its own block scale; MXFP4: one block.
template <int WFMT>
__device__ __forceinline__ float chunk_dot_bf16(u32x4 c, uint32_t sbits, const uint32_t (&x)[16], float acc) {
  uint32_t p[16];
  e2m1x8_to_bf16x8(c.x, *reinterpret_cast<uint32_t(*)[4]>(&p[0]));
  e2m1x8_to_bf16x8(c.y, *reinterpret_cast<uint32_t(*)[4]>(&p[4]));
  e2m1x8_to_bf16x8(c.z, *reinterpret_cast<uint32_t(*)[4]>(&p[8]));
  e2m1x8_to_bf16x8(c.w, *reinterpret_cast<uint32_t(*)[4]>(&p[12]));
  float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
  for (int q = 0; q < 8; ++q) d0 = dot2_bf16(p[q], x[q], d0);
#pragma unroll
  for (int q = 8; q < 16; ++q) d1 = dot2_bf16(p[q], x[q], d1);
  if (WFMT == FP4_FMT_NVFP4) return fmaf(d1, chunk_scale<WFMT, 1>(sbits), fmaf(d0, chunk_scale<WFMT, 0>(sbits), acc));
  return fmaf(d0 + d1, chunk_scale<WFMT, 0>(sbits), acc);
}

// Same with f32 activations h[0..31].
template <int WFMT>
__device__ __forceinline__ float chunk_dot_f32(u32x4 c, uint32_t sbits, const float (&h)[32], float acc) {
  float d0 = 0.0f, d1 = 0.0f;
  float w[8];
  e2m1x8_to_f32x8(c.x, w);
#pragma unroll
  for (int m = 0; m < 8; ++m) d0 = fmaf(w[m], h[m], d0);
  e2m1x8_to_f32x8(c.y, w);
#pragma unroll
  for (int m = 0; m < 8; ++m) d0 = fmaf(w[m], h[8 + m], d0);
  e2m1x8_to_f32x8(c.z, w);
#pragma unroll
  for (int m = 0; m < 8; ++m) d1 = fmaf(w[m], h[16 + m], d1);
  e2m1x8_to_f32x8(c.w, w);
#pragma unroll
  for (int m = 0; m < 8; ++m) d1 = fmaf(w[m], h[24 + m], d1);
  if (WFMT == FP4_FMT_NVFP4) return fmaf(d1, chunk_scale<WFMT, 1>(sbits), fmaf(d0, chunk_scale<WFMT, 0>(sbits), acc));
  return fmaf(d0 + d1, chunk_scale<WFMT, 0>(sbits), acc);
}

constexpr int kGvRounds = 1;    // rounds of 16 outputs per workgroup of the gate_up GEMV
constexpr int kGvOut = 16 * kGvRounds;
constexpr int kGvTokens = 4;    // tokens whose activations are staged in LDS per pass
constexpr int kGdRpg = 1;            // output rows per 4 lanes of the down GEMV
constexpr int kGdRows = 64 * kGdRpg;  // output rows per workgroup of the down GEMV
constexpr int kGdTokens = 8;

// One DMA instruction: lane l copies 16 bytes from its global address to LDS
// address lds + 16 l (lds is wave-uniform).
__device__ __forceinline__ void dma16_to_lds(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// Activation staging shared by both GEMVs: all of a pass's rows are copied
// into LDS by DMA instructions issued after the weight loads, then every
// wave waits for all of its loads (the weights are needed right after
// anyway) and the workgroup synchronises.  Vector loads into registers
// would instead have to wait for the older weight loads before their LDS
// stores could be issued, serialising two memory latencies.

// gate_up + SiLU*up for the pairs of one expert, bf16 activations.
// Grid: (ceil(I / (16 kGvRounds)), max active experts).  Each group of 16
// lanes owns one output j per round (rounds 16 apart): gate row j and up
// row I+j, split into 16-byte chunks of 32 codes (lane l takes chunks l,
// l+16, ...).  Every round's codes and scales are loaded up front (about
// 2.9 KB per group and round at the decode shape) and reused for every
// token of the expert.  One round (46 KB per workgroup, twice the
// workgroups of two rounds) streams the weights faster than two or three.
// The tokens' activations are staged in LDS, four tokens per pass,
// as [token][quarter q][chunk c] 16-byte pieces (rows padded to a multiple
// of 64 chunks for the DMA) so that the 16 lanes of a group read consecutive
// pieces.
template <int WFMT, int CPL>
__global__ void __launch_bounds__(256) gemv_gateup_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ pair_of_row, const int32_t* __restrict__ active,
    const uint8_t* __restrict__ w13, const uint8_t* __restrict__ w13s, const float* __restrict__ w13s2,
    int H, int I, int k, float* __restrict__ h) {
  constexpr int CPAD = (16 * CPL + 63) / 64 * 64;  // chunks per staged (token, quarter) row
  __shared__ __attribute__((aligned(16))) uint8_t xs[kGvTokens * 4 * CPAD * 16];
  const int ai = blockIdx.y;
  if (ai >= active[0]) return;
  const int e = active[1 + ai];
  const int tid = threadIdx.x, l = tid & 15, wave = tid >> 6, lane = tid & 63;
  const int NCH = H >> 5;  // 32-value chunks per row
  const int64_t row_bytes = H >> 1;
  const int64_t srow = scale_row_stride<WFMT>(H);
  int jr[kGvRounds];
  u32x4 cg[kGvRounds][CPL], cu[kGvRounds][CPL];
  uint32_t bg[kGvRounds][CPL], bu[kGvRounds][CPL];
  auto load_round = [&](int rd) __attribute__((always_inline)) {
    const int j = blockIdx.x * kGvOut + rd * 16 + (tid >> 4);
    jr[rd] = j;
    const int jj = j < I ? j : I - 1;
    const uint8_t* wg = w13 + ((int64_t)e * 2 * I + jj) * row_bytes;
    const uint8_t* wu = wg + (int64_t)I * row_bytes;
    const uint8_t* sg = w13s + ((int64_t)e * 2 * I + jj) * srow;
    const uint8_t* su = sg + (int64_t)I * srow;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = l + 16 * i;
      const int cc = c < NCH ? c : 0;
      cg[rd][i] = ld16(wg + 16 * cc);
      cu[rd][i] = ld16(wu + 16 * cc);
      // chunks past the row (c >= NCH) load chunk 0 and are skipped by the
      // dot products; nothing here waits for a load
      bg[rd][i] = chunk_scale_bits<WFMT>(sg, cc);
      bu[rd][i] = chunk_scale_bits<WFMT>(su, cc);
    }
  };
  const float S = WFMT == FP4_FMT_NVFP4 ? w13s2[e] : 1.0f;
  const int r0 = __builtin_amdgcn_readfirstlane(offsets[e]);
  const int n = __builtin_amdgcn_readfirstlane(offsets[e + 1]) - r0;
  // DMA of the activation rows (t, q), t < nt, of one pass: the 4 waves take
  // the 4 quarters q; each row of CPAD chunks is CPAD/64 instructions
  // (padding lanes re-read the last chunk)
  auto stage = [&](int t0) __attribute__((always_inline)) {
    const int nt = min(kGvTokens, n - t0);
    for (int t = 0; t < nt; ++t) {
      const int tok = __builtin_amdgcn_readfirstlane(pair_of_row[r0 + t0 + t]) / k;
      const uint8_t* xrow = reinterpret_cast<const uint8_t*>(x + (int64_t)tok * H) + 16 * wave;
#pragma unroll
      for (int m = 0; m < CPAD / 64; ++m) {
        const int c = min(64 * m + lane, NCH - 1);
        dma16_to_lds(xrow + 64 * c, xs + ((t * 4 + wave) * CPAD + 64 * m) * 16);
      }
    }
  };
  // one token of a pass (t < number of tokens in the pass)
  auto token = [&](int t0, int t) __attribute__((always_inline)) {
    {
      // an opaque zero per token, XORed into the codes and scale bits: keeps
      // the packed codes (not their 4x larger bf16 expansion) live across the
      // token loop, and nothing derived from the weight loads is hoisted
      // ahead of the activation staging
      uint32_t z;
      asm volatile("v_mov_b32 %0, 0" : "=v"(z));
      const u32x4 zz = u32x4{z, z, z, z};
#pragma unroll
      for (int rd = 0; rd < kGvRounds; ++rd) {
        float ag = 0.0f, au = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const int c = l + 16 * i;
          if (c < NCH) {
            uint32_t xv[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const u32x4 v = ld16(xs + ((t * 4 + q) * CPAD + c) * 16);
              xv[4 * q] = v.x; xv[4 * q + 1] = v.y; xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
            }
            ag = chunk_dot_bf16<WFMT>(cg[rd][i] ^ zz, bg[rd][i] ^ z, xv, ag);
            au = chunk_dot_bf16<WFMT>(cu[rd][i] ^ zz, bu[rd][i] ^ z, xv, au);
          }
        }
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) {
          ag += __shfl_xor(ag, off, 16);
          au += __shfl_xor(au, off, 16);
        }
        if (l == 0 && jr[rd] < I) h[(int64_t)(r0 + t0 + t) * I + jr[rd]] = silu_f32(ag * S) * (au * S);
      }
    }
  };
  // the first token is peeled out of the token loop: a loop that uses
  // registers loaded before it starts with a wait for all of them
  auto compute = [&](int t0) __attribute__((always_inline)) {
    const int nt = min(kGvTokens, n - t0);
    if (nt > 0) token(t0, 0);
    for (int t = 1; t < nt; ++t) token(t0, t);
  };
  // First pass: round 0's weights, then the activation DMA, then the later
  // rounds' weights, so that waiting for the DMA (vmcnt counts in issue
  // order) leaves the later rounds in flight while round 0 is computed.
  load_round(0);
  stage(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int rd = 1; rd < kGvRounds; ++rd) load_round(rd);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(4 * CPL * (kGvRounds - 1)));
  asm volatile("s_barrier" ::: "memory");
  compute(0);
  for (int t0 = kGvTokens; t0 < n; t0 += kGvTokens) {
    __syncthreads();  // the previous pass's reads are done
    stage(t0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    compute(t0);
  }
}

// Down projection o[row] = W2[e] h[row] for the rows of one expert, f32 h.
// Grid: (ceil(H / (64 kGdRpg)), max active experts).  Each group of 4 lanes
// owns kGdRpg output rows (n, n + 64, ... of the tile; one row measured
// faster than two), each split into 16-byte chunks of 32
// codes (lane l takes chunks l, l+4, ...).  The tokens' h rows are staged in
// LDS, eight tokens per pass; the eight 16-byte pieces of chunk c sit in
// XOR-swizzled order (piece q at slot q ^ (c & 3)) so that the four lanes of
// a group, which read four consecutive chunks, hit different bank groups.
template <int WFMT, int CPL>
__global__ void __launch_bounds__(256) gemv_down_kernel(
    const float* __restrict__ h, const int32_t* __restrict__ offsets, const int32_t* __restrict__ active,
    const uint8_t* __restrict__ w2, const uint8_t* __restrict__ w2s, const float* __restrict__ w2s2,
    int H, int I, float* __restrict__ o) {
  constexpr int NCP = (4 * CPL + 7) / 8 * 8;  // staged chunks per token (a DMA instruction covers 8)
  constexpr int TOKB = NCP * 128;             // staged bytes per token
  __shared__ __attribute__((aligned(16))) uint8_t hs[kGdTokens * TOKB];
  const int ai = blockIdx.y;
  if (ai >= active[0]) return;
  const int e = active[1 + ai];
  const int tid = threadIdx.x, l = tid & 3, wave = tid >> 6, lane = tid & 63;
  const int NCH = I >> 5;
  const int64_t row_bytes = I >> 1;
  const int64_t srow = scale_row_stride<WFMT>(I);
  const uint8_t* wbase = w2 + (int64_t)e * H * row_bytes;
  const uint8_t* sbase = w2s + (int64_t)e * H * srow;
  int nr[kGdRpg];
  u32x4 cw[kGdRpg][CPL];
  uint32_t bw[kGdRpg][CPL];
#pragma unroll
  for (int r = 0; r < kGdRpg; ++r) {
    nr[r] = blockIdx.x * kGdRows + (tid >> 2) + 64 * r;
    const int64_t row = nr[r] < H ? nr[r] : 0;
    const uint8_t* q = wbase + row * row_bytes;
    const uint8_t* sp = sbase + row * srow;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = l + 4 * i;
      const int cc = c < NCH ? c : 0;
      cw[r][i] = ld16(q + 16 * cc);
      bw[r][i] = chunk_scale_bits<WFMT>(sp, cc);  // chunks c >= NCH are skipped by the dot products
    }
  }
  const float S = WFMT == FP4_FMT_NVFP4 ? w2s2[e] : 1.0f;
  const int r0 = __builtin_amdgcn_readfirstlane(offsets[e]);
  const int n = __builtin_amdgcn_readfirstlane(offsets[e + 1]) - r0;
  auto pass = [&](int t0) __attribute__((always_inline)) {  // first pass peeled, as in gate_up
    const int nt = min(kGdTokens, n - t0);
    if (t0 > 0) __syncthreads();
    // DMA: wave w stages tokens w, w + 4 of the pass; per token, instruction m
    // covers chunks 8m .. 8m+7 (lane = 8 * (c - 8m) + slot; padding chunks re-read the last one)
    for (int t = wave; t < nt; t += 4) {
      const uint8_t* hrow = reinterpret_cast<const uint8_t*>(h + (int64_t)(r0 + t0 + t) * I);
#pragma unroll
      for (int m = 0; m < NCP / 8; ++m) {
        const int c = min(8 * m + (lane >> 3), NCH - 1), slot = lane & 7;
        const int q = slot ^ ((8 * m + (lane >> 3)) & 3);
        dma16_to_lds(hrow + 128 * c + 16 * q, hs + t * TOKB + 8 * m * 128);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = 0; t < nt; ++t) {
      uint32_t z;  // opaque zero: the f32 expansion of the codes stays per token
      asm volatile("v_mov_b32 %0, 0" : "=v"(z));
      const u32x4 zz = u32x4{z, z, z, z};
      float a[kGdRpg];
#pragma unroll
      for (int r = 0; r < kGdRpg; ++r) a[r] = 0.0f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = l + 4 * i;
        if (c < NCH) {
          float hv[32];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const u32x4 v = ld16(hs + t * TOKB + c * 128 + 16 * (q ^ (c & 3)));
            hv[4 * q] = __uint_as_float(v.x); hv[4 * q + 1] = __uint_as_float(v.y);
            hv[4 * q + 2] = __uint_as_float(v.z); hv[4 * q + 3] = __uint_as_float(v.w);
          }
#pragma unroll
          for (int r = 0; r < kGdRpg; ++r) a[r] = chunk_dot_f32<WFMT>(cw[r][i] ^ zz, bw[r][i] ^ z, hv, a[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < kGdRpg; ++r) {
#pragma unroll
        for (int off = 2; off > 0; off >>= 1) a[r] += __shfl_xor(a[r], off, 4);
        if (l == 0 && nr[r] < H) o[(int64_t)(r0 + t0 + t) * H + nr[r]] = a[r] * S;
      }
    }
  };
  if (n > 0) pass(0);
  for (int t0 = kGdTokens; t0 < n; t0 += kGdTokens) pass(t0);
}

// ------------------------------------------------------------------ routing

// Top-k routing of one token per wave: l'_e = fp32(logit_e + bias_e); the k
// largest l' in order (equal values: lower expert id first); weights = the
// softmax over the k selected l' (the renormalized top-k softmax), in fp64,
// rounded once to f32.  Lane i holds experts i, i + 64, ... (up to PL each).
template <int PL>
__global__ void __launch_bounds__(256) route_topk_kernel(const float* __restrict__ logits,
                                                         const float* __restrict__ bias, int64_t T, int E,
                                                         int k, int32_t* __restrict__ ids,
                                                         float* __restrict__ weights) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  float v[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? logits[t * E + e] + (bias ? bias[e] : 0.0f) : -__builtin_huge_valf();
  }
  float sel = 0.0f;   // lane j < k keeps the j-th selected value
  float top = 0.0f;   // the largest selected value
  for (int j = 0; j < k; ++j) {
    // this lane's best: largest value, lowest expert id among equals
    float bv = v[0];
    int be = lane;
#pragma unroll
    for (int i = 1; i < PL; ++i)
      if (v[i] > bv) { bv = v[i]; be = lane + 64 * i; }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
    if (j == 0) top = bv;
    if (lane == j) sel = bv;
    if ((be & 63) == lane) {
#pragma unroll
      for (int i = 0; i < PL; ++i)
        if (lane + 64 * i == be) v[i] = -__builtin_huge_valf();
    }
    if (lane == 0) ids[t * k + j] = be;
  }
  const double z = lane < k ? exp((double)sel - (double)top) : 0.0;
  double sum = z;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  sum = __shfl(sum, 0);  // one summation order for every weight of the token
  if (lane < k) weights[t * k + lane] = (float)(z / sum);
}

// ------------------------------------------------------------------ combine

constexpr int kMaxTopK = 32;

// y[t, :] = sum_j w[t, j] * o[row(t, j), :] (+ extra[t, :]), in slot order, f32.
// The k slots are taken CW at a time: a chunk's row indices and weights are
// read before its o loads are issued.  CW is the smallest of 4, 8, 12, 16
// that covers k (16 and a loop above that), so the registers, and with them
// the waves in flight per SIMD, follow the routing width instead of its
// maximum.
template <int CW>
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ o,
                                                      const int32_t* __restrict__ row_of_pair,
                                                      const float* __restrict__ topk_w, int64_t T, int H,
                                                      int k, const float* __restrict__ extra,
                                                      float* __restrict__ y) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one float4 of y
  int64_t per_row = H / 4;
  if (i >= T * per_row) return;
  int64_t t = i / per_row, c4 = i - t * per_row;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < k; j0 += CW) {
    int rows[CW];
    float w[CW];
#pragma unroll
    for (int u = 0; u < CW; ++u)
      if (j0 + u < k) {
        rows[u] = row_of_pair[t * k + j0 + u];
        w[u] = topk_w[t * k + j0 + u];
      }
    float4 v[CW];
#pragma unroll
    for (int u = 0; u < CW; ++u)
      if (j0 + u < k && rows[u] >= 0) v[u] = reinterpret_cast<const float4*>(o + (int64_t)rows[u] * H)[c4];
#pragma unroll
    for (int u = 0; u < CW; ++u)
      if (j0 + u < k && rows[u] >= 0) {
        acc.x = fmaf(w[u], v[u].x, acc.x);
        acc.y = fmaf(w[u], v[u].y, acc.y);
        acc.z = fmaf(w[u], v[u].z, acc.z);
        acc.w = fmaf(w[u], v[u].w, acc.w);
      }
  }
  if (extra) {
    float4 e = reinterpret_cast<const float4*>(extra + t * H)[c4];
    acc.x += e.x; acc.y += e.y; acc.z += e.z; acc.w += e.w;
  }
  reinterpret_cast<float4*>(y + t * H)[c4] = acc;
}

// The same combine over o in fp16 (the grouped path's down GEMMs leave it
// so; passed as its bit patterns, which keeps the kernel's name readable in
// profiler output): eight outputs per thread, one 16-byte load of o per
// slot, the sum in f32 in the same slot order.
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

template <int CW>
__global__ void __launch_bounds__(256) combine_f16_kernel(const uint16_t* __restrict__ o,
                                                          const int32_t* __restrict__ row_of_pair,
                                                          const float* __restrict__ topk_w, int64_t T, int H,
                                                          int k, const float* __restrict__ extra,
                                                          float* __restrict__ y) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // eight consecutive floats of y
  int64_t per_row = H / 8;
  if (i >= T * per_row) return;
  int64_t t = i / per_row, c8 = i - t * per_row;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  for (int j0 = 0; j0 < k; j0 += CW) {
    int rows[CW];
    float w[CW];
#pragma unroll
    for (int u = 0; u < CW; ++u)
      if (j0 + u < k) {
        rows[u] = row_of_pair[t * k + j0 + u];
        w[u] = topk_w[t * k + j0 + u];
      }
    half8_t v[CW];
#pragma unroll
    for (int u = 0; u < CW; ++u)
      if (j0 + u < k && rows[u] >= 0) v[u] = reinterpret_cast<const half8_t*>(o + (int64_t)rows[u] * H)[c8];
#pragma unroll
    for (int u = 0; u < CW; ++u)
      if (j0 + u < k && rows[u] >= 0) {
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = fmaf(w[u], (float)v[u][q], acc[q]);
      }
  }
  if (extra) {
    const float4* e = reinterpret_cast<const float4*>(extra + t * H) + 2 * c8;
    const float4 e0 = e[0], e1 = e[1];
    acc[0] += e0.x; acc[1] += e0.y; acc[2] += e0.z; acc[3] += e0.w;
    acc[4] += e1.x; acc[5] += e1.y; acc[6] += e1.z; acc[7] += e1.w;
  }
  float4* yo = reinterpret_cast<float4*>(y + t * H) + 2 * c8;
  yo[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  yo[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

static void launch_combine(const void* o, bool o_f16, const int32_t* row_of_pair, const float* topk_w, int64_t T,
                           int H, int k, const float* extra, float* y, hipStream_t st) {
  if (o_f16) {
    const uint16_t* oh = static_cast<const uint16_t*>(o);
    const dim3 grid(grid_1d(T * H / 8, 256)), block(256);
    if (k <= 4) hipLaunchKernelGGL(combine_f16_kernel<4>, grid, block, 0, st, oh, row_of_pair, topk_w, T, H, k, extra, y);
    else if (k <= 8) hipLaunchKernelGGL(combine_f16_kernel<8>, grid, block, 0, st, oh, row_of_pair, topk_w, T, H, k, extra, y);
    else if (k <= 12) hipLaunchKernelGGL(combine_f16_kernel<12>, grid, block, 0, st, oh, row_of_pair, topk_w, T, H, k, extra, y);
    else hipLaunchKernelGGL(combine_f16_kernel<16>, grid, block, 0, st, oh, row_of_pair, topk_w, T, H, k, extra, y);
    return;
  }
  const float* of = static_cast<const float*>(o);
  const dim3 grid(grid_1d(T * H / 4, 256)), block(256);
  if (k <= 4) hipLaunchKernelGGL(combine_kernel<4>, grid, block, 0, st, of, row_of_pair, topk_w, T, H, k, extra, y);
  else if (k <= 8) hipLaunchKernelGGL(combine_kernel<8>, grid, block, 0, st, of, row_of_pair, topk_w, T, H, k, extra, y);
  else if (k <= 12) hipLaunchKernelGGL(combine_kernel<12>, grid, block, 0, st, of, row_of_pair, topk_w, T, H, k, extra, y);
  else hipLaunchKernelGGL(combine_kernel<16>, grid, block, 0, st, of, row_of_pair, topk_w, T, H, k, extra, y);
}

// ---------------------------------------------------------- GEMV dispatch

template <int WFMT>
static int launch_gemv(const uint16_t* x, const WsPtrs& w, const moe_fp4_layer* L, int64_t P,
                       int max_active, hipStream_t st, const Marker& mark, bool requant_h = false) {
  const int cpl = (L->hidden / 32 + 15) / 16;
  dim3 grid((unsigned)((L->inter + kGvOut - 1) / kGvOut), (unsigned)max_active);
#define FP4_GV(B)                                                                                      \
  case B:                                                                                              \
    hipLaunchKernelGGL((gemv_gateup_kernel<WFMT, B>), grid, dim3(256), 0, st, x, w.offsets,            \
                       w.pair_of_row, w.active, L->w13, (const uint8_t*)L->w13_scale, L->w13_scale_2, \
                       L->hidden, L->inter, L->top_k, w.h);                                            \
    break;
  switch (cpl) {
    FP4_GV(1) FP4_GV(2) FP4_GV(3) FP4_GV(4) FP4_GV(5) FP4_GV(6) FP4_GV(7) FP4_GV(8)
    default: return fail(FP4_ERR_UNSUPPORTED, "hidden %d too large for the GEMV path", L->hidden);
  }
#undef FP4_GV
  FP4_CHECK(check_launch("gemv_gateup"));
  FP4_CHECK(mark(3));
  const float* hin = w.h;
  if (requant_h) {  // rows past the valid pairs hold no h; their blocks are never read back
    FP4_CHECK(mxfp8_quantize_dequant(w.h, FP4_DT_F32, P, L->inter, w.hq_codes,
                                     reinterpret_cast<uint8_t*>(w.hq_scales), w.h_deq, FP4_DT_F32, st));
    hin = w.h_deq;
  }
  FP4_CHECK(mark(4));
  const int cpl2 = (L->inter / 32 + 3) / 4;
  dim3 grid2((unsigned)((L->hidden + kGdRows - 1) / kGdRows), (unsigned)max_active);
#define FP4_GD(B)                                                                                      \
  case B:                                                                                              \
    hipLaunchKernelGGL((gemv_down_kernel<WFMT, B>), grid2, dim3(256), 0, st, hin, w.offsets, w.active, \
                       L->w2, (const uint8_t*)L->w2_scale, L->w2_scale_2, L->hidden, L->inter, w.o);   \
    break;
  switch (cpl2) {
    FP4_GD(1) FP4_GD(2) FP4_GD(3) FP4_GD(4) FP4_GD(5) FP4_GD(6) FP4_GD(7) FP4_GD(8)
    default: return fail(FP4_ERR_UNSUPPORTED, "inter %d too large for the GEMV path", L->inter);
  }
#undef FP4_GD
  FP4_CHECK(check_launch("gemv_down"));
  return mark(5);
}

WsPtrs ws_pointers(const WsPlan& p, void* base) {
  char* b = reinterpret_cast<char*>(base);
  WsPtrs w;
  w.error_flag = reinterpret_cast<int32_t*>(b + p.error_flag);
  w.counts = reinterpret_cast<int32_t*>(b + p.counts);
  w.offsets = reinterpret_cast<int32_t*>(b + p.offsets);
  w.pair_of_row = reinterpret_cast<int32_t*>(b + p.pair_of_row);
  w.row_of_pair = reinterpret_cast<int32_t*>(b + p.row_of_pair);
  w.active = reinterpret_cast<int32_t*>(b + p.active);
  w.tile_offsets = reinterpret_cast<int32_t*>(b + p.tile_offsets);
  w.block_counts = reinterpret_cast<int32_t*>(b + p.block_counts);
  w.block_invalid = reinterpret_cast<int32_t*>(b + p.block_invalid);
  w.x_ts = reinterpret_cast<float*>(b + p.x_tensor_scale);
  w.h_ts = reinterpret_cast<float*>(b + p.h_tensor_scale);
  w.h = reinterpret_cast<float*>(b + p.h);
  w.xq_codes = reinterpret_cast<uint8_t*>(b + p.xq_codes);
  w.xq_scales = b + p.xq_scales;
  w.hq_codes = reinterpret_cast<uint8_t*>(b + p.hq_codes);
  w.hq_scales = b + p.hq_scales;
  w.o = reinterpret_cast<float*>(b + p.o);
  w.sx_codes = reinterpret_cast<uint8_t*>(b + p.sx_codes);
  w.sx_scales = reinterpret_cast<uint8_t*>(b + p.sx_scales);
  w.sh = reinterpret_cast<float*>(b + p.sh);
  w.sh_codes = reinterpret_cast<uint8_t*>(b + p.sh_codes);
  w.sh_scales = reinterpret_cast<uint8_t*>(b + p.sh_scales);
  w.s_out = reinterpret_cast<float*>(b + p.s_out);
  w.x_deq = reinterpret_cast<uint16_t*>(b + p.x_deq);
  w.h_deq = reinterpret_cast<float*>(b + p.h_deq);
  w.h_amax_part = reinterpret_cast<float*>(b + p.h_amax_part);
  return w;
}

static int validate_layer(const moe_fp4_layer* L, int64_t T) {
  if (!L) return fail(FP4_ERR_INVALID_ARG, "null layer");
  if (T < 0) return fail(FP4_ERR_SHAPE, "negative token count");
  if (L->num_experts < 1 || L->hidden < 1 || L->inter < 1)
    return fail(FP4_ERR_SHAPE, "experts, hidden and inter must be positive");
  if (L->top_k < 1 || L->top_k > L->num_experts || L->top_k > kMaxTopK)
    return fail(FP4_ERR_INVALID_ARG, "top_k %d outside [1, %d]", L->top_k, L->num_experts);
  if (L->num_experts > kMaxExperts) return fail(FP4_ERR_UNSUPPORTED, "more than %d experts", kMaxExperts);
  const int w = L->w_fmt, a = L->a_fmt;
  bool ok = (w == FP4_FMT_NVFP4 && (a == FP4_FMT_NONE || a == FP4_FMT_NVFP4)) ||
            (w == FP4_FMT_MXFP4 && (a == FP4_FMT_NONE || a == FP4_FMT_MXFP8)) ||
            (w == FP4_FMT_FP8_BLOCK && a == FP4_FMT_FP8_ROW);
  if (!ok) return fail(FP4_ERR_UNSUPPORTED, "format pair (w=%d, a=%d) not provided", w, a);
  // 32: the weight-only GEMV reads weight rows in chunks of 32 codes
  int blk = 32;
  if (w == FP4_FMT_FP8_BLOCK) blk = 128;
  if (a != FP4_FMT_NONE) blk = std::max(blk, 32);
  if (L->hidden % blk || L->inter % blk)
    return fail(FP4_ERR_SHAPE, "hidden %d / inter %d not multiples of %d", L->hidden, L->inter, blk);
  if (a != FP4_FMT_NONE && (L->hidden % 128 || L->inter % 128))
    return fail(FP4_ERR_SHAPE, "quantized-activation paths need hidden and inter multiples of 128");
  if (L->shared_inter < 0) return fail(FP4_ERR_SHAPE, "negative shared width");
  if (L->shared_inter > 0 && (L->shared_inter % 128 || L->hidden % 128))
    return fail(FP4_ERR_SHAPE, "shared width and hidden must be multiples of 128");
  // NVFP4 / MXFP4: tiled codes and tiled scales together; block FP8: codes only
  const bool scales_tiled = w != FP4_FMT_FP8_BLOCK;
  if ((L->w13_tiled && (L->w13_scale_tiled != nullptr) != scales_tiled) ||
      (L->w2_tiled && (L->w2_scale_tiled != nullptr) != scales_tiled) ||
      (!L->w13_tiled && L->w13_scale_tiled) || (!L->w2_tiled && L->w2_scale_tiled))
    return fail(FP4_ERR_INVALID_ARG, "tiled FP4 codes need tiled scales; tiled block-FP8 codes take none");
  if ((L->w13_tiled && L->hidden % 128) || (L->w2_tiled && L->inter % 128))
    return fail(FP4_ERR_SHAPE, "tiled weights need a reduction size that is a multiple of 128");
  return FP4_OK;
}

}  // namespace fp4

using namespace fp4;

extern "C" {

int moe_fp4_workspace_layout(const moe_fp4_layer* layer, int64_t tokens, moe_fp4_ws_layout* out) {
  FP4_CHECK(validate_layer(layer, tokens));
  if (!out) return fail(FP4_ERR_INVALID_ARG, "null layout");
  WsPlan p;
  FP4_CHECK(plan_workspace(layer, tokens, &p));
  out->total = p.total;
  out->error_flag = p.error_flag;
  out->counts = p.counts;
  out->offsets = p.offsets;
  out->pair_of_row = p.pair_of_row;
  out->row_of_pair = p.row_of_pair;
  out->x_tensor_scale = p.x_tensor_scale;
  out->h_tensor_scale = p.h_tensor_scale;
  out->h = p.h;
  out->hq_codes = p.hq_codes;
  out->hq_scales = p.hq_scales;
  out->o = p.o;
  return FP4_OK;
}

int moe_fp4_workspace_size(const moe_fp4_layer* layer, int64_t tokens, size_t* bytes) {
  if (!bytes) return fail(FP4_ERR_INVALID_ARG, "null size pointer");
  FP4_CHECK(validate_layer(layer, tokens));
  WsPlan p;
  FP4_CHECK(plan_workspace(layer, tokens, &p));
  *bytes = p.total;
  return FP4_OK;
}

// Per-device helper stream (default priority) and fork / join events for the
// shared expert, created on first use and kept until the process ends.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
static std::mutex g_side_mu;
static SideStream g_side[kMaxDevices];

static int side_stream(SideStream** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(FP4_ERR_HIP, "no current HIP device");
  SideStream& ss = g_side[dev];
  if (!ss.s) {
    RelaxedCapture relaxed;
    if (hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess)
      return fail(FP4_ERR_HIP, "creating the shared-expert stream failed");
  }
  *out = &ss;
  return FP4_OK;
}

// Joins the shared-expert helper stream back into the caller's stream on
// every exit after the fork: an error return then still leaves no work of
// the call running unjoined (and a captured graph with no dangling fork).
struct SideJoin {
  SideStream* side = nullptr;
  hipStream_t st = nullptr;
  bool joined = false;
  int join() {
    joined = true;
    if (hipEventRecord(side->join, side->s) != hipSuccess || hipStreamWaitEvent(st, side->join, 0) != hipSuccess)
      return fail(FP4_ERR_HIP, "join of the shared-expert stream failed");
    return FP4_OK;
  }
  ~SideJoin() {
    if (side && !joined) (void)join();
  }
};

// inline_shared: the shared expert runs on the caller's stream ahead of the
// routed experts (no helper stream, no fork / join events)
static int forward_impl(const moe_fp4_layer* L, const uint16_t* x, int64_t T, const int32_t* topk_ids,
                        const float* topk_weights, float* y, void* workspace, size_t workspace_bytes,
                        void* stream, void* const* events, bool inline_shared = false) {
  FP4_CHECK(validate_layer(L, T));
  if (T == 0) return FP4_OK;
  if (!x || !topk_ids || !topk_weights || !y) return fail(FP4_ERR_INVALID_ARG, "null tensor pointer");
  if (!L->w13 || !L->w13_scale || !L->w2 || !L->w2_scale)
    return fail(FP4_ERR_INVALID_ARG, "null weight pointer");
  if (L->w_fmt == FP4_FMT_NVFP4 && (!L->w13_scale_2 || !L->w2_scale_2))
    return fail(FP4_ERR_INVALID_ARG, "NVFP4 weights need weight_scale_2");
  if (L->shared_inter > 0 && (!L->ws13 || !L->ws13_scale || !L->ws2 || !L->ws2_scale || !L->shared_gate))
    return fail(FP4_ERR_INVALID_ARG, "null shared-expert pointer");
  WsPlan p;
  FP4_CHECK(plan_workspace(L, T, &p));
  if (!workspace || workspace_bytes < p.total)
    return fail(FP4_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, p.total);
  hipStream_t st = as_stream(stream);
  const Marker mark{events, st};
  WsPtrs w = ws_pointers(p, workspace);
  const int64_t P = T * L->top_k;
  const int max_active = (int)std::min<int64_t>(L->num_experts, P);

  FP4_CHECK(mark(0));
  // The shared expert depends on x only: it runs on a helper stream of the
  // device, forked from and joined back into the caller's stream, so that
  // it overlaps the routed path.  The lock keeps the fork / join events of
  // concurrent callers apart.
  const float* extra = nullptr;
  std::unique_lock<std::mutex> side_lock;
  SideJoin sj;
  if (L->shared_inter > 0 && inline_shared) {
    FP4_CHECK(launch_shared_expert(L, x, T, w, st));
    extra = w.s_out;
  } else if (L->shared_inter > 0) {
    side_lock = std::unique_lock<std::mutex>(g_side_mu);
    SideStream* side = nullptr;
    FP4_CHECK(side_stream(&side));
    if (hipEventRecord(side->fork, st) != hipSuccess || hipStreamWaitEvent(side->s, side->fork, 0) != hipSuccess)
      return fail(FP4_ERR_HIP, "fork to the shared-expert stream failed");
    sj.side = side;
    sj.st = st;
    FP4_CHECK(launch_shared_expert(L, x, T, w, side->s));
    extra = w.s_out;
  }
  FP4_CHECK(launch_permute(topk_ids, P, L->num_experts, kGemmTileM, w, st));
  FP4_CHECK(mark(1));
  bool grouped = false;  // the grouped GEMMs leave o in fp16, the GEMVs in f32
  if (L->a_fmt == FP4_FMT_NONE) {
    FP4_CHECK(mark(2));
    if (L->w_fmt == FP4_FMT_NVFP4) FP4_CHECK(launch_gemv<FP4_FMT_NVFP4>(x, w, L, P, max_active, st, mark));
    else FP4_CHECK(launch_gemv<FP4_FMT_MXFP4>(x, w, L, P, max_active, st, mark));
  } else if (w4a8_gemv(L, T)) {
    // x -> MXFP8 codes and their exact bf16 values in one pass; likewise h (f32)
    FP4_CHECK(mxfp8_quantize_dequant(x, FP4_DT_BF16, T, L->hidden, w.xq_codes,
                                     reinterpret_cast<uint8_t*>(w.xq_scales), w.x_deq, FP4_DT_BF16, st));
    FP4_CHECK(mark(2));
    FP4_CHECK(launch_gemv<FP4_FMT_MXFP4>(w.x_deq, w, L, P, max_active, st, mark, true));
  } else {
    grouped = true;
    FP4_CHECK(launch_grouped(L, x, T, w, max_active, st, mark));
  }
  if (sj.side) FP4_CHECK(sj.join());
  FP4_CHECK(mark(6));  // the "shared" stage is the part of the shared expert not hidden by the routed path
  launch_combine(w.o, grouped, w.row_of_pair, topk_weights, T, L->hidden, L->top_k, extra, y, st);
  FP4_CHECK(check_launch("combine"));
  return mark(7);
}

// ------------------------------------------------- allocation-free forward

// Scratch of moe_fp4_forward_noalloc: one array per device, held by the
// loaded code object until the process ends.  Host code never uses the
// array's name as an address (on the host it is only a stand-in for the
// symbol): each device's address comes from hipGetSymbolAddress, taken once
// per device with that device current.
static __device__ __attribute__((aligned(256))) uint8_t scratch[FP4_NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(FP4_ERR_HIP, "no current HIP device");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(FP4_ERR_HIP, "hipGetSymbolAddress of the scratch array failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FP4_OK;
}

int moe_fp4_forward(const moe_fp4_layer* L, const uint16_t* x, int64_t T, const int32_t* topk_ids,
                    const float* topk_weights, float* y, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return forward_impl(L, x, T, topk_ids, topk_weights, y, workspace, workspace_bytes, stream, nullptr);
}

int moe_fp4_forward_noalloc(const moe_fp4_layer* L, const uint16_t* x, int64_t T, const int32_t* topk_ids,
                            const float* topk_weights, float* y, void* stream) {
  FP4_CHECK(validate_layer(L, T));
  if (T == 0) return FP4_OK;
  WsPlan p;
  FP4_CHECK(plan_workspace(L, T, &p));
  if (p.total > FP4_NOALLOC_SCRATCH_BYTES)
    return fail(FP4_ERR_WORKSPACE, "allocation-free forward: %lld tokens need %zu bytes of scratch, at most %zu held",
                (long long)T, p.total, (size_t)FP4_NOALLOC_SCRATCH_BYTES);
  void* ptr = nullptr;
  FP4_CHECK(scratch_address(&ptr));
  return forward_impl(L, x, T, topk_ids, topk_weights, y, ptr, FP4_NOALLOC_SCRATCH_BYTES, stream, nullptr,
                      /*inline_shared=*/true);
}

int moe_fp4_route(const float* logits, const float* bias, int64_t tokens, int num_experts, int top_k,
                  int32_t* topk_ids, float* topk_weights, void* stream) {
  if (tokens < 0) return fail(FP4_ERR_SHAPE, "negative token count");
  if (num_experts < 1 || top_k < 1 || top_k > num_experts || top_k > kMaxTopK)
    return fail(FP4_ERR_INVALID_ARG, "route: need 1 <= top_k <= min(num_experts, %d), got k=%d, E=%d", kMaxTopK,
                top_k, num_experts);
  if (num_experts > 1024) return fail(FP4_ERR_UNSUPPORTED, "route: more than 1024 experts");
  if (tokens == 0) return FP4_OK;
  if (!logits || !topk_ids || !topk_weights) return fail(FP4_ERR_INVALID_ARG, "route: null pointer");
  if ((tokens + 3) / 4 > INT32_MAX) return fail(FP4_ERR_UNSUPPORTED, "route: too many tokens");
  hipStream_t st = as_stream(stream);
  const dim3 grid((unsigned)((tokens + 3) / 4));
  const int pl = (num_experts + 63) / 64;
  if (pl <= 2)
    hipLaunchKernelGGL(route_topk_kernel<2>, grid, dim3(256), 0, st, logits, bias, tokens, num_experts, top_k,
                       topk_ids, topk_weights);
  else if (pl <= 4)
    hipLaunchKernelGGL(route_topk_kernel<4>, grid, dim3(256), 0, st, logits, bias, tokens, num_experts, top_k,
                       topk_ids, topk_weights);
  else if (pl <= 8)
    hipLaunchKernelGGL(route_topk_kernel<8>, grid, dim3(256), 0, st, logits, bias, tokens, num_experts, top_k,
                       topk_ids, topk_weights);
  else
    hipLaunchKernelGGL(route_topk_kernel<16>, grid, dim3(256), 0, st, logits, bias, tokens, num_experts, top_k,
                       topk_ids, topk_weights);
  return check_launch("route_topk");
}

int moe_fp4_forward_profiled(const moe_fp4_layer* L, const uint16_t* x, int64_t T,
                             const int32_t* topk_ids, const float* topk_weights, float* y,
                             void* workspace, size_t workspace_bytes, void* stream,
                             void* const* events, int n_events) {
  if (!events || n_events != 8) return fail(FP4_ERR_INVALID_ARG, "profiled forward needs 8 events");
  for (int i = 0; i < 8; ++i)
    if (!events[i]) return fail(FP4_ERR_INVALID_ARG, "null event %d", i);
  return forward_impl(L, x, T, topk_ids, topk_weights, y, workspace, workspace_bytes, stream, events);
}

}  // extern "C"
