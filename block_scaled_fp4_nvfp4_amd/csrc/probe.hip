// Device-ceiling microbenchmarks behind include/fp4moe_probe.h (gfx950): the
// measured peaks that the rooflines of the library's kernels are stated
// against next to the vendor figures (a streaming read, the MFMA issue rate
// of each operand type the kernels use), and the experiment that decided how
// the routing-weighted combine is done (fp32 atomics into y against a store
// of o and a separate combine).  Timing is the caller's (events around the
// launch); the kernels only do the measured work.
#include <hip/hip_runtime.h>

#include "../../include/fp4moe_probe.h"
#include "host_common.h"

namespace fp4 {

typedef _Float16 p_half8 __attribute__((ext_vector_type(8)));
typedef __bf16 p_bf16x8 __attribute__((ext_vector_type(8)));
typedef float p_floatx4 __attribute__((ext_vector_type(4)));
typedef int p_intx8 __attribute__((ext_vector_type(8)));
typedef int p_intx4 __attribute__((ext_vector_type(4)));

// Every thread reads 16-byte chunks, four per iteration, grid-stride; the
// XOR of everything read is kept and stored only when it equals a constant
// (so the loads cannot be dropped and nothing is written in practice).
__global__ void __launch_bounds__(256) probe_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// Shader-clock cycles and 100 MHz constant-clock ticks that wave 0 of
// workgroups 0..63 spent in its MFMA loop (their ratio gives the shader clock
// under that load): clk[2 b] and clk[2 b + 1] for workgroup b.
__device__ __forceinline__ void store_clocks(uint64_t* clk, uint64_t t0, uint64_t r0) {
  const uint64_t t1 = __builtin_readcyclecounter();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (clk && threadIdx.x == 0 && blockIdx.x < 64) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// Eight independent accumulator chains per wave (enough to keep one SIMD's
// matrix unit issuing back to back), `iters` rounds; operands are register
// values that never change, accumulators are stored at the end.  The 16 x 16
// MFMAs are written as inline asm on AGPR accumulators tied to their own
// source: from the builtins the register allocator assigns each loop-carried
// accumulator a destination two registers off its source and rotates them
// back with about 50 AGPR copies per round of 8 MFMAs, which wait on the
// MFMA results and halve the measured rate.  The s_nops cover the MFMA
// hazards the compiler cannot see inside the asm (a VALU write of an
// accumulator before its first MFMA, the MFMA results read after the loop);
// a missed hazard could only change the values, not the timing.
template <int KIND>
__global__ void __launch_bounds__(256) probe_mfma_kernel(int iters, float* __restrict__ out, uint64_t* __restrict__ clk) {
  const int lane = threadIdx.x & 63;
  p_floatx4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = p_floatx4{0.f, 0.f, 0.f, 0.f};
  uint64_t t0, r0;
  if constexpr (KIND == FP4_PROBE_MFMA_F16 || KIND == FP4_PROBE_MFMA_BF16) {
    p_half8 a, b;
    p_bf16x8 ab, bb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (_Float16)(0.001f * (lane + i));
      b[i] = (_Float16)(0.002f * (lane - i));
      ab[i] = (__bf16)(0.001f * (lane + i));
      bb[i] = (__bf16)(0.002f * (lane - i));
    }
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
    t0 = __builtin_readcyclecounter();
    r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if constexpr (KIND == FP4_PROBE_MFMA_F16)
          asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc[c]) : "v"(a), "v"(b));
        else
          asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[c]) : "v"(ab), "v"(bb));
      }
    }
  } else {
    // block-scaled f8f6f4 MFMA, both scales 127 (2^0); E2M1 operands take
    // four dwords (cbsz / blgp 4), E4M3 eight
    const int one = 127;
    p_intx8 a, b;
    p_intx4 a4, b4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = 0x38383838 ^ (lane + i);
      b[i] = 0x22222222 ^ (lane * 3 + i);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a4[i] = a[i];
      b4[i] = b[i];
    }
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
    t0 = __builtin_readcyclecounter();
    r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if constexpr (KIND == FP4_PROBE_MFMA_FP8_FP8)
          asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
                       : "+a"(acc[c]) : "v"(a), "v"(b), "v"(one));
        else if constexpr (KIND == FP4_PROBE_MFMA_FP8_FP4)
          asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0] blgp:4"
                       : "+a"(acc[c]) : "v"(a), "v"(b4), "v"(one));
        else
          asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
                       : "+a"(acc[c]) : "v"(a4), "v"(b4), "v"(one));
      }
    }
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  store_clocks(clk, t0, r0);
  p_floatx4 s = acc[0];
#pragma unroll
  for (int c = 1; c < 8; ++c) s += acc[c];
  reinterpret_cast<p_floatx4*>(out)[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// The 32 x 32 shapes: eight chains of 16-register accumulators (from the
// builtins these loops compile to MFMAs only).
template <int KIND>
__global__ void __launch_bounds__(256) probe_mfma32_kernel(int iters, float* __restrict__ out, uint64_t* __restrict__ clk) {
  typedef float floatx16 __attribute__((ext_vector_type(16)));
  const int lane = threadIdx.x & 63;
  floatx16 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  uint64_t t0, r0;
  if constexpr (KIND == FP4_PROBE_MFMA_F16_32) {
    p_half8 a[8], b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int c = 0; c < 8; ++c) a[c][i] = (_Float16)(0.001f * (lane + i + 3 * c));
      b[i] = (_Float16)(0.002f * (lane - i));
    }
    t0 = __builtin_readcyclecounter();
    r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[c], b, acc[c], 0, 0, 0);
    }
  } else {
    constexpr int F = KIND == FP4_PROBE_MFMA_FP4_32 ? 4 : 0;
    p_intx8 a[8], b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int c = 0; c < 8; ++c) a[c][i] = 0x38383838 ^ (lane + i + 8 * c);
      b[i] = 0x22222222 ^ (lane * 3 + i);
    }
    t0 = __builtin_readcyclecounter();
    r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 8; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[c], b, acc[c], F, F, 0, 127, 0, 127);
    }
  }
  store_clocks(clk, t0, r0);
  p_floatx4 s = p_floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r & 3] += acc[c][r];
  reinterpret_cast<p_floatx4*>(out)[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// The down GEMM's epilogue pattern (64-row x 128-column tiles, 4 waves of 32
// columns, 16 consecutive columns x 4 rows per store instruction) with a
// value per element: mode 0 stores o[row][n]; mode 2 adds w[pair] * value
// into y[token(row)][n] with fp32 atomics (no return).
template <int MODE>
__global__ void __launch_bounds__(256) probe_epilogue_kernel(const int32_t* __restrict__ pair_of_row,
                                                             const float* __restrict__ w, int64_t P, int H, int k,
                                                             float* __restrict__ out) {
  const int NT = H / 128;
  const int64_t tile = blockIdx.x;
  const int64_t mt = tile / NT;
  const int nt = (int)(tile % NT);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = nt * 128 + wave * 32 + j * 16 + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = mt * 64 + 16 * i + 4 * lg + r;
        if (row >= P) continue;
        const float v = (float)(row & 7) * 0.25f + (float)(n & 3);
        if (MODE == 0) {
          out[row * H + n] = v;
        } else {
          const int32_t p = pair_of_row[row];
          unsafeAtomicAdd(out + (int64_t)(p / k) * H + n, w[p] * v);
        }
      }
    }
}

// y[t] = sum_j w[t, j] * o[row(t, j)] (float4 per thread, the slots in order).
__global__ void __launch_bounds__(256) probe_combine_kernel(const float* __restrict__ o,
                                                            const int32_t* __restrict__ row_of_pair,
                                                            const float* __restrict__ w, int64_t T, int H, int k,
                                                            float* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_row = H / 4;
  if (i >= T * per_row) return;
  const int64_t t = i / per_row, c4 = i - t * per_row;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int32_t row = row_of_pair[t * k + j];
    const float wj = w[t * k + j];
    const float4 v = reinterpret_cast<const float4*>(o + (int64_t)row * H)[c4];
    acc.x = fmaf(wj, v.x, acc.x);
    acc.y = fmaf(wj, v.y, acc.y);
    acc.z = fmaf(wj, v.z, acc.z);
    acc.w = fmaf(wj, v.w, acc.w);
  }
  reinterpret_cast<float4*>(y + t * H)[c4] = acc;
}

}  // namespace fp4

using namespace fp4;

extern "C" {

int fp4_probe_read(const void* src, size_t bytes, int grid, uint32_t* sink, void* stream) {
  if (!src || !sink || grid < 1 || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16)
    return fail(FP4_ERR_INVALID_ARG, "probe_read: bad arguments");
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)grid), dim3(256), 0, as_stream(stream),
                     reinterpret_cast<const uint4*>(src), bytes / 16, sink);
  return check_launch("probe_read");
}

int fp4_probe_mfma(int kind, int iters, int grid, float* out, uint64_t* clocks, void* stream) {
  if (!out || grid < 1 || iters < 1) return fail(FP4_ERR_INVALID_ARG, "probe_mfma: bad arguments");
  const dim3 g((unsigned)grid), b(256);
  hipStream_t st = as_stream(stream);
  switch (kind) {
    case FP4_PROBE_MFMA_F16: hipLaunchKernelGGL(probe_mfma_kernel<FP4_PROBE_MFMA_F16>, g, b, 0, st, iters, out, clocks); break;
    case FP4_PROBE_MFMA_BF16: hipLaunchKernelGGL(probe_mfma_kernel<FP4_PROBE_MFMA_BF16>, g, b, 0, st, iters, out, clocks); break;
    case FP4_PROBE_MFMA_FP8_FP8:
      hipLaunchKernelGGL(probe_mfma_kernel<FP4_PROBE_MFMA_FP8_FP8>, g, b, 0, st, iters, out, clocks);
      break;
    case FP4_PROBE_MFMA_FP8_FP4:
      hipLaunchKernelGGL(probe_mfma_kernel<FP4_PROBE_MFMA_FP8_FP4>, g, b, 0, st, iters, out, clocks);
      break;
    case FP4_PROBE_MFMA_FP4_FP4:
      hipLaunchKernelGGL(probe_mfma_kernel<FP4_PROBE_MFMA_FP4_FP4>, g, b, 0, st, iters, out, clocks);
      break;
    case FP4_PROBE_MFMA_F16_32:
      hipLaunchKernelGGL(probe_mfma32_kernel<FP4_PROBE_MFMA_F16_32>, g, b, 0, st, iters, out, clocks);
      break;
    case FP4_PROBE_MFMA_FP8_32:
      hipLaunchKernelGGL(probe_mfma32_kernel<FP4_PROBE_MFMA_FP8_32>, g, b, 0, st, iters, out, clocks);
      break;
    case FP4_PROBE_MFMA_FP4_32:
      hipLaunchKernelGGL(probe_mfma32_kernel<FP4_PROBE_MFMA_FP4_32>, g, b, 0, st, iters, out, clocks);
      break;
    default: return fail(FP4_ERR_INVALID_ARG, "probe_mfma: unknown kind %d", kind);
  }
  return check_launch("probe_mfma");
}

int fp4_probe_combine(int mode, const int32_t* pair_of_row, const int32_t* row_of_pair, const float* w,
                      int64_t tokens, int top_k, int hidden, float* o, float* y, void* stream) {
  if (tokens < 1 || top_k < 1 || hidden < 128 || hidden % 128 || !pair_of_row || !row_of_pair || !w || !o || !y)
    return fail(FP4_ERR_INVALID_ARG, "probe_combine: bad arguments");
  const int64_t P = tokens * top_k;
  const int64_t tiles = (P + 63) / 64 * (hidden / 128);
  hipStream_t st = as_stream(stream);
  if (tiles > INT32_MAX) return fail(FP4_ERR_UNSUPPORTED, "probe_combine: too large");
  switch (mode) {
    case FP4_PROBE_STORE_O:
      hipLaunchKernelGGL(probe_epilogue_kernel<0>, dim3((unsigned)tiles), dim3(256), 0, st, pair_of_row, w, P,
                         hidden, top_k, o);
      break;
    case FP4_PROBE_COMBINE:
      hipLaunchKernelGGL(probe_combine_kernel, dim3(grid_1d(tokens * hidden / 4, 256)), dim3(256), 0, st, o,
                         row_of_pair, w, tokens, hidden, top_k, y);
      break;
    case FP4_PROBE_ATOMIC_Y:
      hipLaunchKernelGGL(probe_epilogue_kernel<2>, dim3((unsigned)tiles), dim3(256), 0, st, pair_of_row, w, P,
                         hidden, top_k, y);
      break;
    default: return fail(FP4_ERR_INVALID_ARG, "probe_combine: unknown mode %d", mode);
  }
  return check_launch("probe_combine");
}

}  // extern "C"
