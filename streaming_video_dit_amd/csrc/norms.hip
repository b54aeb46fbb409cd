// RMSNorm and LayerNorm + modulate over the hidden dimension, gfx950.
//
// The Joy-face_change_optimized README (table of changed files) names both
// as fused kernels of the DiT block next to QK-norm + 3D RoPE. Per token row
// of C bf16 values:
//   rmsnorm:            y_c = x_c / sqrt(mean(x^2) + eps) * gamma_c
//   layernorm_modulate: y_c = (x_c - mean) / sqrt(var + eps) * (1 + scale_c) + shift_c
// (population variance; gamma, scale and shift are fp32 vectors over C shared
// by every token), rounded to bf16 once.
//
// HBM-bound: 2 * C bytes in and 2 * C bytes out per token; the fp32 vectors
// (4 or 8 bytes per column) are read by every row but stay in L2. A wave
// owns one row at a time: lane l holds 16-byte chunks l, l + 64, l + 128, ...
// of it in registers (every load of the row is issued before the first
// reduction, and each load instruction covers 1 KB of contiguous row), so x
// is read from HBM once however many passes the statistics take. The
// arithmetic is fp64 with one correctly rounded fp64 -> bf16 conversion at
// the end: in fp32, x - mean of a row whose mean is large against its spread
// loses bits of the small difference; in fp64 every output is within one
// bf16 ulp of the exact value.
#include "sdit_internal.h"

#include <algorithm>

namespace sdit {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;
constexpr int kMaxChunksPerLane = 16;   // C <= 16 * 64 * 8 = 8192
constexpr int kDirectMaxChunks = 4;     // one row per wave up to C = 2048
constexpr int64_t kPipeMaxBlocks = 256 * 8;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// An empty asm that the compiler must assume rewrites w: the fp64 values
// derived from the row are then recomputed in each pass instead of being kept
// in registers across the reductions (16 registers per chunk).
__device__ __forceinline__ void launder(uint32_t (&w)[4]) {
  asm volatile("" : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]));
}

template <bool LAUNDER>
__device__ __forceinline__ void unpack(const uint4& r, uint32_t (&w)[4]) {
  w[0] = r.x; w[1] = r.y; w[2] = r.z; w[3] = r.w;
  if constexpr (LAUNDER) launder(w);
}

template <int K>
__device__ __forceinline__ void load_row(const uint16_t* base, int64_t row, int dim, int lane, uint4 (&r)[K]) {
  const uint4* x = reinterpret_cast<const uint4*>(base + row * dim);
  const int n_chunks = dim >> 3;
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const int c = lane + 64 * i;
    r[i] = c < n_chunks ? x[c] : make_uint4(0, 0, 0, 0);
  }
}

// Row statistics in fp64: the mean (LayerNorm) and 1 / sqrt(mean square or
// population variance + eps). Unused chunks hold +0, which adds nothing to
// the sums; the centred pass masks them explicitly.
template <int K, bool LN, bool LAUNDER>
__device__ __forceinline__ void row_stats(const uint4 (&raw)[K], int lane, int n_chunks, int dim, float eps,
                                          double& mean, double& inv) {
  mean = 0.0;
  double ss = 0.0;
  if constexpr (LN) {
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      uint32_t w[4];
      unpack<LAUNDER>(raw[i], w);
#pragma unroll
      for (int e = 0; e < 4; ++e) s += (double)bf16_lo(w[e]) + (double)bf16_hi(w[e]);
    }
    mean = wave_sum(s) / (double)dim;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      if (lane + 64 * i >= n_chunks) continue;
      uint32_t w[4];
      unpack<LAUNDER>(raw[i], w);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double d0 = (double)bf16_lo(w[e]) - mean, d1 = (double)bf16_hi(w[e]) - mean;
        ss = fma(d0, d0, ss);
        ss = fma(d1, d1, ss);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < K; ++i) {
      uint32_t w[4];
      unpack<LAUNDER>(raw[i], w);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double a = bf16_lo(w[e]), b = bf16_hi(w[e]);
        ss = fma(a, a, ss);
        ss = fma(b, b, ss);
      }
    }
  }
  inv = 1.0 / sqrt(wave_sum(ss) / (double)dim + (double)eps);
}

// The 8 outputs of one chunk, fp64, one correctly rounded conversion each.
// ga / sh point at the chunk's 8 gamma (or scale) and shift values.
template <bool LN, bool LAUNDER>
__device__ __forceinline__ uint4 norm_chunk(const uint4& raw, double mean, double inv, const float* ga,
                                            const float* sh) {
  float g[8], b[8];
  *reinterpret_cast<float4*>(g) = *reinterpret_cast<const float4*>(ga);
  *reinterpret_cast<float4*>(g + 4) = *reinterpret_cast<const float4*>(ga + 4);
  if constexpr (LN) {
    *reinterpret_cast<float4*>(b) = *reinterpret_cast<const float4*>(sh);
    *reinterpret_cast<float4*>(b + 4) = *reinterpret_cast<const float4*>(sh + 4);
  }
  uint32_t w[4];
  unpack<LAUNDER>(raw, w);
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    double v[2] = {bf16_lo(w[e]), bf16_hi(w[e])};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = 2 * e + h;
      if constexpr (LN)
        v[h] = fma((v[h] - mean) * inv, 1.0 + (double)g[j], (double)b[j]);
      else
        v[h] = v[h] * inv * (double)g[j];
    }
    o[e] = f64x2_to_bf16x2(v[0], v[1]);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// K = chunks per lane (ceil(C / 8 / 64)); chunks past C / 8 are idle.
//
// Up to 4 chunks per lane (C <= 2048) every wave takes one row and the grid
// covers all rows: registers stay few, so many rows are in flight per CU.
// Above that (PIPE) the row no longer fits that way: a wave walks rows
// row, row + W, row + 2W, ... (W waves in the grid) and issues the loads of
// its next row before it reduces the current one, the fp32 vectors are
// staged in LDS once per workgroup (their reads then wait on the LDS
// counter, not behind the next row's global loads), and each pass re-derives
// its fp64 values from the packed row.
template <int K, bool LN>
__global__ __launch_bounds__(kThreads) void norm_kernel(NormParams p) {
  constexpr bool PIPE = K > kDirectMaxChunks;
  extern __shared__ float4 vec_lds[];   // PIPE: gamma, or scale then shift, fp32 [dim] each
  if constexpr (PIPE) {
    const int n_vec4 = p.dim >> 2;
    for (int i = threadIdx.x; i < n_vec4; i += kThreads) {
      if constexpr (LN) {
        vec_lds[i] = reinterpret_cast<const float4*>(p.scale)[i];
        vec_lds[n_vec4 + i] = reinterpret_cast<const float4*>(p.shift)[i];
      } else {
        vec_lds[i] = reinterpret_cast<const float4*>(p.gamma)[i];
      }
    }
    __syncthreads();
  }
  const float* ga = PIPE ? reinterpret_cast<const float*>(vec_lds) : (LN ? p.scale : p.gamma);
  const float* sh = PIPE ? reinterpret_cast<const float*>(vec_lds) + p.dim : p.shift;

  const int lane = threadIdx.x & 63;
  const int n_chunks = p.dim >> 3;
  const int64_t stride = (int64_t)gridDim.x * kRowsPerBlock;
  int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= p.n_tok) return;   // whole waves leave together

  uint4 raw[K];
  load_row<K>(p.x, row, p.dim, lane, raw);
  for (;;) {
    const int64_t next = row + stride;
    const bool more = PIPE && next < p.n_tok;
    uint4 nxt[K];
    if (more) load_row<K>(p.x, next, p.dim, lane, nxt);

    double mean, inv;
    row_stats<K, LN, PIPE>(raw, lane, n_chunks, p.dim, p.eps, mean, inv);
    uint4* y = reinterpret_cast<uint4*>(p.y + row * p.dim);
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const int c = lane + 64 * i;
      if (c < n_chunks) y[c] = norm_chunk<LN, PIPE>(raw[i], mean, inv, ga + 8 * c, sh + 8 * c);
    }
    if (!more) break;
#pragma unroll
    for (int i = 0; i < K; ++i) raw[i] = nxt[i];
    row = next;
  }
}

template <bool LN>
hipError_t launch_norm(const NormParams& p, hipStream_t stream) {
  if (p.n_tok == 0) return hipSuccess;
  const int k = (p.dim / 8 + 63) / 64;
  const bool pipe = k > kDirectMaxChunks;
  // direct: one row per wave; pipelined: a few workgroups per CU, each wave
  // walking about n_tok / (4 * blocks) rows
  int64_t blocks = (p.n_tok + kRowsPerBlock - 1) / kRowsPerBlock;
  if (pipe) blocks = std::min<int64_t>(blocks, kPipeMaxBlocks);
  const size_t lds = pipe ? (size_t)p.dim * sizeof(float) * (LN ? 2 : 1) : 0;
  const dim3 grid((unsigned)blocks), block(kThreads);
  switch (k) {
#define SDIT_NORM_CASE(K) \
  case K: hipLaunchKernelGGL((norm_kernel<K, LN>), grid, block, lds, stream, p); break;
    SDIT_NORM_CASE(1) SDIT_NORM_CASE(2) SDIT_NORM_CASE(3) SDIT_NORM_CASE(4)
    SDIT_NORM_CASE(5) SDIT_NORM_CASE(6) SDIT_NORM_CASE(7) SDIT_NORM_CASE(8)
    SDIT_NORM_CASE(9) SDIT_NORM_CASE(10) SDIT_NORM_CASE(11) SDIT_NORM_CASE(12)
    SDIT_NORM_CASE(13) SDIT_NORM_CASE(14) SDIT_NORM_CASE(15) SDIT_NORM_CASE(16)
#undef SDIT_NORM_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

static_assert(kMaxChunksPerLane * 64 * 8 == 8192, "hidden-size limit");

hipError_t launch_rmsnorm(const NormParams& p, hipStream_t stream) { return launch_norm<false>(p, stream); }
hipError_t launch_layernorm_modulate(const NormParams& p, hipStream_t stream) {
  return launch_norm<true>(p, stream);
}

}  // namespace sdit
