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
// (4 or 8 bytes per column) are read by every row but stay in L2. One wave
// owns one row: lane l holds 16-byte chunks l, l + 64, l + 128, ... of it in
// registers (every load of the row is issued before the first reduction, and
// each load instruction covers 1 KB of contiguous row), so x is read from HBM
// once however many passes the statistics take. The arithmetic is fp64 with
// one correctly rounded fp64 -> bf16 conversion at the end: in fp32, x - mean
// of a row whose mean is large against its spread loses bits of the small
// difference; in fp64 every output is within one bf16 ulp of the exact value.
#include "sdit_internal.h"

namespace sdit {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;
constexpr int kMaxChunksPerLane = 16;   // C <= 16 * 64 * 8 = 8192

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ void load_f8(const float* base, int c0, float (&g)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(base + c0);
  const float4 b = *reinterpret_cast<const float4*>(base + c0 + 4);
  g[0] = a.x; g[1] = a.y; g[2] = a.z; g[3] = a.w;
  g[4] = b.x; g[5] = b.y; g[6] = b.z; g[7] = b.w;
}

// K = chunks per lane (ceil(C / 8 / 64)); chunks past C / 8 are idle.
template <int K, bool LN>
__global__ __launch_bounds__(kThreads) void norm_kernel(NormParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= p.n_tok) return;   // whole waves leave together
  const int n_chunks = p.dim >> 3;
  const uint4* x = reinterpret_cast<const uint4*>(p.x + row * p.dim);

  uint4 raw[K];
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const int c = lane + 64 * i;
    raw[i] = c < n_chunks ? x[c] : make_uint4(0, 0, 0, 0);
  }

  // Unused chunks hold +0, which adds nothing to either sum; the centred
  // pass below masks them explicitly.
  double mean = 0.0, inv;
  if constexpr (LN) {
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) s += (double)bf16_lo(w[e]) + (double)bf16_hi(w[e]);
    }
    mean = wave_sum(s) / (double)p.dim;
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      if (lane + 64 * i >= n_chunks) continue;
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double d0 = (double)bf16_lo(w[e]) - mean, d1 = (double)bf16_hi(w[e]) - mean;
        ss = fma(d0, d0, ss);
        ss = fma(d1, d1, ss);
      }
    }
    inv = 1.0 / sqrt(wave_sum(ss) / (double)p.dim + (double)p.eps);
  } else {
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double a = bf16_lo(w[e]), b = bf16_hi(w[e]);
        ss = fma(a, a, ss);
        ss = fma(b, b, ss);
      }
    }
    inv = 1.0 / sqrt(wave_sum(ss) / (double)p.dim + (double)p.eps);
  }

  uint4* y = reinterpret_cast<uint4*>(p.y + row * p.dim);
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const int c = lane + 64 * i;
    if (c >= n_chunks) continue;
    float ga[8], sh[8];
    if constexpr (LN) {
      load_f8(p.scale, 8 * c, ga);
      load_f8(p.shift, 8 * c, sh);
    } else {
      load_f8(p.gamma, 8 * c, ga);
    }
    const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      double v[2] = {bf16_lo(w[e]), bf16_hi(w[e])};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = 2 * e + h;
        if constexpr (LN)
          v[h] = fma((v[h] - mean) * inv, 1.0 + (double)ga[j], (double)sh[j]);
        else
          v[h] = v[h] * inv * (double)ga[j];
      }
      o[e] = f64_to_bf16_rne(v[0]) | (f64_to_bf16_rne(v[1]) << 16);
    }
    y[c] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

template <bool LN>
hipError_t launch_norm(const NormParams& p, hipStream_t stream) {
  if (p.n_tok == 0) return hipSuccess;
  const int k = (p.dim / 8 + 63) / 64;
  const int64_t blocks = (p.n_tok + kRowsPerBlock - 1) / kRowsPerBlock;
  const dim3 grid((unsigned)blocks), block(kThreads);
  switch (k) {
#define SDIT_NORM_CASE(K) \
  case K: hipLaunchKernelGGL((norm_kernel<K, LN>), grid, block, 0, stream, p); break;
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
