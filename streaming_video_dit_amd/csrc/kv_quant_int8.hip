// Symmetric int8 K/V cache quantisation, one fp32 scale per (token, head), gfx950.
//
// The int8 image K/V cache of the Joy-face_change_optimized README
// (section 1, int8 K/V bullet) scales per token and head. Per row
// (token, head) of head_dim bf16 values:
//   amax = max |x|, scale = amax / 127 (IEEE binary32 division),
//   code = clamp(rint(x / scale), -127, 127)  (binary32 quotient, ties to even),
//   amax == 0 -> scale 0, codes 0.
// Rounding is fully specified so the codes are unique. The quotient x / scale
// is the correctly rounded binary32 one, computed without a division per
// element (Markstein's correction): y = RN(1/scale), an fp64 quotient rounded
// to binary32 (1/scale for a binary32 scale is never within 2^-49 relative of
// a binary32 rounding boundary, so this double rounding is exact);
// q0 = RN(x * y) is within one ulp of x / scale; the residual x - q0 * scale
// is exact in one fma; and RN(q0 + residual * y) = RN(x / scale) (Markstein's
// theorem, for y within half an ulp of 1/scale and no underflow). Rows with
// scale < 2^-100 keep the plain division, so every intermediate stays normal.
// v_rndne_f32 then rounds to the nearest code, ties to even.
//
// HBM-bound: each row is read once (2*d bytes) and written once (d + 4 bytes).
// A row is handled by d/8 lanes (16 B loaded per lane); each lane keeps
// kRowsPerLane independent rows in flight to cover HBM latency.
#include "sdit_internal.h"

namespace sdit {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerLane = 4;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int D>
__global__ __launch_bounds__(kThreads) void kv_quant_int8_kernel(QuantParams p) {
  constexpr int LPR = D / 8;                       // lanes per row
  constexpr int GROUPS = kThreads / LPR;           // rows per workgroup per sweep
  const int lane_in_row = threadIdx.x % LPR;
  const int64_t group = (int64_t)blockIdx.x * GROUPS + threadIdx.x / LPR;
  const int64_t stride = (int64_t)gridDim.x * GROUPS;

  uint4 raw[kRowsPerLane];
#pragma unroll
  for (int r = 0; r < kRowsPerLane; ++r) {
    const int64_t row = group + r * stride;
    if (row < p.n_rows)
      raw[r] = *reinterpret_cast<const uint4*>(p.x + row * D + lane_in_row * 8);
    else
      raw[r] = make_uint4(0, 0, 0, 0);
  }

#pragma unroll
  for (int r = 0; r < kRowsPerLane; ++r) {
    const int64_t row = group + r * stride;
    float x[8];
    const uint32_t w[4] = {raw[r].x, raw[r].y, raw[r].z, raw[r].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(w[i]);
      x[2 * i + 1] = bf16_hi(w[i]);
    }
    uint32_t packed[2];
    const float scale = quant_row8<LPR>(x, packed);
    if (row < p.n_rows) {
      *reinterpret_cast<uint2*>(p.codes + row * D + lane_in_row * 8) = make_uint2(packed[0], packed[1]);
      if (lane_in_row == 0) p.scales[row] = scale;
    }
  }
}

template <int D>
hipError_t launch(const QuantParams& p, hipStream_t stream) {
  constexpr int GROUPS = kThreads / (D / 8);
  const int64_t per_block = (int64_t)GROUPS * kRowsPerLane;
  const int64_t blocks = (p.n_rows + per_block - 1) / per_block;
  hipLaunchKernelGGL(kv_quant_int8_kernel<D>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_quant_int8(const QuantParams& p, int head_dim, hipStream_t stream) {
  if (p.n_rows == 0) return hipSuccess;
  return head_dim == 128 ? launch<128>(p, stream) : launch<64>(p, stream);
}

}  // namespace sdit
