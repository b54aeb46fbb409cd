// Internal declarations shared by the C-ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdit {

constexpr int kMaxSegments = 8;

// fp64 -> bf16, round to nearest even, in one step. The fp32 rounding is
// exact unless the fp32 result sits exactly half-way between two bf16 values
// while the fp64 value does not; then the tie is broken by the side the fp64
// value lies on (finite inputs only).
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double x) {
  const float f = (float)x;
  uint32_t u = __float_as_uint(f);
  if ((u & 0xFFFFu) == 0x8000u && (double)f != x) {
    const bool away = fabs(x) > fabs((double)f);
    u = away ? u + 1u : u - 1u;
  }
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp64 values -> two bf16 packed (a in the low half), correctly rounded.
// Rounding to fp32 first and then to bf16 (the hardware conversion, round to
// nearest even) gives the same bf16 as rounding the fp64 value directly
// unless the fp32 value sits exactly half-way between two bf16 values: any
// other bf16 rounding boundary lying between the fp64 value and its fp32
// rounding would itself be an fp32 value closer to the fp64 value. Only that
// case (about one output in 65536) takes the exact path above.
__device__ __forceinline__ uint32_t f64x2_to_bf16x2(double a, double b) {
  const float fa = (float)a, fb = (float)b;
  if (((__float_as_uint(fa) & 0xFFFFu) == 0x8000u) | ((__float_as_uint(fb) & 0xFFFFu) == 0x8000u))
    return f64_to_bf16_rne(a) | (f64_to_bf16_rne(b) << 16);
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)fa, (__bf16)fb};
  return __builtin_bit_cast(uint32_t, v);
}


// ---------------------------------------------------------------- qknorm_rope3d
struct RopeParams {
  const uint16_t* q_in;
  const uint16_t* k_in;
  uint16_t* q_out;
  uint16_t* k_out;
  const float* gamma_q;
  const float* gamma_k;
  int32_t n_tok, Hl, Wl, t0;
  int32_t n_heads, d_t, d_h, d_w;
  double omega[64];    // rotation frequency of pair c/2: theta^(-2j/d_axis), computed on the host
  float eps;
  // fused int8 cache write (sdit_qknorm_rope3d_kv_quant_int8), else NULL:
  // codes and scales of the rotated k (from its bf16 output) and of v_in
  const uint16_t* v_in;
  int8_t* k_codes;
  float* k_scales;
  int8_t* v_codes;
  float* v_scales;
};
hipError_t launch_qknorm_rope3d(const RopeParams& p, int head_dim, hipStream_t stream);

// ---------------------------------------------------------------- kv_quant_int8
// One row's share of the int8 quantisation (the kv_quant_int8 definition):
// the calling lane holds 8 consecutive values x[] of a row spread over LPR
// consecutive lanes (a power of two). Returns the row's scale (every lane)
// and the lane's 8 codes packed in two words. The reciprocal is correctly
// rounded (1/scale in fp64, rounded to binary32) and the quotient corrected
// by Markstein's residual step, so q = RN(x / scale) exactly; rows with
// scale < 2^-100 divide.
// Reductions over a group of LPR (8 or 16) lanes aligned to a 16-lane DPP
// row, in DPP moves (no LDS): swap neighbours, swap pairs inside the quad,
// mirror the half-row, mirror the row. Each step combines disjoint lane sets
// with a commutative op, so every lane of the group ends with the same value.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const long long u = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)u, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned int)hi << 32) | (unsigned int)lo));
}
template <int LPR>
__device__ __forceinline__ float group_max(float x) {
  static_assert(LPR == 8 || LPR == 16, "lane group of 8 or 16");
  x = fmaxf(x, dpp_f32<0xB1>(x));
  x = fmaxf(x, dpp_f32<0x4E>(x));
  x = fmaxf(x, dpp_f32<0x141>(x));
  if (LPR == 16) x = fmaxf(x, dpp_f32<0x140>(x));
  return x;
}
template <int LPR>
__device__ __forceinline__ double group_sum(double x) {
  static_assert(LPR == 8 || LPR == 16, "lane group of 8 or 16");
  x += dpp_f64<0xB1>(x);
  x += dpp_f64<0x4E>(x);
  x += dpp_f64<0x141>(x);
  if (LPR == 16) x += dpp_f64<0x140>(x);
  return x;
}

template <int LPR>
__device__ __forceinline__ float quant_row8(const float (&x)[8], uint32_t (&packed)[2]) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = group_max<LPR>(amax);
  const float scale = amax / 127.0f;
  packed[0] = packed[1] = 0u;
  if (scale >= 0x1p-100f) {
    const float y = (float)(1.0 / (double)scale);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q0 = x[i] * y;
      const float q = fmaf(fmaf(-q0, scale, x[i]), y, q0);
      const float c = fminf(fmaxf(rintf(q), -127.f), 127.f);
      packed[i / 4] |= ((uint32_t)(int32_t)c & 0xFFu) << (8 * (i % 4));
    }
  } else if (amax > 0.f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float c = fminf(fmaxf(rintf(x[i] / scale), -127.f), 127.f);
      packed[i / 4] |= ((uint32_t)(int32_t)c & 0xFFu) << (8 * (i % 4));
    }
  }
  return scale;
}

struct QuantParams {
  const uint16_t* x;
  int8_t* codes;
  float* scales;
  int64_t n_rows;      // n_tok * n_heads
};
hipError_t launch_kv_quant_int8(const QuantParams& p, int head_dim, hipStream_t stream);

// ---------------------------------------------------------------- attn_fwd
struct AttnSegment {
  const void* k;
  const void* v;
  const float* k_scale;
  const float* v_scale;
  int32_t len;
  int32_t is_int8;
  int32_t tile_start;  // first 64-key tile of this segment in the global tile numbering
  int32_t kb_start;    // first mask column (k-block) of this segment
};

struct AttnParams {
  const uint16_t* q;
  uint16_t* out;       // bf16 output, or NULL when out_f32 is set
  float* out_f32;      // partial form: normalised O in fp32
  float* lse;
  const uint8_t* mask;
  AttnSegment seg[kMaxSegments];
  int32_t n_segs;
  int32_t n_q;
  int32_t n_heads;
  int32_t n_qt;        // 128-row query tiles
  int32_t n_tiles;     // total 64-key tiles over all segments
  int32_t n_kb;        // mask columns
  int32_t n_qb;        // mask rows
  int32_t block_q;
  int32_t block_k;
  int32_t block_k_log2;
  float scale_log2;    // softmax_scale * log2(e)
  // Balanced launch. The work units (head, query tile) are dealt to the XCDs
  // in contiguous ranges; on an XCD with R units past its last full wave of
  // CUs, those R units are cut at candidate tile split_tile into a head piece
  // [0, split_tile) and a tail piece [split_tile, n_tiles), which write
  // normalised fp32 O and LSE to workspace slots ((xcd * split_rmax + j) * 2
  // + piece); attn_split_merge then combines them. split_tile 0: no split.
  int32_t split_tile;
  int32_t cu_per_xcd;
  int32_t split_rmax;  // slots per XCD (largest R)
  int32_t grid;        // workgroups of the launch
  float* ws_o;         // [kNumXcd][split_rmax][2][kAttnBQ][head_dim]
  float* ws_lse;       // [kNumXcd][split_rmax][2][kAttnBQ]
};
constexpr int kAttnBQ = 256;  // query rows per workgroup
constexpr int kAttnBK = 64;   // keys per pipeline stage
constexpr int kNumXcd = 8;    // XCDs of an MI355X; workgroup b runs on XCD b % 8
hipError_t launch_attn_fwd(const AttnParams& p, int head_dim, hipStream_t stream);

// Units of a balanced launch on one XCD: the contiguous range [u0, u0 + n)
// of the n_units work units, of which the last r are split (r = n mod
// cu_per_xcd when splitting, else 0).
struct XcdUnits {
  int32_t u0, n, r;
};
__host__ __device__ inline XcdUnits xcd_units(int32_t n_units, int32_t xcd, int32_t cu_per_xcd, bool split) {
  const int32_t q8 = n_units / kNumXcd, r8 = n_units % kNumXcd;
  XcdUnits u;
  u.n = q8 + (xcd < r8 ? 1 : 0);
  u.u0 = xcd * q8 + (xcd < r8 ? xcd : r8);
  u.r = split ? u.n % cu_per_xcd : 0;
  return u;
}

// Library-owned device scratch of the allocation-free balanced attention
// (static_scratch.hip): its device address on the current device, looked up
// once per device.
constexpr int64_t kStaticScratchBytes = (int64_t)64 << 20;
hipError_t static_scratch(void** ptr);

// ---------------------------------------------------------------- attn_merge
constexpr int kMaxMergeParts = 8;
struct MergeParams {
  const float* o[kMaxMergeParts];    // fp32 [n_q][n_heads][head_dim], normalised
  const float* lse[kMaxMergeParts];  // fp32 [n_heads][n_q]
  int32_t n_parts;
  int32_t n_q;
  int32_t n_heads;
  uint16_t* out;                     // bf16 [n_q][n_heads][head_dim]
  float* lse_out;                    // fp32 [n_heads][n_q] or NULL
};
hipError_t launch_attn_merge(const MergeParams& p, int head_dim, hipStream_t stream);
// Merge of the two pieces of every split unit of a balanced attn_fwd launch.
hipError_t launch_attn_split_merge(const AttnParams& p, uint16_t* out, float* lse_out, int head_dim,
                                   hipStream_t stream);

// ---------------------------------------------------------------- window_permute
struct PermuteParams {
  const uint16_t* x;
  uint16_t* y;
  int32_t T, Hl, Wl, win;
  int32_t row_chunks;   // 16-byte chunks per token row (n_heads * head_dim / 8)
  int32_t inverse;      // 0: raster -> window-major, 1: window-major -> raster
  int64_t n_tok;
};
hipError_t launch_window_permute(const PermuteParams& p, hipStream_t stream);

// ---------------------------------------------------------------- rmsnorm / layernorm_modulate
struct NormParams {
  const uint16_t* x;
  uint16_t* y;
  const float* gamma;   // rmsnorm
  const float* scale;   // layernorm_modulate
  const float* shift;
  int64_t n_tok;
  int32_t dim;
  float eps;
};
hipError_t launch_rmsnorm(const NormParams& p, hipStream_t stream);
hipError_t launch_layernorm_modulate(const NormParams& p, hipStream_t stream);

}  // namespace sdit
