// Fused QK-RMSNorm + 3D (t, h, w) rotary embedding, gfx950.
//
// The "QK-norm+3D RoPE" operator of the Joy-face_change_optimized README
// (table of changed files). Per (token, head) row of head_dim bf16 values:
//   y_c = x_c / sqrt(mean(x^2) + eps) * gamma_c
// then interleaved pairs (2j, 2j+1) of the axis blocks t | h | w (widths
// d_t, d_h, d_w) are rotated by p_axis * theta^(-2j/d_axis), and the result
// is rounded to bf16 once.
//
// HBM-bound (2 * 2 * d bytes per row and tensor). Work unit: one token and a
// group of up to kHeadsPerUnit heads of both q and k, handled by d/8 lanes
// that each own 8 consecutive columns (16 B per row, coalesced 256 B rows).
// A lane's four rotation angles depend only on the token, so they are
// computed once per unit and reused for the unit's 2 * kHeadsPerUnit rows,
// whose loads are all issued before the angle math.
// The arithmetic is fp64 (full rate on CDNA4 vector units, so it costs the
// same as fp32 here), ending in one correctly rounded fp64 -> bf16
// conversion. In fp32 a rotation whose two products nearly cancel loses
// several bf16 ulps of its small result; in fp64 every output is within one
// ulp of the exact value.
//
// The fused form (sdit_qknorm_rope3d_kv_quant_int8) also writes the int8
// cache entries of the chunk: each unit loads the v rows of its heads with
// the q and k rows, and quantises the rotated k rows from their bf16 output
// (still in registers, never read back) and the v rows as they are, with the
// arithmetic of kv_quant_int8 (quant_row8), so the codes and scales are the
// ones sdit_kv_quant_int8 of k_out and v would give.
#include "sdit_internal.h"

namespace sdit {
namespace {

constexpr int kThreads = 256;
// Two heads per unit, each unit's loads issued when the unit starts (not a
// unit ahead): the registers then allow more rows in flight per CU. Measured
// on MI355X with rotated buffers against four heads with the next unit's
// loads issued a unit ahead: Wan chunk 26.8 -> 24.6 us, and the fused form
// with the chunk's int8 cache entries 53.2 -> 33.6 us (the three separate
// launches take 45.6 us).
constexpr int kHeadsPerUnit = 2;
// Workgroups of a launch: 1024 x 16 units per sweep (512 was as fast, 256
// much slower; 2048 no faster).
constexpr int kMaxBlocks = 1024;
// The plain form is held to three waves per SIMD (at most 168 registers;
// Wan chunk 22.3 -> 21.2 us); the fused form needs its registers and keeps
// two.

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// sin and cos of an fp64 angle, to about one ulp (rotation angles are
// position x frequency, so |x| stays far below 2^20 pi/2). Cody and Waite's
// argument reduction: k = rint(x * 2/pi) and r = x - k pi/2 with pi/2 split
// into three doubles; the first two carry 33 significant bits, so k times each
// is exact for |k| < 2^20, and the third holds the next 53 bits of pi/2
// (the three together are within 1e-37 of pi/2). Then the Taylor series of
// sin and cos in r^2 on |r| <= pi/4, to the r^19 and r^18 terms (the first
// terms left out are below 1e-19 relative), and the quadrant k mod 4 selects
// +-sin or +-cos. Larger angles fall back to the library routine.
__device__ __forceinline__ void sincos_f64(double x, double& s, double& c) {
  constexpr double kTwoOverPi = 0x1.45f306dc9c883p-1;
  constexpr double kPio2a = 0x1.921fb544p+0;
  constexpr double kPio2b = 0x1.0b4611a6p-34;
  constexpr double kPio2c = 0x1.3198a2e037073p-69;
  if (!(fabs(x) < 0x1p20)) {
    sincos(x, &s, &c);
    return;
  }
  const double k = rint(x * kTwoOverPi);
  const double r = fma(-k, kPio2c, fma(-k, kPio2b, fma(-k, kPio2a, x)));
  const double z = r * r;
  // Horner in z with coefficients (-1)^n / (2n+1)! and (-1)^n / (2n)!, n = 9..1
  double ps = -1.0 / 121645100408832000.0;   // -1/19!
  double pc = -1.0 / 6402373705728000.0;     // -1/18!
  double fs = 121645100408832000.0, fc = 6402373705728000.0;
#pragma unroll
  for (int n = 8; n >= 1; --n) {
    fs /= (double)((2 * n + 2) * (2 * n + 3));
    fc /= (double)((2 * n + 1) * (2 * n + 2));
    const double sign = (n & 1) ? -1.0 : 1.0;
    ps = fma(ps, z, sign / fs);
    pc = fma(pc, z, sign / fc);
  }
  const double sr = fma(r * z, ps, r);
  const double cr = fma(z, pc, 1.0);
  const int q = (int)k & 3;
  const double s0 = (q & 1) ? cr : sr, c0 = (q & 1) ? sr : cr;
  s = (q & 2) ? -s0 : s0;
  c = ((q + 1) & 2) ? -c0 : c0;
}

// Rows per unit: q and k rows (and v rows in the fused form).
template <bool QUANT>
constexpr int unit_rows() { return (QUANT ? 3 : 2) * kHeadsPerUnit; }

// The loads of a unit's rows (q rows, then k rows, then v rows).
template <int D, bool QUANT>
__device__ __forceinline__ void load_unit(const RopeParams& p, int tok, int h0, int nh, int c0,
                                          uint4 (&raw)[unit_rows<QUANT>()]) {
#pragma unroll
  for (int i = 0; i < unit_rows<QUANT>(); ++i) {
    const int hi = i % kHeadsPerUnit;
    const uint16_t* in = i < kHeadsPerUnit ? p.q_in : (i < 2 * kHeadsPerUnit ? p.k_in : p.v_in);
    raw[i] = hi < nh ? *reinterpret_cast<const uint4*>(in + ((int64_t)tok * p.n_heads + h0 + hi) * D + c0)
                     : make_uint4(0, 0, 0, 0);
  }
}

// A 16-lane group walks units unit, unit + S, unit + 2S, ... (S units in the
// grid).
template <int D, bool QUANT>
__global__ __launch_bounds__(kThreads, QUANT ? 1 : 3) void qknorm_rope3d_kernel(RopeParams p) {
  constexpr int NR = unit_rows<QUANT>();
  constexpr int LPR = D / 8;
  constexpr int UNITS_PER_BLOCK = kThreads / LPR;
  const int lane_in_row = threadIdx.x % LPR;
  const int n_hg = (p.n_heads + kHeadsPerUnit - 1) / kHeadsPerUnit;
  const int64_t n_units = (int64_t)p.n_tok * n_hg;
  const int64_t stride = (int64_t)gridDim.x * UNITS_PER_BLOCK;
  int64_t unit = (int64_t)blockIdx.x * UNITS_PER_BLOCK + threadIdx.x / LPR;
  if (unit >= n_units) return;   // a row's 16 lanes leave together
  const int c0 = lane_in_row * 8;

  float g[2][8];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float* gamma = t ? p.gamma_k : p.gamma_q;
    const float4 g0 = *reinterpret_cast<const float4*>(gamma + c0);
    const float4 g1 = *reinterpret_cast<const float4*>(gamma + c0 + 4);
    g[t][0] = g0.x; g[t][1] = g0.y; g[t][2] = g0.z; g[t][3] = g0.w;
    g[t][4] = g1.x; g[t][5] = g1.y; g[t][6] = g1.z; g[t][7] = g1.w;
  }

  int tok = (int)(unit / n_hg);
  int h0 = (int)(unit % n_hg) * kHeadsPerUnit;
  uint4 raw[NR];
  load_unit<D, QUANT>(p, tok, h0, min(kHeadsPerUnit, p.n_heads - h0), c0, raw);
  for (;;) {
    const int nh = min(kHeadsPerUnit, p.n_heads - h0);
    const int64_t next = unit + stride;
    const bool more = next < n_units;
    const int tok_n = (int)(next / n_hg), h0_n = (int)(next % n_hg) * kHeadsPerUnit;

    // Token position on the three axes.
    const int HW = p.Hl * p.Wl;
    const int pos_t = p.t0 + tok / HW;
    const int pos_h = (tok / p.Wl) % p.Hl;
    const int pos_w = tok % p.Wl;

    double cs[4], sn[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = c0 + 2 * i;           // first column of the pair
      const int pos = c < p.d_t ? pos_t : (c < p.d_t + p.d_h ? pos_h : pos_w);
      sincos_f64((double)pos * p.omega[c / 2], sn[i], cs[i]);
    }

#pragma unroll
    for (int i = 0; i < 2 * kHeadsPerUnit; ++i) {
      const int t = i / kHeadsPerUnit, hi = i % kHeadsPerUnit;
      double x[8];
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = (double)bf16_lo(w[e]);
        x[2 * e + 1] = (double)bf16_hi(w[e]);
      }
      double ss = 0.0;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fma(x[e], x[e], ss);
      ss = group_sum<LPR>(ss);
      // 1/sqrt(mean + eps): the hardware estimate (relative error ~5e-8)
      // and two Newton steps (y *= 1.5 - 0.5 a y^2 each) bring it within
      // 2.4e-16 (measured over 2^20 values spanning 2^+-100), against 1.7e-16
      // for a rounded square root and division, with fewer instructions
      const double a = ss / (double)D + (double)p.eps;
      double inv = __builtin_amdgcn_rsq(a);
      inv = inv * fma(-0.5 * a * inv, inv, 1.5);
      inv = inv * fma(-0.5 * a * inv, inv, 1.5);

      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double y0 = x[2 * e] * inv * (double)g[t][2 * e];
        const double y1 = x[2 * e + 1] * inv * (double)g[t][2 * e + 1];
        const double r0 = y0 * cs[e] - y1 * sn[e];
        const double r1 = y0 * sn[e] + y1 * cs[e];
        o[e] = f64x2_to_bf16x2(r0, r1);
      }
      uint16_t* out = t ? p.k_out : p.q_out;
      const int64_t row = (int64_t)tok * p.n_heads + h0 + hi;
      if (hi < nh) *reinterpret_cast<uint4*>(out + row * D + c0) = make_uint4(o[0], o[1], o[2], o[3]);
      if (QUANT && t == 1) {
        // int8 cache entry of the rotated k row, from its bf16 output
        float xq[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xq[2 * e] = bf16_lo(o[e]);
          xq[2 * e + 1] = bf16_hi(o[e]);
        }
        uint32_t packed[2];
        const float scale = quant_row8<LPR>(xq, packed);
        if (hi < nh) {
          *reinterpret_cast<uint2*>(p.k_codes + row * D + c0) = make_uint2(packed[0], packed[1]);
          if (lane_in_row == 0) p.k_scales[row] = scale;
        }
      }
    }
    if (QUANT) {
      // int8 cache entries of the v rows
#pragma unroll
      for (int hi = 0; hi < kHeadsPerUnit; ++hi) {
        const uint4 w = raw[2 * kHeadsPerUnit + hi];
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
        float xv[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xv[2 * e] = bf16_lo(ww[e]);
          xv[2 * e + 1] = bf16_hi(ww[e]);
        }
        uint32_t packed[2];
        const float scale = quant_row8<LPR>(xv, packed);
        const int64_t row = (int64_t)tok * p.n_heads + h0 + hi;
        if (hi < nh) {
          *reinterpret_cast<uint2*>(p.v_codes + row * D + c0) = make_uint2(packed[0], packed[1]);
          if (lane_in_row == 0) p.v_scales[row] = scale;
        }
      }
    }
    if (!more) break;
    load_unit<D, QUANT>(p, tok_n, h0_n, min(kHeadsPerUnit, p.n_heads - h0_n), c0, raw);
    unit = next;
    tok = tok_n;
    h0 = h0_n;
  }
}

template <int D>
hipError_t launch(const RopeParams& p, hipStream_t stream) {
  constexpr int UNITS_PER_BLOCK = kThreads / (D / 8);
  const int n_hg = (p.n_heads + kHeadsPerUnit - 1) / kHeadsPerUnit;
  const int64_t n_units = (int64_t)p.n_tok * n_hg;
  int64_t blocks = (n_units + UNITS_PER_BLOCK - 1) / UNITS_PER_BLOCK;
  blocks = min(blocks, (int64_t)kMaxBlocks);
  if (p.k_codes != nullptr)
    hipLaunchKernelGGL((qknorm_rope3d_kernel<D, true>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((qknorm_rope3d_kernel<D, false>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qknorm_rope3d(const RopeParams& p, int head_dim, hipStream_t stream) {
  if (p.n_tok == 0) return hipSuccess;
  return head_dim == 128 ? launch<128>(p, stream) : launch<64>(p, stream);
}

}  // namespace sdit
