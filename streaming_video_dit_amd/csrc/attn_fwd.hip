// Block-masked flash attention over concatenated K/V segments, gfx950.
//
// What it computes: for each head and query i, softmax attention over the
// keys of every segment whose (q-block, k-block) mask entry is kept; an empty
// visible set gives O = 0 and LSE = -inf. Sources: the concatenated
// [text | history/reference | current] K/V of the Joy-face_change_optimized
// README (section 1, item 1) with its optional int8 cache (same section),
// block-causal chunks (Wave Forcing summary) and block-sparse attention with
// a dense-mask-equals-SDPA contract (FlashVSR deployment notes,
// Block-Sparse-Attention section).
//
// How (MI355X design):
//  * One workgroup = one head x 128 query rows, 4 waves of 32 rows each; two
//    workgroups per CU (LDS ~74 KB each) so two waves share every SIMD and
//    one wave's softmax overlaps the other's matrix work.
//  * Keys stream through LDS in 64-key tiles, double buffered: the next kept
//    tile is fetched into registers while the current one is consumed, then
//    written to the other buffer (one barrier per tile).
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K from LDS is the A operand,
//    Q^T stays in registers as the B operand). In the 32x32 accumulator layout
//    every lane then owns ONE query column and 16 keys, so row max/sum are
//    per-lane plus one v_permlane32_swap, and the rescale of O is a per-lane
//    scalar.
//  * O^T += V^T P^T with v_mfma_f32_32x32x16_f16: the S^T accumulator,
//    converted to fp16, is directly the B operand; V is written to LDS as fp16,
//    transposed ([d][key]) with the middle two quads of every 16 keys swapped,
//    which is exactly the key order in which the accumulator hands P over, so
//    one 16-byte LDS read feeds each MFMA. P and V are fp16 rather than bf16
//    at the same MFMA rate: fp16 has 3 more mantissa bits, and the rounding of
//    P is the dominant error of the output when one key carries most of the
//    weight. bf16 V converts exactly for |v| < 65504; int8 codes always do.
//  * Online softmax in base 2 (scale*log2(e) folded in), with a lazy running
//    max: O and l are only rescaled when a row max grows by more than 2^8, so
//    P stays <= 256 and the rescale is skipped for almost every tile.
//  * Mask: each workgroup compacts the kept 64-key tiles of its q-tile into an
//    LDS list (chunks of 512 candidates); skipped tiles cost nothing and are
//    never read. Tiles whose mask blocks are only partly kept (block sizes
//    below the tile) and ragged segment tails take a per-element path.
//  * int8 segments: codes are widened exactly (K to bf16, V to fp16) while
//    staging into LDS; the per-key K scale multiplies score rows and the
//    per-key V scale multiplies P before its fp16 rounding (no lossy
//    dequantised copy).
//  * Grid is remapped so consecutive (head, q-tile) work items land on the
//    same XCD and share its L2 for K/V.
#include "sdit_internal.h"

namespace sdit {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BQ = kAttnBQ;
constexpr int BK = kAttnBK;
constexpr int NW = 4;
constexpr int NT = NW * 64;
constexpr int LIST_CAP = 512;
constexpr float TAU = 8.0f;           // lazy-rescale threshold (log2 units)
constexpr int NXCD = 8;

template <int D>
struct Smem {
  static constexpr int KS = D + 8;    // K row stride in LDS (bf16 elements)
  static constexpr int VS = BK + 8;   // V^T row stride in LDS (bf16 elements)
  uint16_t k[2][BK * KS];
  uint16_t vt[2][D * VS];             // fp16
  float ksc[2][BK];                   // int8 tiles: k_scale * scale_log2
  float vsc[2][BK];                   // int8 tiles: v_scale
  uint16_t list[LIST_CAP];
  int32_t wave_count[NW];
};

struct TileInfo {
  int seg;
  int key0;      // first key of the tile inside its segment
  int n_valid;   // keys of the tile inside the segment (1..BK)
};

__device__ __forceinline__ TileInfo tile_info(const AttnParams& p, int g) {
  int s = 0;
#pragma unroll 1
  for (int i = 1; i < p.n_segs; ++i)
    if (g >= p.seg[i].tile_start) s = i;
  TileInfo t;
  t.seg = s;
  t.key0 = (g - p.seg[s].tile_start) * BK;
  t.n_valid = min(BK, p.seg[s].len - t.key0);
  return t;
}

// Position of key k (0..BK-1) in a V^T row: the middle two quads of every
// 16 keys are swapped (keys 4..7 <-> 8..11).
__device__ __forceinline__ int vt_pos(int k) {
  const int q = (k >> 2) & 3;
  const int qs = (q == 1) ? 2 : (q == 2 ? 1 : q);
  return (k & ~15) | (qs << 2) | (k & 3);
}

__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t w, int byte0) {
  const int a = (int)(int8_t)((w >> (8 * byte0)) & 0xFF);
  const int b = (int)(int8_t)((w >> (8 * byte0 + 8)) & 0xFF);
  // small integers are exact in bf16: the low 16 bits of the fp32 pattern are zero
  return (__float_as_uint((float)a) >> 16) | (__float_as_uint((float)b) & 0xFFFF0000u);
}

// Registers holding one tile between its global load and its LDS store.
template <int D>
struct Stage {
  static constexpr int KCH = D / 32;   // 16-byte K chunks per thread (bf16)
  uint4 k[KCH];
  uint4 v[4];                          // bf16: 4 keys x 8 columns; int8: 4 keys x 8 columns in .x/.y
  float ks, vs;
};

template <int D>
__device__ __forceinline__ void load_tile(const AttnParams& p, const TileInfo& t, int head, Stage<D>& st) {
  const AttnSegment& sg = p.seg[t.seg];
  const int tid = threadIdx.x;
  const int64_t row_stride = (int64_t)p.n_heads * D;   // elements between consecutive tokens
  if (!sg.is_int8) {
    const uint16_t* kb = (const uint16_t*)sg.k + ((int64_t)t.key0 * p.n_heads + head) * D;
    const uint16_t* vb = (const uint16_t*)sg.v + ((int64_t)t.key0 * p.n_heads + head) * D;
#pragma unroll
    for (int i = 0; i < Stage<D>::KCH; ++i) {
      const int c = tid + i * NT;             // chunk id: row = c / (D/8), column chunk = c % (D/8)
      const int r = c / (D / 8), cc = c % (D / 8);
      st.k[i] = (r < t.n_valid) ? *reinterpret_cast<const uint4*>(kb + r * row_stride + cc * 8)
                                : make_uint4(0, 0, 0, 0);
    }
    // V unit: 4 consecutive keys x 8 columns
    constexpr int UNITS = (BK / 4) * (D / 8);
    if (UNITS >= NT || tid < UNITS) {
      const int kq = tid / (D / 8), dg = tid % (D / 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = kq * 4 + j;
        st.v[j] = (r < t.n_valid) ? *reinterpret_cast<const uint4*>(vb + r * row_stride + dg * 8)
                                  : make_uint4(0, 0, 0, 0);
      }
    }
  } else {
    const int8_t* kb = (const int8_t*)sg.k + ((int64_t)t.key0 * p.n_heads + head) * D;
    const int8_t* vb = (const int8_t*)sg.v + ((int64_t)t.key0 * p.n_heads + head) * D;
    constexpr int KCH8 = D / 64;              // 16-byte int8 chunks per thread
#pragma unroll
    for (int i = 0; i < KCH8; ++i) {
      const int c = tid + i * NT;
      const int r = c / (D / 16), cc = c % (D / 16);
      st.k[i] = (r < t.n_valid) ? *reinterpret_cast<const uint4*>(kb + r * row_stride + cc * 16)
                                : make_uint4(0, 0, 0, 0);
    }
    constexpr int UNITS = (BK / 4) * (D / 8);
    if (UNITS >= NT || tid < UNITS) {
      const int kq = tid / (D / 8), dg = tid % (D / 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = kq * 4 + j;
        uint2 w = make_uint2(0, 0);
        if (r < t.n_valid) w = *reinterpret_cast<const uint2*>(vb + r * row_stride + dg * 8);
        st.v[j] = make_uint4(w.x, w.y, 0, 0);
      }
    }
    if (tid < BK) {
      const int r = tid;
      st.ks = (r < t.n_valid) ? sg.k_scale[(int64_t)(t.key0 + r) * p.n_heads + head] * p.scale_log2 : 0.f;
      st.vs = (r < t.n_valid) ? sg.v_scale[(int64_t)(t.key0 + r) * p.n_heads + head] : 0.f;
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const AttnParams& p, const TileInfo& t, const Stage<D>& st,
                                           Smem<D>& sm, int buf) {
  const int tid = threadIdx.x;
  constexpr int KS = Smem<D>::KS, VS = Smem<D>::VS;
  const bool i8 = p.seg[t.seg].is_int8;
  uint16_t* kl = sm.k[buf];
  uint16_t* vl = sm.vt[buf];
  if (!i8) {
#pragma unroll
    for (int i = 0; i < Stage<D>::KCH; ++i) {
      const int c = tid + i * NT;
      const int r = c / (D / 8), cc = c % (D / 8);
      *reinterpret_cast<uint4*>(kl + r * KS + cc * 8) = st.k[i];
    }
  } else {
    constexpr int KCH8 = D / 64;
#pragma unroll
    for (int i = 0; i < KCH8; ++i) {
      const int c = tid + i * NT;
      const int r = c / (D / 16), cc = c % (D / 16);
      const uint32_t w[4] = {st.k[i].x, st.k[i].y, st.k[i].z, st.k[i].w};
      uint4 lo = make_uint4(i8x2_to_bf16x2(w[0], 0), i8x2_to_bf16x2(w[0], 2),
                            i8x2_to_bf16x2(w[1], 0), i8x2_to_bf16x2(w[1], 2));
      uint4 hi = make_uint4(i8x2_to_bf16x2(w[2], 0), i8x2_to_bf16x2(w[2], 2),
                            i8x2_to_bf16x2(w[3], 0), i8x2_to_bf16x2(w[3], 2));
      *reinterpret_cast<uint4*>(kl + r * KS + cc * 16) = lo;
      *reinterpret_cast<uint4*>(kl + r * KS + cc * 16 + 8) = hi;
    }
    if (tid < BK) {
      sm.ksc[buf][tid] = st.ks;
      sm.vsc[buf][tid] = st.vs;
    }
  }
  constexpr int UNITS = (BK / 4) * (D / 8);
  if (UNITS >= NT || tid < UNITS) {
    const int kq = tid / (D / 8), dg = tid % (D / 8);
    const int pos = vt_pos(kq * 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float f[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!i8) {
          const uint32_t w = (e >> 1) == 0 ? st.v[j].x : (e >> 1) == 1 ? st.v[j].y : (e >> 1) == 2 ? st.v[j].z : st.v[j].w;
          f[j] = __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
        } else {
          const uint32_t w = (e < 4) ? st.v[j].x : st.v[j].y;
          f[j] = (float)(int)(int8_t)((w >> (8 * (e & 3))) & 0xFF);
        }
      }
      f16x2 lo, hi;
      lo[0] = (_Float16)f[0]; lo[1] = (_Float16)f[1];
      hi[0] = (_Float16)f[2]; hi[1] = (_Float16)f[3];
      *reinterpret_cast<uint2*>(vl + (dg * 8 + e) * VS + pos) =
          make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    }
  }
}

__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

template <int D>
__global__ __launch_bounds__(NT, 2) void attn_fwd_kernel(AttnParams p) {
  __shared__ Smem<D> sm;
  constexpr int KS = Smem<D>::KS, VS = Smem<D>::VS;
  constexpr int NKS = D / 16;   // MFMA k-steps over the head dimension
  constexpr int NDT = D / 32;   // 32-wide column tiles of O^T

  // ---- XCD-aware work mapping: consecutive items on one XCD
  const int G = gridDim.x, b = blockIdx.x;
  const int xcd = b % NXCD, local = b / NXCD;
  const int q8 = G / NXCD, r8 = G % NXCD;
  const int item = (xcd < r8) ? xcd * (q8 + 1) + local : r8 * (q8 + 1) + (xcd - r8) * q8 + local;
  const int head = item / p.n_qt;
  const int qt = item % p.n_qt;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 31;       // query column of this lane inside the wave's 32 rows
  const int hh = lane >> 5;      // which half of the MFMA k-slice this lane supplies
  const int q_row = qt * BQ + wave * 32 + r;
  const bool q_ok = q_row < p.n_q;

  // ---- Q^T fragments (B operand), held for the whole kernel
  bf16x8 qf[NKS];
  {
    const uint16_t* qp = p.q + ((int64_t)q_row * p.n_heads + head) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      uint4 w = q_ok ? *reinterpret_cast<const uint4*>(qp + ks * 16) : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  f32x16 o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
  float m_run = -INFINITY;   // running max, log2 units
  float l_run = 0.f;         // this lane's half of the row sum

  // q-block range of this workgroup (for mask lookups)
  const int q_lo = qt * BQ;
  const int q_hi = min(p.n_q, q_lo + BQ) - 1;
  const int qb_lo = q_lo / p.block_q, qb_hi = q_hi / p.block_q;
  const int my_qb = min(q_row, p.n_q - 1) / p.block_q;

  int buf = 0;
  Stage<D> st;

#pragma unroll 1
  for (int cbase = 0; cbase < p.n_tiles; cbase += LIST_CAP) {
    // ---- compact the kept tiles of this chunk into sm.list (order preserved)
    const int ncand = min(LIST_CAP, p.n_tiles - cbase);
    bool keep[2], part[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = 2 * tid + i;
      keep[i] = false;
      part[i] = false;
      if (c < ncand) {
        const TileInfo t = tile_info(p, cbase + c);
        const AttnSegment& sg = p.seg[t.seg];
        const int kb_lo = sg.kb_start + t.key0 / p.block_k;
        const int kb_hi = sg.kb_start + (t.key0 + t.n_valid - 1) / p.block_k;
        bool any = false, all = true;
        for (int qb = qb_lo; qb <= qb_hi; ++qb)
          for (int kb = kb_lo; kb <= kb_hi; ++kb) {
            const bool m = p.mask[(int64_t)qb * p.n_kb + kb] != 0;
            any |= m;
            all &= m;
          }
        keep[i] = any;
        part[i] = !all;
      }
    }
    const uint64_t b0 = __ballot(keep[0]);
    const uint64_t b1 = __ballot(keep[1]);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (lane == 0) sm.wave_count[wave] = __popcll(b0) + __popcll(b1);
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int cnt = sm.wave_count[w];
      base += (w < wave) ? cnt : 0;
      total += cnt;
    }
    {
      int pos = base + __popcll(b0 & lt) + __popcll(b1 & lt);
      if (keep[0]) sm.list[pos++] = (uint16_t)((2 * tid) | (part[0] ? 0x8000 : 0));
      if (keep[1]) sm.list[pos] = (uint16_t)((2 * tid + 1) | (part[1] ? 0x8000 : 0));
    }
    __syncthreads();
    if (total == 0) continue;

    // ---- prologue: first kept tile into LDS
    {
      const uint16_t e = sm.list[0];
      const TileInfo t = tile_info(p, cbase + (e & 0x7FFF));
      load_tile<D>(p, t, head, st);
      store_tile<D>(p, t, st, sm, buf);
    }
    __syncthreads();

#pragma unroll 1
    for (int it = 0; it < total; ++it) {
      const uint16_t e = sm.list[it];
      const TileInfo t = tile_info(p, cbase + (e & 0x7FFF));
      const bool partial = (e & 0x8000) != 0;
      const bool i8 = p.seg[t.seg].is_int8;

      TileInfo tn;
      const bool has_next = it + 1 < total;
      if (has_next) {
        tn = tile_info(p, cbase + (sm.list[it + 1] & 0x7FFF));
        load_tile<D>(p, tn, head, st);
      }

      const uint16_t* kl = sm.k[buf];
      const uint16_t* vl = sm.vt[buf];

      // ---- S^T = K Q^T for two 32-key subtiles
      f32x16 s[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int e2 = 0; e2 < 16; ++e2) s[kt][e2] = 0.f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kl + (kt * 32 + r) * KS + ks * 16 + 8 * hh);
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kt], 0, 0, 0);
        }
      }

      // ---- scores to log2 units, masking
      // element e2 of subtile kt holds key kt*32 + 8*(e2/4) + 4*hh + e2%4
      float x[2][16];
      if (i8) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 sc = *reinterpret_cast<const float4*>(&sm.ksc[buf][kt * 32 + 8 * g + 4 * hh]);
            x[kt][4 * g + 0] = s[kt][4 * g + 0] * sc.x;
            x[kt][4 * g + 1] = s[kt][4 * g + 1] * sc.y;
            x[kt][4 * g + 2] = s[kt][4 * g + 2] * sc.z;
            x[kt][4 * g + 3] = s[kt][4 * g + 3] * sc.w;
          }
      } else {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e2 = 0; e2 < 16; ++e2) x[kt][e2] = s[kt][e2] * p.scale_log2;
      }
      if (partial || t.n_valid < BK) {
        // per-element keep: inside the segment and, for partly kept tiles, in a kept block
        uint32_t kbits = 0xFu;
        if (partial) {
          const AttnSegment& sg = p.seg[t.seg];
          const int kb0 = sg.kb_start + t.key0 / p.block_k;
          const int nkb = (BK + p.block_k - 1) / p.block_k;
          kbits = 0;
          for (int j = 0; j < nkb && j < 4; ++j) {
            const int kb = kb0 + j;
            if (kb < p.n_kb && p.mask[(int64_t)my_qb * p.n_kb + kb] != 0) kbits |= 1u << j;
          }
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e2 = 0; e2 < 16; ++e2) {
            const int key = kt * 32 + 8 * (e2 >> 2) + 4 * hh + (e2 & 3);
            const bool ok = key < t.n_valid && ((kbits >> (key / p.block_k)) & 1u);
            x[kt][e2] = ok ? x[kt][e2] : -INFINITY;
          }
      }

      // ---- online softmax (lazy running max)
      float mt = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e2 = 0; e2 < 16; e2 += 2) mt = max3(mt, x[kt][e2], x[kt][e2 + 1]);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
        mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const bool need = mt > m_run + TAU;
      if (__ballot(need)) {
        const float m_new = need ? mt : m_run;
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < NDT; ++i)
#pragma unroll
          for (int e2 = 0; e2 < 16; ++e2) o[i][e2] *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

      f16x8 pb[4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        float pv[16];
#pragma unroll
        for (int e2 = 0; e2 < 16; ++e2) {
          pv[e2] = __builtin_amdgcn_exp2f(x[kt][e2] - m_use);
          l_run += pv[e2];
        }
        if (i8) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 sc = *reinterpret_cast<const float4*>(&sm.vsc[buf][kt * 32 + 8 * g + 4 * hh]);
            pv[4 * g + 0] *= sc.x;
            pv[4 * g + 1] *= sc.y;
            pv[4 * g + 2] *= sc.z;
            pv[4 * g + 3] *= sc.w;
          }
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          f16x8 v;
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = (_Float16)pv[8 * half + j];
          pb[2 * kt + half] = v;
        }
      }

      // ---- O^T += V^T P^T
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const f16x8 a = *reinterpret_cast<const f16x8*>(vl + (dt * 32 + r) * VS + kk * 16 + 8 * hh);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[kk], o[dt], 0, 0, 0);
        }

      if (has_next) store_tile<D>(p, tn, st, sm, buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  // ---- finalise
  float l_tot;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  const float inv = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
  if (q_ok) {
    uint16_t* op = p.out + ((int64_t)q_row * p.n_heads + head) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = dt * 32 + 8 * g + 4 * hh;
        const __bf16 v0 = (__bf16)(o[dt][4 * g + 0] * inv);
        const __bf16 v1 = (__bf16)(o[dt][4 * g + 1] * inv);
        const __bf16 v2 = (__bf16)(o[dt][4 * g + 2] * inv);
        const __bf16 v3 = (__bf16)(o[dt][4 * g + 3] * inv);
        const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, v0) | ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
        const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, v2) | ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
        *reinterpret_cast<uint2*>(op + d) = make_uint2(w0, w1);
      }
    if (p.lse != nullptr && hh == 0) {
      const float ln2 = 0.69314718055994530942f;
      p.lse[(int64_t)head * p.n_q + q_row] = (l_tot > 0.f) ? (m_run + __log2f(l_tot)) * ln2 : -INFINITY;
    }
  }
}

template <int D>
hipError_t launch(const AttnParams& p, hipStream_t stream) {
  const unsigned blocks = (unsigned)(p.n_qt * p.n_heads);
  hipLaunchKernelGGL(attn_fwd_kernel<D>, dim3(blocks), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const AttnParams& p, int head_dim, hipStream_t stream) {
  if (p.n_q == 0) return hipSuccess;
  return head_dim == 128 ? launch<128>(p, stream) : launch<64>(p, stream);
}

}  // namespace sdit
