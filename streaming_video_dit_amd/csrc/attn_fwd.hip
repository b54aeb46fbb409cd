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
//    workgroups per CU (LDS ~76 KB each) so two waves share every SIMD and
//    one wave's softmax overlaps the other's matrix work.
//  * Keys stream through LDS in 64-key tiles, double buffered, one barrier
//    per tile. bf16 K goes straight from global memory into LDS
//    (global_load_lds_dwordx4: lane t lands at base + 16 t, so each lane's
//    source address is chosen to realise the padded layout below). V is
//    staged through registers once per workgroup and converted to fp16; int8
//    K/V codes are widened exactly on the same path.
//  * LDS tiles are row-major ([key][d]) with padded rows: K rows are D+8
//    bf16 (16 rows read at one column land on 16 different 4-bank groups), V
//    rows are D+32 fp16 (the 4 rows x 64 bytes that one transposed read
//    covers land on all 64 banks exactly once); row writes cover whole bank
//    sets. Every LDS read address is one per-lane base plus a compile-time
//    offset, and operand reads run a fixed distance ahead of their MFMA, so
//    the accumulators keep the register budget.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K from LDS is the A operand,
//    Q^T stays in registers as the B operand). In the 32x32 accumulator layout
//    every lane then owns ONE query column and 16 keys, so row max/sum are
//    per-lane plus one v_permlane32_swap, and the rescale of O is a per-lane
//    scalar.
//  * O^T += V^T P^T with v_mfma_f32_32x32x16_f16: the S^T accumulator,
//    converted to fp16, is directly the B operand. The V^T A operand is read
//    from the row-major V tile with ds_read_b64_tr_b16: inside each group of
//    16 lanes, lane i receives element i%4 of the 8-byte rows addressed by
//    lanes 4j + i/4 (j = 0..3); pointing those lanes at 4 consecutive keys
//    and 4-column slices hands every lane 4 keys of one column, in the key
//    order in which the accumulator hands P over. fp16 rather than bf16 for
//    P and V (same MFMA rate): 3 more mantissa bits, and the rounding of P
//    dominates the output error when one key carries most of the weight.
//    bf16 V converts exactly for |v| < 65504; int8 codes always do.
//  * Online softmax in base 2 (scale*log2(e) folded in), with a lazy running
//    max: O and l are only rescaled when a row max grows by more than 2^8, so
//    P stays <= 256 and the rescale is skipped for almost every tile.
//  * Mask: each workgroup compacts the kept 64-key tiles of its q-tile into an
//    LDS list (chunks of 512 candidates); skipped tiles cost nothing and are
//    never read. Keys that must not count inside a processed tile (past a
//    segment end, or in a dropped block when mask blocks are smaller than the
//    tile) get a -1e30 bias added by one extra MFMA k-step: A[key][slot] is
//    0 or -1e30, B[slot][q] selects the query's slot (its q-block), so no
//    per-element compare/select is needed. -1e30 is finite, so no 0 x inf.
//  * int8 segments: the per-key K scale (floored at 2^-40, so that the bias
//    of a masked key stays far below any real score) multiplies score rows and the per-key
//    V scale multiplies P before its fp16 rounding (no lossy dequantised
//    copy). Calls with an int8 segment use that scaled path for every tile
//    (bf16 tiles get scale_log2 and 1); calls without one use the cheaper
//    unscaled path, with the row sum taken by v_dot2_f32_f16 over the same
//    fp16 P the MFMA multiplies.
//  * Grid is remapped so consecutive (head, q-tile) work items land on the
//    same XCD and share its L2 for K/V.
#include "sdit_internal.h"

namespace sdit {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BQ = kAttnBQ;
constexpr int BK = kAttnBK;
constexpr int NW = 4;
constexpr int NT = NW * 64;
constexpr int LIST_CAP = 512;
constexpr float TAU = 8.0f;           // lazy-rescale threshold (log2 units)
constexpr float MASK_BIAS = -1.0e30f; // added to scores of keys that must not count
// A row max below this comes only from biased keys: such a tile holds nothing
// visible for the row. Real scores in log2 units stay far above it, and a
// biased key stays below it because every score multiplier is >= KSC_MIN.
constexpr float MASKED_MAX = -1.0e15f;
constexpr float KSC_MIN = 0x1p-40f;   // floor of the per-key score multiplier
constexpr int NXCD = 8;

template <int D>
struct Layout {
  static constexpr int CPR = D / 8;            // 16-byte data chunks per row
  static constexpr int KS = D + 8;             // K row stride (bf16 elements)
  static constexpr int VS = D + 32;            // V row stride (fp16 elements)
  static constexpr int K_CH = KS / 8;          // chunks per padded K row
  static constexpr int K_BLKS = BK * K_CH / 64;  // 64-lane direct-load blocks per K tile
  static_assert(BK * K_CH % 64 == 0, "K tile must be whole 64-lane blocks");
};

template <int D>
struct Smem {
  uint16_t k[2][BK * Layout<D>::KS];  // bf16, padded rows
  uint16_t v[2][BK * Layout<D>::VS];  // fp16, padded rows
  float ksc[2][BK];                   // scaled path: per-key multiplier of the raw score
  float vsc[2][BK];                   // scaled path: per-key multiplier of P
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

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float i8_at(uint32_t w, int b) { return (float)(int)(int8_t)((w >> (8 * b)) & 0xFFu); }

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f16x2 h;
  h[0] = (_Float16)a;
  h[1] = (_Float16)b;
  return __builtin_bit_cast(uint32_t, h);
}

// 8 bf16 (one 16-byte chunk) -> 8 fp16
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 w) {
  return make_uint4(pack_f16(bf16_lo(w.x), bf16_hi(w.x)), pack_f16(bf16_lo(w.y), bf16_hi(w.y)),
                    pack_f16(bf16_lo(w.z), bf16_hi(w.z)), pack_f16(bf16_lo(w.w), bf16_hi(w.w)));
}

// 8 int8 codes (two words) -> 8 bf16 / 8 fp16 (exact: |code| <= 128)
__device__ __forceinline__ uint32_t i8pair_bf16(uint32_t w, int b) {
  return (__float_as_uint(i8_at(w, b)) >> 16) | (__float_as_uint(i8_at(w, b + 1)) & 0xFFFF0000u);
}
__device__ __forceinline__ uint4 i8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  return make_uint4(i8pair_bf16(w0, 0), i8pair_bf16(w0, 2), i8pair_bf16(w1, 0), i8pair_bf16(w1, 2));
}
__device__ __forceinline__ uint4 i8x8_to_f16x8(uint32_t w0, uint32_t w1) {
  return make_uint4(pack_f16(i8_at(w0, 0), i8_at(w0, 1)), pack_f16(i8_at(w0, 2), i8_at(w0, 3)),
                    pack_f16(i8_at(w1, 0), i8_at(w1, 1)), pack_f16(i8_at(w1, 2), i8_at(w1, 3)));
}

// Registers holding the register-staged part of one tile between its global
// load and its LDS store. bf16 tiles: D/32 chunks of 8 V values. int8 tiles:
// D/64 chunks of 16 K codes, then D/64 chunks of 16 V codes.
template <int D>
struct Stage {
  uint4 r[D / 32];
  float ks, vs;
};

// Per-thread load geometry, fixed for the whole kernel: element offsets (from
// a tile's first row, head included) of every chunk this thread moves.
template <int D>
struct LoadPlan {
  static constexpr int KMAX = (Layout<D>::K_BLKS + NW - 1) / NW;   // direct-load blocks per wave
  int k_off[KMAX];   // bf16 K, padded-tile block wave + NW*i (padding chunks reload chunk 0)
  int v_off;         // bf16 V chunk j adds j * (NT / CPR) rows
  int i8_off;        // int8 K/V chunk j adds j * (NT / (D/16)) rows
};

template <int D>
__device__ __forceinline__ void make_plan(LoadPlan<D>& pl, int row_stride) {
  using L = Layout<D>;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int i = 0; i < LoadPlan<D>::KMAX; ++i) {
    const int lin = (wave + NW * i) * 64 + lane;
    const int row = lin / L::K_CH, pc = lin % L::K_CH;
    pl.k_off[i] = row * row_stride + (pc < L::CPR ? pc : 0) * 8;
  }
  pl.v_off = (tid / L::CPR) * row_stride + (tid % L::CPR) * 8;
  pl.i8_off = (tid / (D / 16)) * row_stride + (tid % (D / 16)) * 16;
}

// Start loading tile t into buffer buf: bf16 K directly into LDS, the rest
// into registers (finished by commit_tile). Rows past the segment end are
// loaded from its last row: their scores get the -1e30 bias, so their
// probabilities are exactly 0 and any finite data there is harmless.
template <int D, bool SCALED>
__device__ __forceinline__ void issue_tile(const AttnParams& p, const TileInfo& t, int head, Stage<D>& st,
                                           Smem<D>& sm, int buf, const LoadPlan<D>& pl) {
  using L = Layout<D>;
  const AttnSegment& sg = p.seg[t.seg];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int row_stride = p.n_heads * D;   // elements between consecutive tokens
  const int64_t base = ((int64_t)t.key0 * p.n_heads + head) * D;
  const bool ragged = t.n_valid < BK;
  if (!SCALED || !sg.is_int8) {
    const uint16_t* kb = (const uint16_t*)sg.k + base;
    const uint16_t* vb = (const uint16_t*)sg.v + base;
#pragma unroll
    for (int i = 0; i < LoadPlan<D>::KMAX; ++i) {
      const int blk = wave + NW * i;
      if (blk < L::K_BLKS) {
        int off = pl.k_off[i];
        if (ragged) {
          const int lin = blk * 64 + lane;
          const int row = lin / L::K_CH, pc = lin % L::K_CH;
          off = min(row, t.n_valid - 1) * row_stride + (pc < L::CPR ? pc : 0) * 8;
        }
        __builtin_amdgcn_global_load_lds((const void*)(kb + off), (lds_void*)(sm.k[buf] + blk * 64 * 8), 16, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
      constexpr int RSTEP = NT / L::CPR;
      int off = pl.v_off + j * RSTEP * row_stride;
      if (ragged) off = min(tid / L::CPR + j * RSTEP, t.n_valid - 1) * row_stride + (tid % L::CPR) * 8;
      st.r[j] = *reinterpret_cast<const uint4*>(vb + off);
    }
    if (SCALED && tid < BK) {
      st.ks = p.scale_log2;
      st.vs = tid < t.n_valid ? 1.0f : 0.0f;
    }
  } else {
    const int8_t* kb = (const int8_t*)sg.k + base;
    const int8_t* vb = (const int8_t*)sg.v + base;
#pragma unroll
    for (int j = 0; j < D / 64; ++j) {
      constexpr int RSTEP = NT / (D / 16);
      int off = pl.i8_off + j * RSTEP * row_stride;
      if (ragged) off = min(tid / (D / 16) + j * RSTEP, t.n_valid - 1) * row_stride + (tid % (D / 16)) * 16;
      st.r[j] = *reinterpret_cast<const uint4*>(kb + off);
      st.r[D / 64 + j] = *reinterpret_cast<const uint4*>(vb + off);
    }
    if (tid < BK) {
      // keys past the segment end keep a positive K multiplier so their bias stays -1e30
      const bool ok = tid < t.n_valid;
      const int64_t si = (int64_t)(t.key0 + min(tid, t.n_valid - 1)) * p.n_heads + head;
      const float ksv = sg.k_scale[si], vsv = sg.v_scale[si];
      st.ks = ok ? fmaxf(ksv * p.scale_log2, KSC_MIN) : p.scale_log2;
      st.vs = ok ? vsv : 0.f;
    }
  }
}

template <int D, bool SCALED>
__device__ __forceinline__ void commit_tile(const AttnParams& p, const TileInfo& t, const Stage<D>& st,
                                            Smem<D>& sm, int buf) {
  using L = Layout<D>;
  const int tid = threadIdx.x;
  if (!SCALED || !p.seg[t.seg].is_int8) {
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
      const int lin = tid + j * NT;
      const int row = lin / L::CPR, c = lin % L::CPR;
      *reinterpret_cast<uint4*>(sm.v[buf] + row * L::VS + c * 8) = bf16x8_to_f16x8(st.r[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < D / 64; ++j) {
      const int lin = tid + j * NT;
      const int row = lin / (D / 16), c16 = lin % (D / 16);
      uint16_t* kr = sm.k[buf] + row * L::KS + 16 * c16;
      uint16_t* vr = sm.v[buf] + row * L::VS + 16 * c16;
      const uint4 kc = st.r[j], vc = st.r[D / 64 + j];
      *reinterpret_cast<uint4*>(kr) = i8x8_to_bf16x8(kc.x, kc.y);
      *reinterpret_cast<uint4*>(kr + 8) = i8x8_to_bf16x8(kc.z, kc.w);
      *reinterpret_cast<uint4*>(vr) = i8x8_to_f16x8(vc.x, vc.y);
      *reinterpret_cast<uint4*>(vr + 8) = i8x8_to_f16x8(vc.z, vc.w);
    }
  }
  if (SCALED && tid < BK) {
    sm.ksc[buf][tid] = st.ks;
    sm.vsc[buf][tid] = st.vs;
  }
}

__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

__device__ __forceinline__ float swap_halves_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

__device__ __forceinline__ float swap_halves_sum(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// V^T operand for column tile dt and 16-key group kk: two transposed 8-byte
// reads (keys 4*hh + 0..3 and 8 + 4*hh + 0..3 of the group, one column per lane).
template <int D>
__device__ __forceinline__ f16x8 read_vt(const uint16_t* vl, int v_lane, int dt, int kk) {
  using L = Layout<D>;
  const uint16_t* va = vl + v_lane + kk * 16 * L::VS + dt * 32;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(va));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(va + 8 * L::VS));
  const f16x4 lo_h = __builtin_bit_cast(f16x4, lo);
  const f16x4 hi_h = __builtin_bit_cast(f16x4, hi);
  return f16x8{lo_h[0], lo_h[1], lo_h[2], lo_h[3], hi_h[0], hi_h[1], hi_h[2], hi_h[3]};
}

// Per-lane state of one wave that persists across tiles.
template <int D>
struct WaveState {
  bf16x8 qf[D / 16];   // Q^T fragments (B operand of S^T = K Q^T)
  bf16x8 qsel;         // B operand of the bias k-step: picks the lane's slot
  f32x16 o[D / 32];    // O^T accumulators
  float m_run;         // running max, log2 units
  float l_run;         // this lane's half of the row sum
  bool seen;           // general masks: a kept key reached this row
};

// One 64-key tile for one wave: S^T = K Q^T, masking bias, online softmax,
// O^T += V^T P^T. Element e2 of score subtile kt is key kt*32 + 8*(e2/4) +
// 4*hh + e2%4 of the tile.
template <int D, bool SCALED, bool GENERAL>
__device__ __forceinline__ void compute_tile(const AttnParams& p, const TileInfo& t, WaveState<D>& ws,
                                             const uint16_t* kl, const uint16_t* vl, const float* ksc,
                                             const float* vsc, int k_lane, int v_lane, int r, int hh,
                                             int my_qb, int qb_lo, int n_qbt) {
  using L = Layout<D>;
  constexpr int NKS = D / 16;
  constexpr int NDT = D / 32;
  // LDS operand reads in flight ahead of their MFMA (the scaled path needs the registers)
  constexpr int PF = SCALED ? 2 : 4;

  // ---- S^T = K Q^T for two 32-key subtiles; operand reads PF steps ahead,
  // scheduling fences keep the compiler from hoisting all of them
  constexpr int NQK = 2 * NKS;
  f32x16 s[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int e2 = 0; e2 < 16; ++e2) s[kt][e2] = 0.f;
  {
    bf16x8 ka[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i)
      ka[i] = *reinterpret_cast<const bf16x8*>(kl + k_lane + (i / NKS) * 32 * L::KS + (i % NKS) * 16);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const bf16x8 a = ka[i % PF];
      if (i + PF < NQK)
        ka[i % PF] = *reinterpret_cast<const bf16x8*>(kl + k_lane + ((i + PF) / NKS) * 32 * L::KS +
                                                      ((i + PF) % NKS) * 16);
      s[i / NKS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ws.qf[i % NKS], s[i / NKS], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- masking bias: one extra k-step. A[key][slot] in lane (key, hh = 0)
  if (GENERAL || t.n_valid < BK) {
    const AttnSegment& sg = p.seg[t.seg];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = kt * 32 + r;
      const bool kvalid = key < t.n_valid;
      bf16x8 a;
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] = (__bf16)0.0f;
      if (hh == 0) {
        if (GENERAL) {
          const int kb = sg.kb_start + (t.key0 + min(key, t.n_valid - 1)) / p.block_k;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const bool keep = kvalid && j < n_qbt && p.mask[(int64_t)(qb_lo + j) * p.n_kb + kb] != 0;
            a[j] = keep ? (__bf16)0.0f : (__bf16)MASK_BIAS;
          }
        } else {
          a[0] = kvalid ? (__bf16)0.0f : (__bf16)MASK_BIAS;
        }
      }
      s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ws.qsel, s[kt], 0, 0, 0);
    }
    if (GENERAL) {
      // does any kept key of this tile reach this lane's query row?
      const int kb_lo = sg.kb_start + t.key0 / p.block_k;
      const int kb_hi = sg.kb_start + (t.key0 + t.n_valid - 1) / p.block_k;
      for (int kb = kb_lo; kb <= kb_hi; ++kb) ws.seen |= p.mask[(int64_t)my_qb * p.n_kb + kb] != 0;
    }
  }

  // ---- scores in log2 units and the tile's row max
  float mt = -INFINITY;
  if (SCALED) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 sc = *reinterpret_cast<const float4*>(&ksc[kt * 32 + 8 * g + 4 * hh]);
        s[kt][4 * g + 0] *= sc.x;
        s[kt][4 * g + 1] *= sc.y;
        s[kt][4 * g + 2] *= sc.z;
        s[kt][4 * g + 3] *= sc.w;
      }
  }
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int e2 = 0; e2 < 16; e2 += 2) mt = max3(mt, s[kt][e2], s[kt][e2 + 1]);
  // unscaled path: raw scores, scale_log2 folded into the exponent's FMA
  const float cs = SCALED ? 1.0f : p.scale_log2;
  mt = swap_halves_max(mt) * cs;
  if (mt < MASKED_MAX) mt = -INFINITY;   // nothing visible for this row in the tile

  // ---- online softmax (lazy running max)
  const bool need = mt > ws.m_run + TAU;
  if (__ballot(need)) {
    const float m_new = need ? mt : ws.m_run;
    const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(ws.m_run - m_new);
    ws.m_run = m_new;
    ws.l_run *= alpha;
#pragma unroll
    for (int i = 0; i < NDT; ++i)
#pragma unroll
      for (int e2 = 0; e2 < 16; ++e2) ws.o[i][e2] *= alpha;
  }
  const float m_use = (ws.m_run == -INFINITY) ? 0.f : ws.m_run;

  f16x2 ones;
  ones[0] = (_Float16)1.0f;
  ones[1] = (_Float16)1.0f;
  f16x8 pb[4];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    float pv[16];
#pragma unroll
    for (int e2 = 0; e2 < 16; ++e2) pv[e2] = __builtin_amdgcn_exp2f(fmaf(s[kt][e2], cs, -m_use));
    if (SCALED) {
#pragma unroll
      for (int e2 = 0; e2 < 16; ++e2) ws.l_run += pv[e2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 sc = *reinterpret_cast<const float4*>(&vsc[kt * 32 + 8 * g + 4 * hh]);
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
      if (!SCALED) {
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          f16x2 pr;
          pr[0] = v[j];
          pr[1] = v[j + 1];
          ws.l_run = __builtin_amdgcn_fdot2(pr, ones, ws.l_run, false);
        }
      }
    }
  }

  // ---- O^T += V^T P^T (transposed reads of the row-major fp16 V tile)
  {
    constexpr int NPV = 4 * NDT;
    f16x8 va[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) va[i] = read_vt<D>(vl, v_lane, i / 4, i % 4);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const f16x8 a = va[i % PF];
      if (i + PF < NPV) va[i % PF] = read_vt<D>(vl, v_lane, (i + PF) / 4, (i + PF) % 4);
      ws.o[i / 4] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[i % 4], ws.o[i / 4], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int D, bool SCALED, bool GENERAL>
__global__ __launch_bounds__(NT, 2) void attn_fwd_kernel(AttnParams p) {
  using L = Layout<D>;
  __shared__ __attribute__((aligned(16))) Smem<D> sm;
  constexpr int NKS = D / 16;
  constexpr int NDT = D / 32;

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
  const int s16 = lane & 15;     // lane inside its 16-lane group (transposed V reads)
  const int g16 = lane >> 4;
  const int q_row = qt * BQ + wave * 32 + r;
  const bool q_ok = q_row < p.n_q;

  // q-block range of this workgroup (mask lookups and bias slots)
  const int q_lo = qt * BQ;
  const int q_hi = min(p.n_q, q_lo + BQ) - 1;
  const int qb_lo = q_lo / p.block_q, qb_hi = q_hi / p.block_q;
  const int n_qbt = qb_hi - qb_lo + 1;
  const int my_qb = min(q_row, p.n_q - 1) / p.block_q;

  WaveState<D> ws;
  {
    const uint16_t* qp = p.q + ((int64_t)q_row * p.n_heads + head) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      uint4 w = q_ok ? *reinterpret_cast<const uint4*>(qp + ks * 16) : make_uint4(0, 0, 0, 0);
      ws.qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
    // bias selector: slot = the lane's q-block inside the tile (general masks) or slot 0
    const int slot = GENERAL ? my_qb - qb_lo : 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) ws.qsel[j] = (hh == 0 && j == slot) ? (__bf16)1.0f : (__bf16)0.0f;
  }
#pragma unroll
  for (int i = 0; i < NDT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) ws.o[i][e] = 0.f;
  ws.m_run = -INFINITY;
  ws.l_run = 0.f;
  ws.seen = !GENERAL;

  // per-lane LDS offsets (elements) that do not change over the loop
  const int k_lane = r * L::KS + 8 * hh;
  // transposed V read: row (4*hh + s16/4) of each 8-key group, 4 columns at
  // 16*(g16&1) + 4*(s16&3) inside each 32-column tile
  const int v_lane = (4 * hh + (s16 >> 2)) * L::VS + 16 * (g16 & 1) + 4 * (s16 & 3);

  int buf = 0;
  Stage<D> st;
  LoadPlan<D> plan;
  make_plan<D>(plan, p.n_heads * D);

#pragma unroll 1
  for (int cbase = 0; cbase < p.n_tiles; cbase += LIST_CAP) {
    // ---- compact the kept tiles of this chunk into sm.list (order preserved)
    const int ncand = min(LIST_CAP, p.n_tiles - cbase);
    bool keep[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = 2 * tid + i;
      keep[i] = false;
      if (c < ncand) {
        const TileInfo t = tile_info(p, cbase + c);
        const AttnSegment& sg = p.seg[t.seg];
        const int kb_lo = sg.kb_start + t.key0 / p.block_k;
        const int kb_hi = sg.kb_start + (t.key0 + t.n_valid - 1) / p.block_k;
        bool any = false;
        for (int qb = qb_lo; qb <= qb_hi && !any; ++qb)
          for (int kb = kb_lo; kb <= kb_hi; ++kb) any |= p.mask[(int64_t)qb * p.n_kb + kb] != 0;
        keep[i] = any;
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
      if (keep[0]) sm.list[pos++] = (uint16_t)(2 * tid);
      if (keep[1]) sm.list[pos] = (uint16_t)(2 * tid + 1);
    }
    __syncthreads();
    if (total == 0) continue;

    // ---- prologue: first kept tile into LDS
    {
      const TileInfo t = tile_info(p, cbase + sm.list[0]);
      issue_tile<D, SCALED>(p, t, head, st, sm, buf, plan);
      commit_tile<D, SCALED>(p, t, st, sm, buf);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    TileInfo tn = tile_info(p, cbase + sm.list[0]);
#pragma unroll 1
    for (int it = 0; it < total; ++it) {
      const TileInfo t = tn;
      const bool has_next = it + 1 < total;
      if (has_next) {
        tn = tile_info(p, cbase + sm.list[it + 1]);
        issue_tile<D, SCALED>(p, tn, head, st, sm, buf ^ 1, plan);
      }
      compute_tile<D, SCALED, GENERAL>(p, t, ws, sm.k[buf], sm.v[buf], sm.ksc[buf], sm.vsc[buf], k_lane, v_lane,
                                       r, hh, my_qb, qb_lo, n_qbt);
      if (has_next) commit_tile<D, SCALED>(p, tn, st, sm, buf ^ 1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      buf ^= 1;
    }
  }

  // ---- finalise
  const float l_tot = swap_halves_sum(ws.l_run);
  const bool any = ws.seen && l_tot > 0.f;
  const float inv = any ? 1.0f / l_tot : 0.f;
  if (q_ok) {
    uint16_t* op = p.out + ((int64_t)q_row * p.n_heads + head) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = dt * 32 + 8 * g + 4 * hh;
        // rows without a visible key store +0 (o * 0 could give -0)
        const __bf16 v0 = (__bf16)(any ? ws.o[dt][4 * g + 0] * inv : 0.0f);
        const __bf16 v1 = (__bf16)(any ? ws.o[dt][4 * g + 1] * inv : 0.0f);
        const __bf16 v2 = (__bf16)(any ? ws.o[dt][4 * g + 2] * inv : 0.0f);
        const __bf16 v3 = (__bf16)(any ? ws.o[dt][4 * g + 3] * inv : 0.0f);
        const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, v0) | ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
        const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, v2) | ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
        *reinterpret_cast<uint2*>(op + d) = make_uint2(w0, w1);
      }
    if (p.lse != nullptr && hh == 0) {
      const float ln2 = 0.69314718055994530942f;
      p.lse[(int64_t)head * p.n_q + q_row] = any ? (ws.m_run + __log2f(l_tot)) * ln2 : -INFINITY;
    }
  }
}

template <int D, bool SCALED, bool GENERAL>
hipError_t launch(const AttnParams& p, hipStream_t stream) {
  const unsigned blocks = (unsigned)(p.n_qt * p.n_heads);
  hipLaunchKernelGGL((attn_fwd_kernel<D, SCALED, GENERAL>), dim3(blocks), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnParams& p, hipStream_t stream) {
  bool scaled = false;
  for (int s = 0; s < p.n_segs; ++s) scaled |= p.seg[s].is_int8 && p.seg[s].len > 0;
  // mask blocks finer than the 128-row x 64-key tile need the per-q-block bias
  const bool general = p.block_q < BQ || p.block_k < BK;
  if (scaled) return general ? launch<D, true, true>(p, stream) : launch<D, true, false>(p, stream);
  return general ? launch<D, false, true>(p, stream) : launch<D, false, false>(p, stream);
}

}  // namespace

hipError_t launch_attn_fwd(const AttnParams& p, int head_dim, hipStream_t stream) {
  if (p.n_q == 0) return hipSuccess;
  return head_dim == 128 ? launch_d<128>(p, stream) : launch_d<64>(p, stream);
}

}  // namespace sdit
