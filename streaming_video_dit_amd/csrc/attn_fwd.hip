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
//  * One workgroup = one head x 256 query rows, 8 waves of 32 rows each, one
//    workgroup per CU (LDS ~105 KB), so two waves share every SIMD. Waves
//    4..7 run half a tile behind waves 0..3: in each step they first
//    multiply the previous tile's P with V, then compute the current tile's
//    scores and softmax, while waves 0..3 do scores, softmax, P.V of the
//    current tile. On every SIMD one wave's softmax (vector ALU) then
//    overlaps the other wave's matrix work. A 64-key K/V tile loaded once
//    serves all 256 rows.
//  * Keys stream through LDS in 64-key tiles, one barrier per tile. K is
//    double buffered, V triple buffered (the lagging waves still read tile
//    i-1 while tile i+1 is written). bf16 K goes straight from global memory
//    into LDS (buffer_load_dwordx4 ... lds: lane t lands at base + 16 t, so
//    each lane's source offset is chosen to realise the padded layout below).
//    V is staged through registers and converted to fp16; int8 K/V codes are
//    widened exactly on the same path. Every tile load addresses a per-tile
//    buffer resource with a fixed 32-bit per-lane offset (no address
//    arithmetic in the loop); rows past a segment end read as zeros. Each wave's share of a tile's
//    register loads is issued between its score MFMAs rather than all at
//    once (a burst from every wave queues in the CU's address unit and
//    stalls the issuing waves).
//  * Who moves the tiles differs by kernel. Without int8 segments every tile
//    is loaded one step ahead: the four leading waves issue the direct K
//    loads and stage V, during their score MFMAs (they wait at the barrier
//    for the lagging waves, which then carry none of the loading; measured
//    1.5% faster than spreading V over all eight waves on the dense chunks,
//    within noise on the block-sparse one). With int8 segments all eight waves
//    stage (the int8 tiles need the registers), two steps ahead: each wave
//    commits its share of tile i+1 in step i, the leading waves first (then
//    scores, softmax, P.V: vector, matrix, vector, matrix), the lagging ones
//    between their P.V of tile i-1 and their scores of tile i (matrix,
//    vector, matrix, vector), so on every SIMD the two waves alternate
//    between the matrix and the vector units.
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
//    P stays <= 256 and the rescale is skipped for almost every tile. The
//    exponentials are taken with the running max first; the tile's row max is
//    only computed when some lane's P sum reaches 2^8.
//  * Mask: each workgroup compacts the kept 64-key tiles of its 256 rows into
//    an LDS list of packed descriptors (key offset, segment, valid keys, and
//    which waves have a kept (q-block, k-block) pair in the tile), passes of
//    1024 candidates; skipped tiles cost nothing and are never read, a wave
//    whose rows keep nothing in a listed tile skips its compute, and the
//    loop reads one descriptor per tile instead of searching the segment
//    table. Keys that must not count inside a processed tile (past a segment
//    end, or in a dropped block when mask blocks are finer than a wave's 32
//    rows or the 64-key tile) get a -1e30 bias added by one extra MFMA
//    k-step: A[key][slot] is 0 or -1e30, B[slot][q] selects the query's slot
//    (its q-block inside the workgroup, up to 16 slots over the two lane
//    halves), so no per-element compare/select is needed. -1e30 is finite,
//    so no 0 x inf.
//  * int8 segments: the per-key K scale (floored at 2^-40, so that the bias
//    of a masked key stays far below any real score) multiplies score rows
//    (K itself stays the exact code in bf16). V is staged as code x scale in
//    fp16: the code is exact in fp16, the row's scale is rounded to fp16 and
//    the product rounded once (each at most 2^-11 relative, the size of P's
//    own fp16 rounding); done once per tile while staging, rather than as a
//    multiply of P in every wave. Calls with an int8 segment use the scaled
//    path for every tile (bf16 tiles get scale_log2); calls without one
//    skip the per-key score multiply. Both take the row sum with
//    v_dot2_f32_f16 over the same fp16 P the MFMA multiplies.
//  * Grid is remapped so consecutive (head, q-tile) work items land on the
//    same XCD and share its L2 for K/V.
//  * Balanced launches (sdit_attn_fwd_balanced): on an XCD whose units leave
//    a partial last wave, those units run as head pieces over the candidate
//    tiles before a cut and tail pieces over the rest, on the CUs the partial
//    wave would leave idle; both write normalised fp32 O and LSE to
//    workspace slots, merged afterwards by attn_split_merge_kernel. The head
//    pieces all start at the first key tile, so the XCD's units still walk
//    the keys together.
#include "sdit_internal.h"

#include <type_traits>

namespace sdit {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource over the bytes [base, base + n_bytes): raw (stride 0),
// word 3 = the gfx9 32-bit data format. A tile's loads address it with one
// 32-bit per-lane offset (no 64-bit address arithmetic in the loop), and a
// load at or past n_bytes reads zeros without touching memory: that is how
// the rows past a segment end are read.
// Both arguments are wave-uniform; readfirstlane states it, so the compiler
// never wraps a load in a loop over distinct resources.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, uint32_t n_bytes) {
  const uint64_t a = (uint64_t)base;
  const uint64_t u = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a) |
                     ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) << 32);
  return __builtin_amdgcn_make_buffer_rsrc((void*)u, (short)0, __builtin_amdgcn_readfirstlane((int)n_bytes), 0x00020000);
}
// 16 bytes per lane from the resource at byte offset off straight into LDS:
// lane t lands at lds_dst + 16 t
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t rs, void* lds_dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds_dst, 16, off, 0, 0, 0);
}

constexpr int BQ = kAttnBQ;
constexpr int BK = kAttnBK;
constexpr int NW = 8;                 // waves per workgroup, 32 query rows each
constexpr int NT = NW * 64;
constexpr int LIST_CAP = 2 * NT;      // kept-tile list entries per compaction pass
constexpr int NVBUF = 3;              // V tiles in flight: two being read, one being written
constexpr float TAU = 8.0f;           // lazy-rescale threshold (log2 units)
constexpr float MASK_BIAS = -1.0e30f; // added to scores of keys that must not count
// A row max below this comes only from biased keys: such a tile holds nothing
// visible for the row. Real scores in log2 units stay far above it, and a
// biased key stays below it because every score multiplier is >= KSC_MIN.
constexpr float MASKED_MAX = -1.0e15f;
constexpr float KSC_MIN = 0x1p-40f;   // floor of the per-key score multiplier
constexpr int NXCD = kNumXcd;
// A test-only build (SDIT_SINGLE_STAGE=1) replaces the pipelined schedules by
// one that loads a tile, waits, and computes it with every wave, one tile at
// a time. Each wave then does the same arithmetic on the same tiles in the
// same order, so its results must match the pipelined kernel bit for bit
// (a drifting prefetch would show up as a difference).
#ifndef SDIT_SINGLE_STAGE
#define SDIT_SINGLE_STAGE 0
#endif
constexpr bool kSingleStage = SDIT_SINGLE_STAGE != 0;
static_assert(BQ == NW * 32, "one wave per 32 query rows");

template <int D>
struct Layout {
  static constexpr int CPR = D / 8;            // 16-byte data chunks per row
  static constexpr int KS = D + 8;             // K row stride (bf16 elements)
  static constexpr int VS = D + 32;            // V row stride (fp16 elements)
  static constexpr int K_CH = KS / 8;          // chunks per padded K row
  static constexpr int K_BLKS = BK * K_CH / 64;  // 64-lane direct-load blocks per K tile
  static_assert(BK * K_CH % 64 == 0, "K tile must be whole 64-lane blocks");
};

// Who moves a tile. bf16 K goes from global memory straight into LDS,
// issued by the first KW waves (the ones that run ahead). V (bf16 -> fp16)
// and int8 K/V codes are staged through the registers of the first ST
// threads: the four leading waves in the unscaled kernels, all eight in
// the scaled ones (the int8 tiles need the registers).
template <int D, int ST>
struct Loader {
  static constexpr int KW = NW / 2;
  static constexpr int VCH = BK * Layout<D>::CPR / ST;  // bf16 V chunks staged per thread
  static constexpr int I8_THREADS = BK * (D / 16);      // threads moving 16 int8 codes of K and of V
  static constexpr int I8CH = I8_THREADS >= ST ? I8_THREADS / ST : 1;
  static constexpr int KMAX = (Layout<D>::K_BLKS + KW - 1) / KW;   // direct-load blocks per K wave
  // staged registers and one-instruction load parts per tile (scaled kernels
  // also stage int8 tiles: K codes, V codes, then the per-key scales)
  template <bool SCALED>
  static constexpr int sr() { return SCALED && 2 * I8CH > VCH ? 2 * I8CH : VCH; }
  template <bool SCALED>
  static constexpr int npart() { return SCALED && 2 * I8CH + 1 > VCH ? 2 * I8CH + 1 : VCH; }
  static_assert(VCH >= 1 && BK * Layout<D>::CPR % ST == 0, "V tile must be whole chunks per thread");
  static_assert(I8_THREADS % ST == 0 || I8_THREADS < ST, "int8 tile split");
};

template <int D>
struct Smem {
  uint16_t k[2][BK * Layout<D>::KS];      // bf16, padded rows
  uint16_t v[NVBUF][BK * Layout<D>::VS];  // fp16, padded rows
  float ksc[2][BK];                       // scaled path: per-key multiplier of the raw score
  uint2 desc[LIST_CAP];                   // kept tiles of the current pass (pack_desc)
  // fine masks: per listed tile, bit 16 j + s = mask[first q-block + s][first
  // k-block of the tile + j] (up to 16 q-blocks of the rows, 4 k-blocks of a tile)
  uint64_t kbits[LIST_CAP];
  int32_t wave_count[NW];
  float vmax[NW];   // every wave's largest staged V magnitude (exact form)
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

// A kept tile as the main loop sees it: wave-uniform values read once per
// step from the LDS descriptor list and the segment table.
struct TileRef {
  const void* k;
  const void* v;
  const float* k_scale;
  const float* v_scale;
  int key0;
  int n_valid;
  int is_int8;
  int kb_start;
  int wmask;   // waves with a kept (q-block, k-block) pair in the tile
  uint64_t kbits;  // fine masks only: the tile's (q-block, k-block) keep bits (Smem::kbits)
};

// descriptor: x = first key inside the segment, y = segment | n_valid << 8 | wave mask << 16
__device__ __forceinline__ uint2 pack_desc(const TileInfo& t, uint32_t wmask) {
  return make_uint2((uint32_t)t.key0, (uint32_t)t.seg | ((uint32_t)t.n_valid << 8) | (wmask << 16));
}

__device__ __forceinline__ TileRef tile_ref(const AttnParams& p, uint2 d) {
  const uint32_t x = __builtin_amdgcn_readfirstlane(d.x);
  const uint32_t y = __builtin_amdgcn_readfirstlane(d.y);
  const AttnSegment& sg = p.seg[y & 0xFF];
  TileRef t;
  t.k = sg.k;
  t.v = sg.v;
  t.k_scale = sg.k_scale;
  t.v_scale = sg.v_scale;
  t.is_int8 = sg.is_int8;
  t.kb_start = sg.kb_start;
  t.key0 = (int)x;
  t.n_valid = (int)((y >> 8) & 0xFF);
  t.wmask = (int)(y >> 16);
  // complete the scalar loads here, before the step's LDS traffic starts
  // (their wait would otherwise also wait for every LDS read in flight)
  asm volatile("" ::"s"(t.k), "s"(t.v), "s"(t.k_scale), "s"(t.v_scale), "s"(t.is_int8), "s"(t.kb_start));
  return t;
}

// Listed tile i (fine masks: with its keep bits).
template <int D, bool GENERAL>
__device__ __forceinline__ TileRef tile_at(const AttnParams& p, const Smem<D>& sm, int i) {
  TileRef t = tile_ref(p, sm.desc[i]);
  t.kbits = 0;
  if (GENERAL) {
    const uint64_t b = sm.kbits[i];
    // readfirstlane returns int: widen through uint32_t (no sign extension)
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    t.kbits = (uint64_t)lo | ((uint64_t)hi << 32);
  }
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
// the same, each value times 2^e before its one rounding to fp16
__device__ __forceinline__ uint32_t pack_f16_exp(float a, float b, int e) { return pack_f16(ldexpf(a, e), ldexpf(b, e)); }
__device__ __forceinline__ uint4 bf16x8_to_f16x8_exp(uint4 w, int e) {
  return make_uint4(pack_f16_exp(bf16_lo(w.x), bf16_hi(w.x), e), pack_f16_exp(bf16_lo(w.y), bf16_hi(w.y), e),
                    pack_f16_exp(bf16_lo(w.z), bf16_hi(w.z), e), pack_f16_exp(bf16_lo(w.w), bf16_hi(w.w), e));
}
// largest magnitude among 8 bf16 values and m
__device__ __forceinline__ float absmax_bf16x8(uint4 w, float m) {
  m = fmaxf(m, fmaxf(fabsf(bf16_lo(w.x)), fabsf(bf16_hi(w.x))));
  m = fmaxf(m, fmaxf(fabsf(bf16_lo(w.y)), fabsf(bf16_hi(w.y))));
  m = fmaxf(m, fmaxf(fabsf(bf16_lo(w.z)), fabsf(bf16_hi(w.z))));
  return fmaxf(m, fmaxf(fabsf(bf16_lo(w.w)), fabsf(bf16_hi(w.w))));
}

// ---- V exponents. P.V multiplies fp16 P with fp16 V. bf16 V converts to fp16
// exactly only between 2^-17 and 65280 in magnitude (below, fp16 has too few
// bits; above, it overflows), and an int8 row's V = code * fp16(scale) keeps
// 11 bits only while the scale is a normal fp16 (>= 2^-14). So every 64-key V
// tile is staged as V * 2^e, one exponent for the whole tile chosen from its
// largest magnitude M (bf16 tiles: max |v|; int8 tiles: the largest V scale):
// e = 0 while M lies in the band below, else the multiple of 16 that brings M
// into it. A wave folds 2^(e - e_prev) into its fp32 O accumulators whenever
// the exponent of the tiles it multiplies changes (an exact power-of-two
// rescale, like the lazy max) and 2^-e into the final 1/l. Within a tile every
// staged value then carries at most 2^-11 relative error, or 2^-17 M absolute
// for elements more than 2^14 below the tile's largest (the fp16 subnormal
// step), and nothing overflows: P <= 2^8 times |V 2^e| < 2^16 per product.
constexpr float V_BF16_LO = 0x1p-8f, V_BF16_HI = 0x1p16f;   // bf16 band [2^-8, 2^16)
constexpr float V_I8_LO = 0x1p-8f, V_I8_HI = 0x1p8f;        // int8 scale band [2^-8, 2^8)

__device__ __forceinline__ int band_exponent(float m, float lo, float hi) {
  if (!(m > 0.f) || (m >= lo && m < hi) || !(m < INFINITY)) return 0;
  const int k = __builtin_amdgcn_frexp_expf(m) - 1;   // m in [2^k, 2^(k+1))
  // floor((k + 8) / 16) for negative k + 8 too
  const int f = (k + 8) >= 0 ? (k + 8) / 16 : -((15 - (k + 8)) / 16);
  return -16 * f;
}
__device__ __forceinline__ int v_exponent(float m, bool is_int8) {
  return is_int8 ? band_exponent(m, V_I8_LO, V_I8_HI) : band_exponent(m, V_BF16_LO, V_BF16_HI);
}

// largest value of x over the wave (x >= 0), returned in every lane
__device__ __forceinline__ float wave_max(float x) {
  auto dpp = [](float v, int ctrl) -> float {
    switch (ctrl) {
      case 0: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
      case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
      case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true));
      default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, true));
    }
  };
  x = fmaxf(x, dpp(x, 0));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp(x, 1));   // quad_perm [2,3,0,1]: every quad holds its max
  x = fmaxf(x, dpp(x, 2));   // row_half_mirror: groups of 8
  x = fmaxf(x, dpp(x, 3));   // row_mirror: rows of 16
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// 8 int8 codes (two words) -> 8 bf16 / 8 fp16 (exact: |code| <= 128)
// Two int8 codes (bytes b, b+1 of w) -> two bf16: |code| <= 128 is exact in
// fp32 and bf16, so the upper halves of the fp32 values are the bf16 values
// (one byte permute packs them).
__device__ __forceinline__ uint32_t i8pair_bf16(uint32_t w, int b) {
  return __builtin_amdgcn_perm(__float_as_uint(i8_at(w, b + 1)), __float_as_uint(i8_at(w, b)), 0x07060302u);
}
__device__ __forceinline__ uint4 i8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  return make_uint4(i8pair_bf16(w0, 0), i8pair_bf16(w0, 2), i8pair_bf16(w1, 0), i8pair_bf16(w1, 2));
}
// Four int8 codes -> four fp16, exactly: flipping the sign bits gives the
// bytes u = code + 128 in [0, 255]; placed under the fp16 exponent of 1024
// (bit pattern 0x6400 | u) they read 1024 + u, and subtracting 1152 leaves
// the code (an exact difference of nearby values).
__device__ __forceinline__ uint2 i8x4_to_f16x4(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  const f16x2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  const f16x2 lo = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) + bias;
  const f16x2 hi = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) + bias;
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}
__device__ __forceinline__ uint4 i8x8_to_f16x8(uint32_t w0, uint32_t w1) {
  const uint2 a = i8x4_to_f16x4(w0), b = i8x4_to_f16x4(w1);
  return make_uint4(a.x, a.y, b.x, b.y);
}
// 8 fp16 values times s (packed fp16 multiplies, one rounding each)
__device__ __forceinline__ uint4 scale_f16x8(uint4 x, f16x2 s) {
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, x.x) * s),
                    __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, x.y) * s),
                    __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, x.z) * s),
                    __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, x.w) * s));
}

// Registers holding the register-staged part of one tile between its global
// load and its LDS store. bf16 tiles: VCH chunks of 8 V values. int8 tiles:
// 16 K codes and 16 V codes of one key row, that row's V scale (vs), and
// (threads 0..BK-1) the K scale of key row tid (ks).
template <int D, int ST, bool SCALED>
struct Stage {
  uint4 r[Loader<D, ST>::template sr<SCALED>()];
  float ks, vs;
};

// Per-thread load geometry, fixed for the whole kernel: byte offsets, from a
// tile's first row (head included), of every chunk this thread moves. The
// host allows at most 65536 heads, so a row is at most 2^24 bytes and every
// offset and resource size within a 64-key tile stays below 2^30.
template <int D, int ST>
struct LoadPlan {
  static constexpr int KMAX = Loader<D, ST>::KMAX;
  static constexpr int VCH = Loader<D, ST>::VCH;
  uint32_t k_off[KMAX];   // bf16 K (K waves), padded-tile block wave + KW*i (padding chunks reload chunk 0)
  uint32_t v_off[VCH];    // bf16 V chunk j: rows j * (ST / CPR) further down
  uint32_t i8_off;        // int8 K/V codes (one chunk)
};

template <int D, int ST>
__device__ __forceinline__ void make_plan(LoadPlan<D, ST>& pl, uint32_t row_bytes) {
  using L = Layout<D>;
  constexpr int KW = Loader<D, ST>::KW;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int i = 0; i < LoadPlan<D, ST>::KMAX; ++i) {
    const int lin = (wave + KW * i) * 64 + lane;
    const int row = lin / L::K_CH, pc = lin % L::K_CH;
    pl.k_off[i] = row * row_bytes + (pc < L::CPR ? pc : 0) * 16;
  }
#pragma unroll
  for (int j = 0; j < LoadPlan<D, ST>::VCH; ++j)
    pl.v_off[j] = (tid / L::CPR + j * (ST / L::CPR)) * row_bytes + (tid % L::CPR) * 16;
  // int8 rows are half as long as bf16 rows
  pl.i8_off = (tid / (D / 16)) * (row_bytes / 2) + (tid % (D / 16)) * 16;
}

// bf16 K of tile t straight into LDS buffer kbuf (K waves only). Rows past
// the segment end read as zeros (the tile's buffer resource ends with the
// segment): their scores get the -1e30 bias, so their probabilities are
// exactly 0.
template <int D, int ST>
__device__ __forceinline__ void issue_kdma_to(const AttnParams& p, const TileRef& t, int head, uint16_t* kdst,
                                              const LoadPlan<D, ST>& pl) {
  using L = Layout<D>;
  constexpr int KW = Loader<D, ST>::KW;
  // only the K waves (0..KW-1) get here; the mask tells the compiler so, and
  // readfirstlane keeps the LDS destinations in scalar registers
  static_assert((KW & (KW - 1)) == 0, "KW is a power of two");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & (KW - 1);
  const uint32_t row_bytes = (uint32_t)p.n_heads * D * 2;
  const auto rs = tile_rsrc((const uint16_t*)t.k + ((int64_t)t.key0 * p.n_heads + head) * D,
                            (uint32_t)t.n_valid * row_bytes);
#pragma unroll
  for (int j = 0; j < Loader<D, ST>::KMAX; ++j) {
    const int blk = wave + KW * j;
    if (blk < L::K_BLKS)
      buffer_to_lds16(rs, kdst + blk * 64 * 8, pl.k_off[j]);
  }
}

template <int D, int ST>
__device__ __forceinline__ void issue_kdma(const AttnParams& p, const TileRef& t, int head, Smem<D>& sm, int kbuf,
                                           const LoadPlan<D, ST>& pl) {
  issue_kdma_to<D, ST>(p, t, head, sm.k[kbuf], pl);
}

// Register-staged loads of tile t, cut into NPART one-instruction parts so
// that they can ride on a wave's matrix work (a burst from every wave queues
// in the CU's address unit). bf16 tiles: V chunks. int8 tiles: K codes, V
// codes, then the scales (commit_tile applies them; using them here would
// wait for the loads).
template <int D, int ST, bool SCALED>
__device__ __forceinline__ void issue_stage_part(const AttnParams& p, const TileRef& t, int head,
                                                 Stage<D, ST, SCALED>& st, const LoadPlan<D, ST>& pl, int j) {
  using L = Layout<D>;
  using LD = Loader<D, ST>;
  const int tid = threadIdx.x;
  const int64_t base = ((int64_t)t.key0 * p.n_heads + head) * D;
  static_assert(!SCALED || LD::I8CH == 1, "a staging thread moves one row's 16 K and 16 V codes");
  if (!SCALED || !t.is_int8) {
    if (j < LD::VCH) {
      // rows past the segment end read as zeros (their probabilities are 0)
      const auto rs = tile_rsrc((const uint16_t*)t.v + base, (uint32_t)t.n_valid * p.n_heads * D * 2);
      st.r[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, pl.v_off[j], 0, 0));
    }
  } else {
    if (j < 2 * LD::I8CH) {
      if (LD::I8_THREADS >= ST || tid < LD::I8_THREADS) {
        // zero codes past the segment end (their keys are masked, their P is 0)
        const auto rs = tile_rsrc((const int8_t*)(j < LD::I8CH ? t.k : t.v) + base, (uint32_t)t.n_valid * p.n_heads * D);
        st.r[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, pl.i8_off, 0, 0));
      }
    } else if (j == 2 * LD::I8CH) {
      if (tid < BK) st.ks = t.k_scale[(int64_t)(t.key0 + min(tid, t.n_valid - 1)) * p.n_heads + head];
      if (LD::I8_THREADS >= ST || tid < LD::I8_THREADS) {
        const int row = min(tid / (D / 16), t.n_valid - 1);   // this thread's V row
        st.vs = t.v_scale[(int64_t)(t.key0 + row) * p.n_heads + head];
      }
    }
  }
}

template <int D, int ST, bool SCALED>
__device__ __forceinline__ void issue_stage(const AttnParams& p, const TileRef& t, int head,
                                            Stage<D, ST, SCALED>& st, const LoadPlan<D, ST>& pl) {
#pragma unroll
  for (int j = 0; j < Loader<D, ST>::template npart<SCALED>(); ++j)
    issue_stage_part<D, ST, SCALED>(p, t, head, st, pl, j);
}

// Largest magnitude of this thread's staged share of a tile: max |v| of a
// bf16 tile's V chunks, or the V scale of an int8 tile's row (0 for threads
// that stage nothing of it).
template <int D, int ST, bool SCALED>
__device__ __forceinline__ float staged_magnitude(const TileRef& t, const Stage<D, ST, SCALED>& st) {
  using LD = Loader<D, ST>;
  float m = 0.f;
  if (!SCALED || !t.is_int8) {
#pragma unroll
    for (int j = 0; j < LD::VCH; ++j) m = absmax_bf16x8(st.r[j], m);
  } else if (LD::I8_THREADS >= ST || (int)threadIdx.x < LD::I8_THREADS) {
    m = st.vs;
  }
  return m;
}

// The bf16 V chunks of a staged tile into LDS buffer vdst, times 2^e.
template <int D, int ST, bool SCALED>
__device__ __forceinline__ void store_v_bf16(const Stage<D, ST, SCALED>& st, uint16_t* vdst, int e) {
  using L = Layout<D>;
  using LD = Loader<D, ST>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < LD::VCH; ++j) {
    const int lin = tid + j * ST;
    const int row = lin / L::CPR, c = lin % L::CPR;
    *reinterpret_cast<uint4*>(vdst + row * L::VS + c * 8) =
        e == 0 ? bf16x8_to_f16x8(st.r[j]) : bf16x8_to_f16x8_exp(st.r[j], e);
  }
}

// Finish tile t: register-staged V (and int8 K) into LDS buffers vbuf (kbuf),
// scaled-path multipliers into slot kbuf; V times 2^e (see v_exponent).
// min_scale keeps the smallest positive int8 V row scale committed.
template <int D, int ST, bool SCALED>
__device__ __forceinline__ void commit_tile(const AttnParams& p, const TileRef& t, const Stage<D, ST, SCALED>& st,
                                            Smem<D>& sm, int kbuf, int vbuf, int e, float& min_scale) {
  using L = Layout<D>;
  using LD = Loader<D, ST>;
  const int tid = threadIdx.x;
  if (!SCALED || !t.is_int8) {
    store_v_bf16<D, ST, SCALED>(st, sm.v[vbuf], e);
  } else if (LD::I8_THREADS >= ST || tid < LD::I8_THREADS) {
#pragma unroll
    for (int j = 0; j < LD::I8CH; ++j) {
      const int lin = tid + j * ST;
      const int row = lin / (D / 16), c16 = lin % (D / 16);
      uint16_t* kr = sm.k[kbuf] + row * L::KS + 16 * c16;
      uint16_t* vr = sm.v[vbuf] + row * L::VS + 16 * c16;
      const uint4 kc = st.r[j], vc = st.r[LD::I8CH + j];
      *reinterpret_cast<uint4*>(kr) = i8x8_to_bf16x8(kc.x, kc.y);
      *reinterpret_cast<uint4*>(kr + 8) = i8x8_to_bf16x8(kc.z, kc.w);
      // V 2^e = code * scale 2^e in fp16: the exact fp16 code times the row's
      // scale 2^e (exact in fp32) rounded to fp16, one rounding of the product
      const _Float16 sv = (_Float16)ldexpf(st.vs, e);
      min_scale = fminf(min_scale, st.vs > 0.f ? st.vs : INFINITY);
      const f16x2 sv2 = {sv, sv};
      *reinterpret_cast<uint4*>(vr) = scale_f16x8(i8x8_to_f16x8(vc.x, vc.y), sv2);
      *reinterpret_cast<uint4*>(vr + 8) = scale_f16x8(i8x8_to_f16x8(vc.z, vc.w), sv2);
    }
  }
  if (SCALED && tid < BK) {
    // per-key multipliers of the raw score (log2 units); keys past the segment
    // end keep a positive multiplier so that their bias stays -1e30
    const bool ok = tid < t.n_valid;
    sm.ksc[kbuf][tid] = (t.is_int8 && ok) ? fmaxf(st.ks * p.scale_log2, KSC_MIN) : p.scale_log2;
  }
}

__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// x[n] *= (a of lane n of the caller's 16-lane row), n = N..15: a DPP row
// broadcast folded into each multiply (v_mul_f32_dpp row_newbcast:n).
template <int N>
__device__ __forceinline__ void scale_by_row_lanes(f32x16& x, float a) {
  if constexpr (N < 16) {
    x[N] *= __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x150 + N, 0xF, 0xF, true));
    scale_by_row_lanes<N + 1>(x, a);
  }
}

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
  int e_o;             // o holds O * 2^e_o (the V exponent of the tiles last multiplied)
};

// S^T = K Q^T for the two 32-key subtiles of a 64-key tile, plus the masking
// bias, for one wave; int8 tiles of the scaled kernels multiplied per key.
// Returns the factor that brings s to log2 units. after_mfma(i) runs after
// the i-th of the 2*D/16 score MFMAs, after_scores() after the last one.
// Element e2 of subtile kt is key kt*32 + 8*(e2/4) + 4*hh + e2%4 of the tile.
template <int D, bool SCALED, bool GENERAL, typename Hook, typename Tail>
__device__ __forceinline__ float qk_scores(const AttnParams& p, const TileRef& t, WaveState<D>& ws,
                                           const uint16_t* kl, const float* ksc, int k_lane,
                                           int r, int hh, int my_qb, int qb_lo, f32x16 (&s)[2],
                                           Hook&& after_mfma, Tail&& after_scores) {
  using L = Layout<D>;
  constexpr int NKS = D / 16;
  // LDS operand reads in flight ahead of their MFMA (the scaled path needs the registers)
  constexpr int PF = SCALED ? 2 : 4;

  // int8 tiles of the scaled kernels: per-key multipliers applied to the raw
  // scores; every other tile: raw scores, scale_log2 folded into the
  // exponent's FMA. Every lane of a 16-lane row needs the same 16 multipliers
  // per subtile (its row lies in one lane half): lane n of the row reads the
  // one for element n (key kt*32 + 8(n/4) + 4hh + n%4) here, ahead of the
  // score MFMAs, and each multiply takes it by a DPP row broadcast; two
  // 4-byte LDS reads per lane instead of eight 16-byte ones.
  const bool per_key = SCALED && t.is_int8;
  float kmul[2] = {1.f, 1.f};
  if (SCALED) {
    const int n16 = r & 15;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) kmul[kt] = ksc[kt * 32 + 8 * (n16 >> 2) + 4 * hh + (n16 & 3)];
  }

  // ---- S^T = K Q^T for two 32-key subtiles; operand reads PF steps ahead,
  // scheduling fences keep the compiler from hoisting all of them. MFMA i
  // takes k-slice i/2 of subtile i%2: consecutive MFMAs feed different
  // accumulators (each subtile still sums its slices in order), which
  // measured 2-3% faster than finishing one subtile before the other.
  constexpr int NQK = 2 * NKS;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int e2 = 0; e2 < 16; ++e2) s[kt][e2] = 0.f;
  {
    bf16x8 ka[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i)
      ka[i] = *reinterpret_cast<const bf16x8*>(kl + k_lane + (i % 2) * 32 * L::KS + (i / 2) * 16);
    // the score and P.V MFMA sequences run at raised wave priority (the
    // SIMD's arbiter then favours the wave issuing matrix work; measured with
    // a settled clock: 0.3-0.7% faster on every workload)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const bf16x8 a = ka[i % PF];
      if (i + PF < NQK)
        ka[i % PF] = *reinterpret_cast<const bf16x8*>(kl + k_lane + ((i + PF) % 2) * 32 * L::KS +
                                                      ((i + PF) / 2) * 16);
      s[i % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ws.qf[i / 2], s[i % 2], 0, 0, 0);
      after_mfma(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  after_scores();

  // ---- masking bias: one extra k-step. Lane (key, hh) supplies A[key][slot]
  // for slots 8*hh .. 8*hh+7 (slot = q-block inside the workgroup's rows)
  if (GENERAL || t.n_valid < BK) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = kt * 32 + r;
      const bool kvalid = key < t.n_valid;
      bf16x8 a;
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] = (__bf16)0.0f;
      if (GENERAL) {
        // this key's k-block inside the tile, and the keep bits of its q-blocks
        const int jk = ((t.key0 + key) >> p.block_k_log2) - (t.key0 >> p.block_k_log2);
        const uint32_t qkeep = kvalid ? (uint32_t)(t.kbits >> (16 * jk)) >> (8 * hh) : 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] = ((qkeep >> j) & 1u) ? (__bf16)0.0f : (__bf16)MASK_BIAS;
      } else if (hh == 0) {
        a[0] = kvalid ? (__bf16)0.0f : (__bf16)MASK_BIAS;
      }
      s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ws.qsel, s[kt], 0, 0, 0);
    }
    if (GENERAL) {
      // does any kept key of this tile reach this lane's query row?
      ws.seen |= (t.kbits & (0x0001000100010001ull << (my_qb - qb_lo))) != 0;
    }
  }

  if (per_key) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) scale_by_row_lanes<0>(s[kt], kmul[kt]);
  }
  return per_key ? 1.0f : p.scale_log2;
}

// Group kk (0..3) of a tile's scores: subtile kk/2, elements 8(kk%2)..+7,
// which are P^T B-operand kk of the P.V MFMAs.
__device__ __forceinline__ float score_of(const f32x16 (&s)[2], int kk, int j) { return s[kk >> 1][8 * (kk & 1) + j]; }

// P of group kk in fp16 and the sum of those fp16 values into lt (pairs in
// order, fp32 accumulation)
__device__ __forceinline__ f16x8 pack_group(const float (&f)[8], float& lt) {
  f16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (_Float16)f[j];
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
  for (int j = 0; j < 8; j += 2) lt = __builtin_amdgcn_fdot2(f16x2{v[j], v[j + 1]}, ones, lt, false);
  return v;
}

// P = 2^(s cs - m) for a whole tile into pb; lt = sum of this lane's P,
// accumulated in NACC independent partial sums (group kk into sum kk % NACC,
// added pairwise at the end): one chain of 16 dependent dot products would
// hold the softmax up on its latency.
template <int NACC>
__device__ __forceinline__ void exp_tile(const f32x16 (&s)[2], float cs, float m, f16x8 (&pb)[4], float& lt) {
  static_assert(NACC == 2 || NACC == 4, "two or four partial sums");
  float part[NACC];
#pragma unroll
  for (int a = 0; a < NACC; ++a) part[a] = 0.f;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    float f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = __builtin_amdgcn_exp2f(fmaf(score_of(s, kk, j), cs, -m));
    pb[kk] = pack_group(f, part[kk % NACC]);
  }
  if constexpr (NACC == 4)
    lt = (part[0] + part[1]) + (part[2] + part[3]);
  else
    lt = part[0] + part[1];
}
// Partial sums of a tile's P per kernel kind, the faster count of each as
// measured: two in the kernels with int8 segments, four in the others.
template <bool SCALED>
constexpr int kSumParts = SCALED ? 2 : 4;

// Online softmax with a lazy running max: O and l are only rescaled when a
// row's max grows by more than 2^TAU, so P stays <= 2^TAU. The exponentials
// are taken first with the running max as it stands; a lane whose P sum
// stays below 2^TAU has every P below it, so no row max is needed then. Only
// when some lane reaches it (or a row has seen nothing yet) does the wave
// take the tile's row max; if a row max has grown past the threshold, O and
// l are rescaled and the exponentials taken again. The same rare branch
// brings o to the tile's V exponent e (exact power-of-two rescale). Runs
// after every earlier tile's P.V has reached o.
template <int D, bool EXACT, int NACC>
__device__ __forceinline__ void settle_tile(WaveState<D>& ws, const f32x16 (&s)[2], float cs, f16x8 (&pb)[4],
                                            float lt, int e) {
  constexpr int NDT = D / 32;
  static_assert(TAU == 8.0f, "threshold below is 2^TAU");
  const bool suspect = ws.m_run == -INFINITY || !(lt < 0x1p8f);
  if (__ballot(suspect) || (EXACT && e != ws.e_o)) {
    float mt = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e2 = 0; e2 < 16; e2 += 2) mt = max3(mt, s[kt][e2], s[kt][e2 + 1]);
    mt = swap_halves_max(mt) * cs;
    if (mt < MASKED_MAX) mt = -INFINITY;   // nothing visible for this row in the tile
    const bool need = mt > ws.m_run + TAU;
    const bool grow = __ballot(need) != 0;
    if (grow || (EXACT && e != ws.e_o)) {
      const float m_new = need ? mt : ws.m_run;
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(ws.m_run - m_new);
      ws.m_run = m_new;
      ws.l_run *= alpha;
      const int sh = EXACT ? e - ws.e_o : 0;
      ws.e_o = EXACT ? e : ws.e_o;
      if (sh == 0) {
#pragma unroll
        for (int i = 0; i < NDT; ++i)
#pragma unroll
          for (int e2 = 0; e2 < 16; ++e2) ws.o[i][e2] *= alpha;
      } else {
#pragma unroll
        for (int i = 0; i < NDT; ++i)
#pragma unroll
          for (int e2 = 0; e2 < 16; ++e2) ws.o[i][e2] = ldexpf(ws.o[i][e2] * alpha, sh);
      }
    }
    if (grow) exp_tile<NACC>(s, cs, (ws.m_run == -INFINITY) ? 0.f : ws.m_run, pb, lt);
  }
  ws.l_run += lt;
}

// A whole tile for one wave: scores, then the softmax (P^T left in pb).
template <int D, bool SCALED, bool GENERAL, bool EXACT, typename Hook, typename Tail>
__device__ __forceinline__ void qk_softmax(const AttnParams& p, const TileRef& t, WaveState<D>& ws,
                                           const uint16_t* kl, const float* ksc, int k_lane,
                                           int r, int hh, int my_qb, int qb_lo, f16x8 (&pb)[4],
                                           int e, Hook&& after_mfma, Tail&& after_scores) {
  f32x16 s[2];
  const float cs = qk_scores<D, SCALED, GENERAL>(p, t, ws, kl, ksc, k_lane, r, hh, my_qb, qb_lo, s, after_mfma,
                                                 after_scores);
  float lt;
  exp_tile<kSumParts<SCALED>>(s, cs, (ws.m_run == -INFINITY) ? 0.f : ws.m_run, pb, lt);
  settle_tile<D, EXACT, kSumParts<SCALED>>(ws, s, cs, pb, lt, e);
}

// Second half of a tile: O^T += V^T P^T (transposed reads of the row-major
// fp16 V tile, which holds V * 2^e; the tile's settle_tile has brought o to
// the same exponent). MFMA i multiplies key group kk = i / NDT into column
// tile dt = i % NDT.
template <int D, int PF>
__device__ __forceinline__ void pv_tile(WaveState<D>& ws, const uint16_t* vl, int v_lane, const f16x8 (&pb)[4]) {
  constexpr int NDT = D / 32;
  constexpr int NPV = 4 * NDT;
  f16x8 va[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) va[i] = read_vt<D>(vl, v_lane, i % NDT, i / NDT);
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int i = 0; i < NPV; ++i) {
    const f16x8 a = va[i % PF];
    if (i + PF < NPV) va[i % PF] = read_vt<D>(vl, v_lane, (i + PF) % NDT, (i + PF) / NDT);
    ws.o[i % NDT] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[i / NDT], ws.o[i % NDT], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
}

// Scaled kernels, leading waves: the next tile's direct K loads, then scores,
// softmax and P.V of this tile. The LDS buffers come in as restrict-qualified
// pointers: the compiler then knows that the K and V reads do not touch the K
// buffer being filled and does not make them wait for those loads (with one
// shared buffer object it waited for the whole load before the first score
// MFMA).
template <int D, bool SCALED, bool GENERAL, bool EXACT, int ST, int PF, typename Ride>
__device__ __forceinline__ void lead_tile_scaled(const AttnParams& p, const TileRef& t, const TileRef& tn, int head,
                                                 WaveState<D>& ws, const uint16_t* __restrict__ kcur,
                                                 const float* __restrict__ ksc,
                                                 const uint16_t* __restrict__ vcur, uint16_t* __restrict__ knew,
                                                 bool dma, const LoadPlan<D, ST>& plan, int k_lane, int v_lane,
                                                 int r, int hh, int my_qb, int qb_lo, f16x8 (&pb)[4],
                                                 Ride&& ride, int e) {
  if (dma) issue_kdma_to<D, ST>(p, tn, head, knew, plan);
  qk_softmax<D, SCALED, GENERAL, EXACT>(p, t, ws, kcur, ksc, k_lane, r, hh, my_qb, qb_lo, pb, e, ride, [] {});
  pv_tile<D, PF>(ws, vcur, v_lane, pb);
}

// Query-block bits (relative to the workgroup's first q-block) that wave w's
// 32 rows touch; 0 for a wave whose rows all lie past n_q.
__device__ __forceinline__ uint32_t wave_qbits(const AttnParams& p, int q_lo, int qb_lo, int w) {
  const int r0 = q_lo + 32 * w;
  if (r0 >= p.n_q) return 0u;
  const int r1 = min(p.n_q, r0 + 32) - 1;
  const int b0 = r0 / p.block_q - qb_lo, b1 = r1 / p.block_q - qb_lo;
  return ((2u << b1) - 1u) & ~((1u << b0) - 1u);
}

// Exact V exponent of a staged tile (every wave calls it; one barrier): the
// largest magnitude over all staging threads' shares.
template <int D>
__device__ __forceinline__ int exact_v_exponent(Smem<D>& sm, float m, bool is_int8, int wave, int lane) {
  const float wm = wave_max(m);
  if (lane == 0) sm.vmax[wave] = wm;
  __syncthreads();
  float mm = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) mm = fmaxf(mm, sm.vmax[w]);
  mm = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mm)));
  return v_exponent(mm, is_int8);
}

template <int D, bool SCALED, bool GENERAL>
__global__ __launch_bounds__(NT, 1) void attn_fwd_kernel(AttnParams p) {
  using L = Layout<D>;
  __shared__ __attribute__((aligned(16))) Smem<D> sm;
  constexpr int NKS = D / 16;
  constexpr int NDT = D / 32;
  // V^T operand reads in flight ahead of their P.V MFMA (two measured 0.4-0.8%
  // faster than four once the score MFMAs alternate between subtiles)
  constexpr int PF_PV = 2;

  // ---- XCD-aware work mapping: each XCD takes a contiguous range of work
  // units (head, query tile), so the units on one XCD share its L2 for K/V.
  // Balanced launches: the XCD's last r units run as head pieces (candidate
  // tiles [0, split_tile)) and their tail pieces follow as workgroups
  // n .. n + r - 1 of the XCD, on the CUs that the head pieces leave free.
  const int xcd = blockIdx.x % NXCD, local = blockIdx.x / NXCD;
  const XcdUnits xu = xcd_units(p.n_qt * p.n_heads, xcd, p.cu_per_xcd, p.split_tile > 0);
  int item = xu.u0 + local, c_lo = 0, c_hi = p.n_tiles, slot = -1;
  if (local >= xu.n) {
    const int j = local - xu.n;
    if (j >= xu.r) return;   // padding of the grid
    item = xu.u0 + xu.n - xu.r + j;
    slot = (xcd * p.split_rmax + j) * 2 + 1;
    c_lo = p.split_tile;
  } else if (local >= xu.n - xu.r) {
    slot = (xcd * p.split_rmax + local - (xu.n - xu.r)) * 2;
    c_hi = p.split_tile;
  }
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
  // Waves NW/2.. run half a tile behind the others: they multiply the
  // previous tile's P with V first, so on every SIMD one wave's softmax
  // overlaps the other's matrix work.
  const bool lagging = wave >= NW / 2;

  // q-block range of this workgroup (mask lookups and bias slots)
  const int q_lo = qt * BQ;
  const int q_hi = min(p.n_q, q_lo + BQ) - 1;
  const int qb_lo = q_lo / p.block_q, qb_hi = q_hi / p.block_q;
  const int my_qb = min(q_row, p.n_q - 1) / p.block_q;

  WaveState<D> ws;
  {
    const uint16_t* qp = p.q + ((int64_t)q_row * p.n_heads + head) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      uint4 w = q_ok ? *reinterpret_cast<const uint4*>(qp + ks * 16) : make_uint4(0, 0, 0, 0);
      ws.qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
    // bias selector: slot = the lane's q-block inside the workgroup (general
    // masks) or slot 0; slot s sits in lane half s/8, element s%8
    const int slot = GENERAL ? my_qb - qb_lo : 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) ws.qsel[j] = (8 * hh + j == slot) ? (__bf16)1.0f : (__bf16)0.0f;
  }
#pragma unroll
  for (int i = 0; i < NDT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) ws.o[i][e] = 0.f;
  ws.m_run = -INFINITY;
  ws.l_run = 0.f;
  ws.seen = !GENERAL;
  ws.e_o = 0;

  // per-lane LDS offsets (elements) that do not change over the loop
  const int k_lane = r * L::KS + 8 * hh;
  // transposed V read: row (4*hh + s16/4) of each 8-key group, 4 columns at
  // 16*(g16&1) + 4*(s16&3) inside each 32-column tile
  const int v_lane = (4 * hh + (s16 >> 2)) * L::VS + 16 * (g16 & 1) + 4 * (s16 & 3);

  constexpr int ST = SCALED ? NT : NT / 2;   // staging threads (see Loader)
  using LD = Loader<D, ST>;
  Stage<D, ST, SCALED> st;
  LoadPlan<D, ST> plan;
  make_plan<D, ST>(plan, (uint32_t)p.n_heads * D * 2);
  constexpr int NPART = LD::template npart<SCALED>();
  constexpr int STRIDE = (2 * NKS) / NPART;
  const bool k_wave = wave < LD::KW;
  const bool stager = tid < ST;
  // q-block bits of every wave of the workgroup (tile compaction)
  uint32_t wq[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) wq[w] = wave_qbits(p, q_lo, qb_lo, w);

  // Every pass over the kept tiles, in one of two forms. The fast form
  // stages every V tile as it is (exponent 0); it is exact while each int8
  // row scale is 0 or a normal fp16 (>= 2^-14) and every staged value is
  // finite, and otherwise off by at most 2^-25 per bf16 element (values below
  // 2^-17, where fp16 has fewer bits). The exact form settles every tile's V
  // exponent from its largest magnitude before the tile is committed (one
  // more barrier per tile). The workgroup runs the fast form, checks its
  // result (below), and runs the exact form from the start only when the
  // check fails.
  // fast form: smallest positive int8 row scale this thread staged (a float,
  // not a flag: a per-lane flag would live in scalar registers the loop needs)
  float i8_min_scale = INFINITY;
  auto all_passes = [&](auto exact_tag) {
    constexpr bool EXACT = decltype(exact_tag)::value;
#pragma unroll 1
  for (int cbase = c_lo; cbase < c_hi; cbase += LIST_CAP) {
    // ---- compact the kept tiles of this pass into sm.list (order preserved),
    // with the set of waves that have a kept (q-block, k-block) pair in each
    const int ncand = min(LIST_CAP, c_hi - cbase);
    uint32_t wmk[2];
    uint64_t kbt[2];
    TileInfo ti[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = 2 * tid + i;
      wmk[i] = 0;
      kbt[i] = 0;
      if (c < ncand) {
        const TileInfo t = tile_info(p, cbase + c);
        ti[i] = t;
        const AttnSegment& sg = p.seg[t.seg];
        const int kb_lo = sg.kb_start + (t.key0 >> p.block_k_log2);
        const int kb_hi = sg.kb_start + ((t.key0 + t.n_valid - 1) >> p.block_k_log2);
        uint32_t qbits = 0;
        for (int qb = qb_lo; qb <= qb_hi; ++qb) {
          bool any = false;
          if (GENERAL) {
            for (int kb = kb_lo; kb <= kb_hi; ++kb)
              if (p.mask[(int64_t)qb * p.n_kb + kb] != 0) {
                any = true;
                kbt[i] |= 1ull << (16 * (kb - kb_lo) + (qb - qb_lo));
              }
          } else {
            for (int kb = kb_lo; kb <= kb_hi && !any; ++kb) any = p.mask[(int64_t)qb * p.n_kb + kb] != 0;
          }
          if (any) qbits |= 1u << (qb - qb_lo);
        }
#pragma unroll
        for (int w = 0; w < NW; ++w) wmk[i] |= (qbits & wq[w]) ? (1u << w) : 0u;
      }
    }
    const uint64_t b0 = __ballot(wmk[0] != 0);
    const uint64_t b1 = __ballot(wmk[1] != 0);
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
      if (wmk[0]) {
        if (GENERAL) sm.kbits[pos] = kbt[0];
        sm.desc[pos++] = pack_desc(ti[0], wmk[0]);
      }
      if (wmk[1]) {
        if (GENERAL) sm.kbits[pos] = kbt[1];
        sm.desc[pos] = pack_desc(ti[1], wmk[1]);
      }
    }
    __syncthreads();
    if (total == 0) continue;

    if constexpr (kSingleStage) {
      // ---- single-stage schedule (test-only build): V buffer 0, K buffers
      // alternating (one fixed K buffer trips the compiler's address-space
      // handling of the direct-to-LDS loads)
#pragma unroll 1
      for (int it = 0; it < total; ++it) {
        const TileRef t = tile_at<D, GENERAL>(p, sm, it);
        const bool direct_k = k_wave && !(SCALED && t.is_int8);
        if (direct_k) issue_kdma<D, ST>(p, t, head, sm, it & 1, plan);
        if (stager) issue_stage<D, ST, SCALED>(p, t, head, st, plan);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        int e = 0;
        if (EXACT) e = exact_v_exponent(sm, stager ? staged_magnitude<D, ST, SCALED>(t, st) : 0.f, t.is_int8, wave, lane);
        if (stager) commit_tile<D, ST, SCALED>(p, t, st, sm, it & 1, 0, e, i8_min_scale);
        __syncthreads();
        if ((t.wmask >> wave) & 1) {
          f16x8 pb[4];
          qk_softmax<D, SCALED, GENERAL, EXACT>(p, t, ws, sm.k[it & 1], sm.ksc[it & 1], k_lane, r, hh, my_qb, qb_lo,
                                                pb, e, [](int) {}, [] {});
          pv_tile<D, PF_PV>(ws, sm.v[0], v_lane, pb);
        }
        __syncthreads();
      }
    } else if constexpr (!SCALED) {
      // ---- unscaled kernels: every tile moves one step ahead. Tile i lives
      // in K buffer i%2 and V buffer i%3. During step i every wave's V loads
      // of tile i+1 ride on its score MFMAs, and the leading waves' direct K
      // loads follow their last score MFMA (the compiler waits for every LDS
      // read in flight after one of those, which inside the MFMA sequence
      // drained the operand prefetch); V is converted and stored at the end
      // of the step. Waves 4..7 run half a tile behind:
      // they multiply the previous tile's P with V first, then compute the
      // current tile's scores and softmax.
      TileRef tn = tile_at<D, GENERAL>(p, sm, 0);
      if (stager) {
        if (k_wave) issue_kdma<D, ST>(p, tn, head, sm, 0, plan);
        issue_stage<D, ST, SCALED>(p, tn, head, st, plan);
        commit_tile<D, ST, SCALED>(p, tn, st, sm, 0, 0, 0, i8_min_scale);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      f16x8 pb[4];
      bool pending = false;   // lagging waves: P of the previous tile awaits its P.V
      int kbuf = 0, vbuf = 0, vprev = NVBUF - 1;
#pragma unroll 1
      for (int it = 0; it < total; ++it) {
        const TileRef t = tn;
        const bool has_next = it + 1 < total;
        const int knext = kbuf ^ 1;
        const int vnext = (vbuf + 1 == NVBUF) ? 0 : vbuf + 1;
        if (has_next) tn = tile_at<D, GENERAL>(p, sm, it + 1);
        // exact form: tile it's V exponent from its largest magnitude; the
        // stagers, whose registers still hold its bf16 V, store it again
        // times 2^e when e is not 0
        int e_it = 0;
        if constexpr (EXACT) {
          e_it = exact_v_exponent(sm, stager ? staged_magnitude<D, ST, SCALED>(t, st) : 0.f, false, wave, lane);
          if (e_it != 0) {
            if (stager) store_v_bf16<D, ST, SCALED>(st, sm.v[vbuf], e_it);
            __syncthreads();
          }
        }
        if (lagging && pending) pv_tile<D, PF_PV>(ws, sm.v[vprev], v_lane, pb);
        pending = false;
        if ((t.wmask >> wave) & 1) {
          qk_softmax<D, SCALED, GENERAL, EXACT>(
              p, t, ws, sm.k[kbuf], sm.ksc[kbuf], k_lane, r, hh, my_qb, qb_lo, pb, e_it,
              [&](int i) {
                if (stager && has_next && i % STRIDE == 0 && i / STRIDE < NPART)
                  issue_stage_part<D, ST, SCALED>(p, tn, head, st, plan, i / STRIDE);
              },
              [&]() {
                if (k_wave && has_next) issue_kdma<D, ST>(p, tn, head, sm, knext, plan);
              });
          if (lagging)
            pending = true;
          else
            pv_tile<D, PF_PV>(ws, sm.v[vbuf], v_lane, pb);
        } else if (has_next && stager) {
          if (k_wave) issue_kdma<D, ST>(p, tn, head, sm, knext, plan);
          issue_stage<D, ST, SCALED>(p, tn, head, st, plan);
        }
        if (has_next && stager) commit_tile<D, ST, SCALED>(p, tn, st, sm, knext, vnext, 0, i8_min_scale);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        vprev = vbuf;
        kbuf = knext;
        vbuf = vnext;
      }
      // the last tile's V buffer stays untouched until the next pass's barriers
      if (pending) pv_tile<D, PF_PV>(ws, sm.v[vprev], v_lane, pb);
    } else {
      // ---- scaled kernels. Prologue: first kept tile into K buffer 0 / V
      // buffer 0, the second one's staged loads into registers.
      TileRef tc = tile_at<D, GENERAL>(p, sm, 0);
      if (k_wave && !tc.is_int8) issue_kdma<D, ST>(p, tc, head, sm, 0, plan);
      issue_stage<D, ST, SCALED>(p, tc, head, st, plan);
      int e_cur = 0;
      if constexpr (EXACT) e_cur = exact_v_exponent(sm, staged_magnitude<D, ST, SCALED>(tc, st), tc.is_int8, wave, lane);
      commit_tile<D, ST, SCALED>(p, tc, st, sm, 0, 0, e_cur, i8_min_scale);
      TileRef tn1 = tc;
      if (total > 1) {
        tn1 = tile_at<D, GENERAL>(p, sm, 1);
        issue_stage<D, ST, SCALED>(p, tn1, head, st, plan);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();

      // Tile i lives in K buffer i%2 (and scale slot i%2) and V buffer i%3.
      // Step i: every wave commits its staged share of tile i+1 (loaded during
      // step i-1) and loads its share of tile i+2 into the freed registers; the
      // K waves also issue tile i+1's direct K loads. Waves 0..3 commit first,
      // then run scores + softmax and P.V of tile i (vector, matrix, vector,
      // matrix); waves 4..7 first multiply the previous tile's P with V, then
      // commit, then run scores + softmax of tile i, keeping P for the next
      // step (matrix, vector, matrix, vector), so on every SIMD the two waves
      // alternate between the matrix and the vector units. In the exact form
      // the V exponent of tile i+1 is settled at the top of step i (one
      // barrier), before anyone commits it.
      f16x8 pb[4];
      bool pending = false;   // lagging waves: P of the previous tile awaits its P.V
      int kbuf = 0, vbuf = 0, vprev = NVBUF - 1;
#pragma unroll 1
      for (int it = 0; it < total; ++it) {
        const TileRef t = tc;
        const bool has1 = it + 1 < total, has2 = it + 2 < total;
        const int knext = kbuf ^ 1;
        const int vnext = (vbuf + 1 == NVBUF) ? 0 : vbuf + 1;
        TileRef tn2 = tn1;
        if (has2) tn2 = tile_at<D, GENERAL>(p, sm, it + 2);
        int e_next = 0;
        if constexpr (EXACT) {
          if (has1) e_next = exact_v_exponent(sm, staged_magnitude<D, ST, SCALED>(tn1, st), tn1.is_int8, wave, lane);
        }
        const bool compute = (t.wmask >> wave) & 1;
        auto ride = [&](int i) {
          if (has2 && i % STRIDE == 0 && i / STRIDE < NPART)
            issue_stage_part<D, ST, SCALED>(p, tn2, head, st, plan, i / STRIDE);
        };
        auto none = [&]() {};
        if (!lagging) {
          const bool dma = has1 && k_wave && !tn1.is_int8;
          if (has1) commit_tile<D, ST, SCALED>(p, tn1, st, sm, knext, vnext, e_next, i8_min_scale);
          if (compute) {
            lead_tile_scaled<D, SCALED, GENERAL, EXACT, ST, PF_PV>(p, t, tn1, head, ws, sm.k[kbuf], sm.ksc[kbuf],
                                                                   sm.v[vbuf], sm.k[knext], dma, plan,
                                                                   k_lane, v_lane, r, hh, my_qb, qb_lo, pb,
                                                                   ride, e_cur);
          } else {
            if (dma) issue_kdma<D, ST>(p, tn1, head, sm, knext, plan);
            if (has2) issue_stage<D, ST, SCALED>(p, tn2, head, st, plan);
          }
        } else {
          if (pending) pv_tile<D, PF_PV>(ws, sm.v[vprev], v_lane, pb);
          pending = false;
          if (has1) commit_tile<D, ST, SCALED>(p, tn1, st, sm, knext, vnext, e_next, i8_min_scale);
          if (compute) {
            qk_softmax<D, SCALED, GENERAL, EXACT>(p, t, ws, sm.k[kbuf], sm.ksc[kbuf], k_lane, r, hh, my_qb,
                                                  qb_lo, pb, e_cur, ride, none);
            pending = true;
          } else if (has2) {
            issue_stage<D, ST, SCALED>(p, tn2, head, st, plan);
          }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        vprev = vbuf;
        kbuf = knext;
        vbuf = vnext;
        tc = tn1;
        tn1 = tn2;
        e_cur = e_next;
      }
      // the last tile's V buffer stays untouched until the next pass's barriers
      if (pending) pv_tile<D, PF_PV>(ws, sm.v[vprev], v_lane, pb);
    }
  }
  };

  all_passes(std::integral_constant<bool, false>());
  // ---- check of the fast form, per query row of this wave: its output
  // (o / l) must be finite and, where the row sees a key, reach 2^-12 in its
  // largest column (then the 2^-25 that a bf16 V element below 2^-17 may lose
  // in fp16 stays below 2^-13 of the row's largest output); no int8 row scale
  // may have been an fp16 subnormal. If any wave's check fails, the whole
  // workgroup runs again in the exact form.
  {
    float omax = 0.f;
#pragma unroll
    for (int i = 0; i < NDT; ++i)
#pragma unroll
      for (int e2 = 0; e2 < 16; ++e2) omax = fmaxf(omax, fabsf(ws.o[i][e2]));
    omax = swap_halves_max(omax);
    const float l_tot = swap_halves_sum(ws.l_run);
    const bool sees = ws.seen && l_tot > 0.f;
    float osum = 0.f;   // a sum keeps NaN and infinity, which fmaxf would drop
#pragma unroll
    for (int i = 0; i < NDT; ++i)
#pragma unroll
      for (int e2 = 0; e2 < 16; ++e2) osum += fabsf(ws.o[i][e2]);
    const bool o_finite = __builtin_isfinite(osum);
    const bool fail = i8_min_scale < 0x1p-14f || (q_ok && sees && (!o_finite || omax < 0x1p-12f * l_tot));
    const bool any_fail = __ballot(fail) != 0;
    if (lane == 0) sm.wave_count[wave] = any_fail ? 1 : 0;
    __syncthreads();
    int redo = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) redo |= sm.wave_count[w];
    __syncthreads();
    if (redo) {
#pragma unroll
      for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int e2 = 0; e2 < 16; ++e2) ws.o[i][e2] = 0.f;
      ws.m_run = -INFINITY;
      ws.l_run = 0.f;
      ws.seen = !GENERAL;
      ws.e_o = 0;
      all_passes(std::integral_constant<bool, true>());
    }
  }

  // ---- finalise
  const float l_tot = swap_halves_sum(ws.l_run);
  const bool any = ws.seen && l_tot > 0.f;
  const float inv = any ? 1.0f / l_tot : 0.f;
  // o holds O * 2^e_o: each o / l is scaled by 2^-e_o (exact)
  const int esh = -ws.e_o;
  // partial form and pieces of split units: normalised O in fp32, merged
  // later without another rounding
  float* const of32 = slot >= 0 ? p.ws_o + ((int64_t)slot * BQ + (q_row - q_lo)) * D
                                : (p.out_f32 != nullptr ? p.out_f32 + ((int64_t)q_row * p.n_heads + head) * D : nullptr);
  float* const lsep = slot >= 0 ? p.ws_lse + (int64_t)slot * BQ + (q_row - q_lo)
                                : (p.lse != nullptr ? p.lse + (int64_t)head * p.n_q + q_row : nullptr);
  if (q_ok && of32 != nullptr) {
    float* op = of32;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(op + dt * 32 + 8 * g + 4 * hh) =
            make_float4(any ? ldexpf(ws.o[dt][4 * g + 0] * inv, esh) : 0.0f, any ? ldexpf(ws.o[dt][4 * g + 1] * inv, esh) : 0.0f,
                        any ? ldexpf(ws.o[dt][4 * g + 2] * inv, esh) : 0.0f, any ? ldexpf(ws.o[dt][4 * g + 3] * inv, esh) : 0.0f);
  } else if (q_ok) {
    uint16_t* op = p.out + ((int64_t)q_row * p.n_heads + head) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = dt * 32 + 8 * g + 4 * hh;
        // rows without a visible key store +0 (o * 0 could give -0)
        const __bf16 v0 = (__bf16)(any ? ldexpf(ws.o[dt][4 * g + 0] * inv, esh) : 0.0f);
        const __bf16 v1 = (__bf16)(any ? ldexpf(ws.o[dt][4 * g + 1] * inv, esh) : 0.0f);
        const __bf16 v2 = (__bf16)(any ? ldexpf(ws.o[dt][4 * g + 2] * inv, esh) : 0.0f);
        const __bf16 v3 = (__bf16)(any ? ldexpf(ws.o[dt][4 * g + 3] * inv, esh) : 0.0f);
        const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, v0) | ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
        const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, v2) | ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
        *reinterpret_cast<uint2*>(op + d) = make_uint2(w0, w1);
      }
  }
  if (q_ok && lsep != nullptr && hh == 0) {
    const float ln2 = 0.69314718055994530942f;
    *lsep = any ? (ws.m_run + __log2f(l_tot)) * ln2 : -INFINITY;
  }
}

template <int D, bool SCALED, bool GENERAL>
hipError_t launch(const AttnParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, SCALED, GENERAL>), dim3((unsigned)p.grid), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnParams& p, hipStream_t stream) {
  bool scaled = false;
  for (int s = 0; s < p.n_segs; ++s) scaled |= p.seg[s].is_int8 && p.seg[s].len > 0;
  // A wave's 32 rows lie in one q-block when block_q >= 32, and a 64-key tile
  // in one k-block when block_k >= 64: then a wave either skips a tile or sees
  // all of its keys. Finer mask blocks need the per-q-block bias.
  const bool general = p.block_q < 32 || p.block_k < BK;
  if (scaled) return general ? launch<D, true, true>(p, stream) : launch<D, true, false>(p, stream);
  return general ? launch<D, false, true>(p, stream) : launch<D, false, false>(p, stream);
}

}  // namespace

hipError_t launch_attn_fwd(const AttnParams& p, int head_dim, hipStream_t stream) {
  if (p.n_q == 0) return hipSuccess;
  return head_dim == 128 ? launch_d<128>(p, stream) : launch_d<64>(p, stream);
}

}  // namespace sdit
