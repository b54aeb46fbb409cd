/*
 * sdit: attention core of a streaming video diffusion transformer, for
 * AMD Instinct MI355X (gfx950).
 *
 * For one chunk of latent-frame query tokens the library
 *   1. applies QK-RMSNorm and the 3D (t, h, w) rotary embedding to the
 *      chunk's q and k                       -> sdit_qknorm_rope3d
 *   2. optionally stores K/V as int8 with one fp32 scale per (token, head)
 *                                            -> sdit_kv_quant_int8
 *   3. runs block-masked softmax attention of the queries against a K/V
 *      cache made of ordered segments, e.g.
 *      [cached text | history chunks or reference image | current chunk]
 *                                            -> sdit_attn_fwd
 *
 * Conventions shared by every entry point
 *   - bf16 tensors are passed as raw 16-bit words (upper half of binary32).
 *   - Token-major layout [tokens][heads][head_dim], head_dim contiguous.
 *   - Every tensor pointer is DEVICE memory, except `segs` of sdit_attn_fwd,
 *     which is a HOST array. The caller allocates and frees everything; the
 *     library allocates nothing and keeps no per-call state.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work; nothing synchronises. A fault inside a kernel
 *     surfaces at the caller's next synchronisation.
 *   - Arguments are validated on the host before anything is launched. On
 *     a validation failure nothing is launched, the call returns a nonzero
 *     sdit_status and sdit_last_error() describes the problem (the message
 *     is per thread). Launch failures return SDIT_ERR_DEVICE; a device
 *     without a gfx950 code object returns SDIT_ERR_UNSUPPORTED.
 *   - Pointers to bf16/int8 tensors must be 16-byte aligned, fp32 arrays
 *     4-byte aligned.
 *   - Inputs must be finite. Only tiles that the block mask skips may hold
 *     non-finite values (they are never read).
 *   - No one tensor may hold more than 2^40 elements (tokens x heads x
 *     head_dim): larger requests return SDIT_ERR_INVALID. Size products are
 *     formed without integer overflow, so extreme 32-bit arguments are
 *     rejected, never wrapped into a small size.
 */
#ifndef SDIT_H
#define SDIT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDIT_ABI_VERSION 1
#define SDIT_MAX_SEGMENTS 8
#define SDIT_MAX_MERGE_PARTS 8

typedef enum sdit_status {
  SDIT_OK = 0,
  SDIT_ERR_INVALID = 1,     /* bad argument; nothing was launched            */
  SDIT_ERR_UNSUPPORTED = 2, /* valid request this library/device cannot run  */
  SDIT_ERR_DEVICE = 3       /* the HIP runtime reported an error at launch   */
} sdit_status;

typedef enum sdit_dtype {
  SDIT_BF16 = 0,
  SDIT_INT8 = 1
} sdit_dtype;

/* One K/V segment of the attention cache (host struct, device pointers).
 *   k, v      [len][n_heads][head_dim], bf16 words or int8 codes (dtype)
 *   k_scale,  [len][n_heads] fp32, int8 segments only (NULL for bf16);
 *   v_scale   the value of element c is code_c * scale.
 *   len       number of tokens (0 allowed: the segment is empty)
 *   dtype     sdit_dtype
 * Joy-face_change_optimized README, section 1, item 1: attention K/V is the
 * static text cache + the image cache + the current chunk; the int8 cache
 * bullet of the same section scales per token and head. */
typedef struct sdit_kv_segment {
  const void* k;
  const void* v;
  const float* k_scale;
  const float* v_scale;
  int32_t len;
  int32_t dtype;
} sdit_kv_segment;

int sdit_abi_version(void);
const char* sdit_status_string(int status);
const char* sdit_last_error(void);

/* QK-RMSNorm followed by the 3D rotary embedding, for the chunk's q and k.
 * ("QK-norm+3D RoPE" fused operator: Joy-face_change_optimized README,
 * table of changed files; cached text keys are stored after the qk-norm,
 * section 1, item 1.)
 *
 * For every token n and head h, over the head dimension d:
 *   y_c = x_c / sqrt(mean_c(x_c^2) + eps) * gamma_c      (gamma per tensor)
 * then the head dimension is cut into axis blocks t | h | w of widths
 * d_t, d_h, d_w (even, summing to head_dim); in an axis block of width d_a,
 * the interleaved pair (2j, 2j+1) is rotated by the angle
 *   p_a * theta^(-2j/d_a),
 * p_a being the token's position on that axis. Tokens are in (t, h, w)
 * row-major order, w fastest: n -> t = t0 + n/(Hl*Wl), h = (n/Wl) % Hl,
 * w = n % Wl. Arithmetic is fp64 with one rounding to bf16 at the end.
 *
 *   q_in, k_in     bf16 [T*Hl*Wl][n_heads][head_dim]
 *   q_out, k_out   bf16, same shape; may equal q_in / k_in (in place),
 *                  must not otherwise overlap any other tensor argument
 *   gamma_q/_k     fp32 [head_dim]
 *   head_dim       64 or 128
 *   theta > 0, eps >= 0, t0 >= 0; T, Hl or Wl == 0 is a no-op. */
int sdit_qknorm_rope3d(const void* q_in, const void* k_in, void* q_out, void* k_out,
                       const float* gamma_q, const float* gamma_k,
                       int32_t T, int32_t Hl, int32_t Wl, int32_t t0,
                       int32_t n_heads, int32_t head_dim,
                       int32_t d_t, int32_t d_h, int32_t d_w,
                       float theta, float eps, void* stream);

/* sdit_qknorm_rope3d of the chunk's q and k, together with the int8 cache
 * entries of the chunk (the per-(token, head) int8 K/V cache of the
 * Joy-face_change_optimized README, section 1, int8 K/V bullet, written for
 * later chunks while this one attends to its own bf16 k and v): one pass
 * that reads q_in, k_in and v_in once and writes
 *   q_out, k_out   as sdit_qknorm_rope3d (bit for bit),
 *   k_codes/_scales  sdit_kv_quant_int8 of k_out (from the rounded bf16
 *                  values, so the codes are exactly those of quantising
 *                  k_out afterwards, without reading it back),
 *   v_codes/_scales  sdit_kv_quant_int8 of v_in.
 *   v_in           bf16 [T*Hl*Wl][n_heads][head_dim], 16-byte aligned
 *   k_codes, v_codes  int8 [T*Hl*Wl][n_heads][head_dim], 16-byte aligned
 *   k_scales, v_scales  fp32 [T*Hl*Wl][n_heads], 4-byte aligned
 * Other arguments and rules as sdit_qknorm_rope3d; the codes and scales must
 * not overlap each other or any other argument, nor q_out/k_out v_in. */
int sdit_qknorm_rope3d_kv_quant_int8(const void* q_in, const void* k_in, const void* v_in,
                                     void* q_out, void* k_out,
                                     int8_t* k_codes, float* k_scales, int8_t* v_codes, float* v_scales,
                                     const float* gamma_q, const float* gamma_k,
                                     int32_t T, int32_t Hl, int32_t Wl, int32_t t0,
                                     int32_t n_heads, int32_t head_dim,
                                     int32_t d_t, int32_t d_h, int32_t d_w,
                                     float theta, float eps, void* stream);

/* Symmetric int8 quantisation of a K or V tensor, one fp32 scale per
 * (token, head) (Joy-face_change_optimized README, section 1, int8 K/V
 * bullet). Call once for K and once for V.
 *   amax   = max_c |x_c|
 *   scale  = amax / 127                      (IEEE binary32 division)
 *   code_c = clamp(rne(x_c / scale), -127, 127)
 *            (binary32 quotient, then round half to even)
 *   amax == 0 -> scale = 0 and all codes 0.
 *   x       bf16 [n_tok][n_heads][head_dim]
 *   codes   int8 [n_tok][n_heads][head_dim]
 *   scales  fp32 [n_tok][n_heads]
 *   head_dim 64 or 128; n_tok == 0 is a no-op. Outputs must not overlap x. */
int sdit_kv_quant_int8(const void* x, int8_t* codes, float* scales,
                       int32_t n_tok, int32_t n_heads, int32_t head_dim, void* stream);

/* Block-masked softmax attention of n_q queries over the concatenation of
 * the segments (Joy-face_change_optimized README, section 1, item 1;
 * block-causal chunks: Wave Forcing summary; block-sparse attention with a
 * (q-block, k-block) mask that, when dense, equals ordinary
 * scaled-dot-product attention: FlashVSR deployment notes,
 * Block-Sparse-Attention section).
 *
 *   q            bf16 [n_q][n_heads][head_dim] (after sdit_qknorm_rope3d)
 *   segs         HOST array of n_segs segments, 1 <= n_segs <= 8
 *   block_mask   uint8 [ceil(n_q/block_q)][sum_s ceil(len_s/block_k)],
 *                row-major, nonzero = keep. Query i is in row i/block_q.
 *                k-blocks restart at every segment: key j of segment s is in
 *                column sum_{s'<s} ceil(len_s'/block_k) + j/block_k, so a
 *                block never straddles two segments; last blocks may be
 *                partial.
 *   block_q, block_k   16, 32, 64 or 128
 *   head_dim     64 or 128
 *   softmax_scale  <= 0 selects 1/sqrt(head_dim); a positive scale below
 *                2^-40 is rejected (SDIT_ERR_INVALID): masking adds a -1e30
 *                bias to a key's raw score, which has to stay far below every
 *                visible score once scaled
 *   out          bf16 [n_q][n_heads][head_dim]
 *   lse          fp32 [n_heads][n_q] natural-log sum of exponentials of the
 *                scaled scores, or NULL
 * For query i with visible keys V(i) = {j : mask[qb(i)][kb(j)] != 0}:
 *   s_j = scale * q_i . k_j,  o_i = sum_j softmax(s)_j v_j,  lse_i = log sum_j e^{s_j};
 * a query with no visible key gets o_i = 0 and lse_i = -inf.
 * Scores accumulate in fp32 from bf16 q.k products; the probability-weighted
 * sum of V multiplies fp16 probabilities with V staged in fp16, accumulating
 * in fp32. Any finite V is accepted: where fp16 would not hold a 64-key tile
 * of V (bf16 values below 2^-17 or at 65536 and above, int8 row scales below
 * 2^-14), the tile is staged times a power of two chosen from its largest
 * magnitude and the accumulators are rescaled exactly (a workgroup whose
 * result shows such data runs again in that form). int8 K row scales below
 * about 1e-11 are out of contract (the score multiplier is floored).
 * Output must not overlap any input. */
int sdit_attn_fwd(const void* q, int32_t n_q,
                  const sdit_kv_segment* segs, int32_t n_segs,
                  const uint8_t* block_mask, int32_t block_q, int32_t block_k,
                  int32_t n_heads, int32_t head_dim, float softmax_scale,
                  void* out, float* lse, void* stream);

/* sdit_attn_fwd with the grid's last partial wave balanced over the CUs.
 * Same computation and arguments as sdit_attn_fwd (so the same passages),
 * plus a caller-owned device workspace. Work units (head, 256 query rows)
 * are dealt to the 8 XCDs in contiguous ranges; on an XCD whose units do not
 * fill whole waves of its CUs, the units of the last partial wave are cut at
 * one key tile into a head piece and a tail piece, which run on the CUs
 * that the partial wave would leave idle, and a second kernel combines the
 * two pieces' normalised fp32 partials with the log-sum-exp identity of
 * sdit_attn_merge (so outputs may differ from sdit_attn_fwd in the last
 * bf16 bit). Head pieces all start at the first key tile, so the units on an
 * XCD still walk the keys together and share its L2.
 *   workspace        device memory, 16-byte aligned, at least
 *                    SDIT_ATTN_WORKSPACE_BYTES(head_dim) bytes, not
 *                    overlapping any argument; its contents on entry do not
 *                    matter and are undefined after the call. Calls that
 *                    share a workspace must be ordered on one stream.
 *   workspace_bytes  its size
 *   split_tile       -1: the library plans the cut from the shape and the
 *                    device's CU count (no cut when it would not pay);
 *                    0: never cut (then this is sdit_attn_fwd);
 *                    t >= 1: cut at key tile t (64-key tiles counted over the
 *                    concatenated segments, t < their total), for tests. */
#define SDIT_ATTN_WORKSPACE_BYTES(head_dim) ((int64_t)8 * 31 * 2 * 256 * ((head_dim) + 1) * 4)
/* The cut sdit_attn_fwd_balanced makes (host only, nothing launched): for
 * n_q queries, n_heads heads and n_tiles 64-key tiles over the segments on
 * a device of n_cus CUs, *tile receives the key tile of the cut (0: none)
 * and *grid the workgroups of the attention launch. split_tile as above. */
int sdit_attn_balanced_plan(int32_t n_q, int32_t n_heads, int32_t n_tiles, int32_t n_cus,
                            int32_t split_tile, int32_t* tile, int32_t* grid);
int sdit_attn_fwd_balanced(const void* q, int32_t n_q,
                           const sdit_kv_segment* segs, int32_t n_segs,
                           const uint8_t* block_mask, int32_t block_q, int32_t block_k,
                           int32_t n_heads, int32_t head_dim, float softmax_scale,
                           void* out, float* lse, void* workspace, int64_t workspace_bytes,
                           int32_t split_tile, void* stream);

/* sdit_attn_fwd_balanced for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same computation, arguments and plan as sdit_attn_fwd_balanced
 * without the workspace: the pieces' partials go to a device array the
 * library owns, SDIT_STATIC_SCRATCH_BYTES (64 MiB) per GPU, held from the
 * library's first use on that GPU until the process ends. That covers the
 * largest plan at head_dim 128; a plan that needed more would be rejected
 * with SDIT_ERR_INVALID before anything is launched. The call allocates
 * nothing and calls no allocating routine. Every call on one GPU shares that
 * GPU's array: calls that overlap in time on one GPU (different streams, or
 * graph replays running concurrently) race and must be ordered by the
 * caller. Nothing in the array has to start at any value (each call writes
 * every entry it later reads). */
#define SDIT_STATIC_SCRATCH_BYTES ((int64_t)64 << 20)
int sdit_attn_fwd_balanced_static(const void* q, int32_t n_q,
                                  const sdit_kv_segment* segs, int32_t n_segs,
                                  const uint8_t* block_mask, int32_t block_q, int32_t block_k,
                                  int32_t n_heads, int32_t head_dim, float softmax_scale,
                                  void* out, float* lse, int32_t split_tile, void* stream);

/* Partial attention for a split of the keys (split-KV): the computation of
 * sdit_attn_fwd over the given segments, with O written normalised in fp32
 * so that results over disjoint key sets combine without another rounding
 * in sdit_attn_merge. Context-parallel attention of the Ulysses / Ring kind
 * (which the Wave Forcing summary compares Wave Parallelism against) attends
 * to one key shard per step and merges the shards this way.
 *   Arguments as sdit_attn_fwd, except
 *   out   fp32 [n_q][n_heads][head_dim], 16-byte aligned
 *   lse   fp32 [n_heads][n_q], required (the merge needs it)
 * A query with no visible key gets o = 0 and lse = -inf. The block mask
 * covers only the given segments (its columns restart with them). */
int sdit_attn_fwd_partial(const void* q, int32_t n_q,
                          const sdit_kv_segment* segs, int32_t n_segs,
                          const uint8_t* block_mask, int32_t block_q, int32_t block_k,
                          int32_t n_heads, int32_t head_dim, float softmax_scale,
                          float* out, float* lse, void* stream);

/* Merge of attention results over disjoint key sets (same passage as
 * sdit_attn_fwd_partial). Per query and head, with m = max_p lse_p and
 * w_p = e^(lse_p - m):
 *   out = sum_p w_p o_p / sum_p w_p   (bf16, rounded once)
 *   lse_out = m + log sum_p w_p
 * A part with lse = -inf adds nothing; a query with lse = -inf in every part
 * gets out = 0 and lse_out = -inf.
 *   o_parts     HOST array of n_parts device pointers, fp32
 *               [n_q][n_heads][head_dim], 16-byte aligned
 *   lse_parts   HOST array of n_parts device pointers, fp32 [n_heads][n_q]
 *   n_parts     1 .. SDIT_MAX_MERGE_PARTS
 *   out         bf16 [n_q][n_heads][head_dim]; must not overlap any input
 *   lse_out     fp32 [n_heads][n_q] or NULL
 *   head_dim    64 or 128 */
int sdit_attn_merge(const float* const* o_parts, const float* const* lse_parts, int32_t n_parts,
                    int32_t n_q, int32_t n_heads, int32_t head_dim,
                    void* out, float* lse_out, void* stream);

/* Token reordering for windowed sparse attention (FlashVSR deployment
 * notes, spatial tiling section: one attention block is a window of 8 x 8
 * tokens, and local_range counts such blocks). Tokens of a clip of T frames
 * of Hl x Wl tokens move between raster order (t, h, w) and window-major
 * order (t, h / window, w / window, h % window, w % window), so that every
 * window x window consecutive tokens form one spatial window (a block of
 * sdit_attn_fwd with block size window^2).
 *   x, y       bf16 [T*Hl*Wl][n_heads][head_dim]; must not overlap
 *   inverse    0: x raster -> y window-major; 1: x window-major -> y raster
 *   window     2, 4, 8 or 16; Hl and Wl multiples of it
 *   head_dim   64 or 128; T, Hl or Wl == 0 is a no-op
 *   T*Hl*Wl    below 2^30; n_heads * head_dim at most 2^24 (else
 *              SDIT_ERR_UNSUPPORTED). */
int sdit_window_permute(const void* x, void* y, int32_t T, int32_t Hl, int32_t Wl,
                        int32_t n_heads, int32_t head_dim, int32_t window, int32_t inverse, void* stream);

/* Per-token normalisations of the DiT block over the hidden dimension
 * (Joy-face_change_optimized README, table of changed files: RMSNorm and
 * LayerNorm + modulate are fused kernels beside QK-norm + 3D RoPE; the pages
 * give no formulas, so these are the usual definitions). Arithmetic in fp64,
 * one rounding to bf16 per output.
 *   sdit_rmsnorm:            y = x / sqrt(mean(x^2) + eps) * gamma
 *   sdit_layernorm_modulate: y = (x - mean) / sqrt(var + eps) * (1 + scale) + shift
 *                            (population variance; no affine parameters of its own)
 *   x, y          bf16 [n_tok][dim]; y == x (in place) is allowed, any other
 *                 overlap is rejected; 16-byte aligned
 *   gamma, scale, shift  fp32 [dim], shared by every token; 16-byte aligned
 *   dim           multiple of 8, 8 .. SDIT_MAX_NORM_DIM
 *   n_tok         0 .. 2^26 - 1; 0 is a no-op
 *   eps           0 <= eps <= 1
 * The library keeps no pointer past the call; nothing is allocated. */
#define SDIT_MAX_NORM_DIM 8192
int sdit_rmsnorm(const void* x, void* y, const float* gamma, int64_t n_tok, int32_t dim, float eps,
                 void* stream);
int sdit_layernorm_modulate(const void* x, void* y, const float* scale, const float* shift,
                            int64_t n_tok, int32_t dim, float eps, void* stream);

/* Host-only validators: the exact checks the entry points run before a
 * launch, without touching any device. They return SDIT_OK or the status
 * the entry point would return, and set sdit_last_error() likewise. */
int sdit_validate_qknorm_rope3d_args(const void* q_in, const void* k_in, void* q_out, void* k_out,
                                     const float* gamma_q, const float* gamma_k,
                                     int32_t T, int32_t Hl, int32_t Wl, int32_t t0,
                                     int32_t n_heads, int32_t head_dim,
                                     int32_t d_t, int32_t d_h, int32_t d_w,
                                     float theta, float eps);
int sdit_validate_qknorm_rope3d_kv_quant_int8_args(const void* q_in, const void* k_in, const void* v_in,
                                                   void* q_out, void* k_out, const int8_t* k_codes,
                                                   const float* k_scales, const int8_t* v_codes,
                                                   const float* v_scales, const float* gamma_q,
                                                   const float* gamma_k, int32_t T, int32_t Hl, int32_t Wl,
                                                   int32_t t0, int32_t n_heads, int32_t head_dim,
                                                   int32_t d_t, int32_t d_h, int32_t d_w, float theta, float eps);
int sdit_validate_kv_quant_args(const void* x, const int8_t* codes, const float* scales,
                                int32_t n_tok, int32_t n_heads, int32_t head_dim);
int sdit_validate_attn_args(const void* q, int32_t n_q,
                            const sdit_kv_segment* segs, int32_t n_segs,
                            const uint8_t* block_mask, int32_t block_q, int32_t block_k,
                            int32_t n_heads, int32_t head_dim, float softmax_scale,
                            const void* out, const float* lse);
int sdit_validate_attn_balanced_args(const void* q, int32_t n_q,
                                     const sdit_kv_segment* segs, int32_t n_segs,
                                     const uint8_t* block_mask, int32_t block_q, int32_t block_k,
                                     int32_t n_heads, int32_t head_dim, float softmax_scale,
                                     const void* out, const float* lse, const void* workspace,
                                     int64_t workspace_bytes, int32_t split_tile);
int sdit_validate_attn_partial_args(const void* q, int32_t n_q,
                                    const sdit_kv_segment* segs, int32_t n_segs,
                                    const uint8_t* block_mask, int32_t block_q, int32_t block_k,
                                    int32_t n_heads, int32_t head_dim, float softmax_scale,
                                    const float* out, const float* lse);
int sdit_validate_window_permute_args(const void* x, const void* y, int32_t T, int32_t Hl, int32_t Wl,
                                      int32_t n_heads, int32_t head_dim, int32_t window, int32_t inverse);
int sdit_validate_attn_merge_args(const float* const* o_parts, const float* const* lse_parts,
                                  int32_t n_parts, int32_t n_q, int32_t n_heads, int32_t head_dim,
                                  const void* out, const float* lse_out);
int sdit_validate_rmsnorm_args(const void* x, const void* y, const float* gamma, int64_t n_tok,
                               int32_t dim, float eps);
int sdit_validate_layernorm_modulate_args(const void* x, const void* y, const float* scale,
                                          const float* shift, int64_t n_tok, int32_t dim, float eps);

#ifdef __cplusplus
}
#endif

#endif /* SDIT_H */
