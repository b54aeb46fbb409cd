// C ABI of the sdit library: argument validation, launch geometry, errors.
// Every check runs on the host before a launch; nothing here allocates.
#include "../../include/sdit.h"

#include <math.h>
#include <stdarg.h>

#include <algorithm>
#include <atomic>
#include <stdio.h>
#include <string.h>

#include "sdit_internal.h"

#define SDIT_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return SDIT_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  if (na <= 0 || nb <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

int device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  if (e == hipErrorNoBinaryForGpu || e == hipErrorInvalidDeviceFunction || e == hipErrorInvalidImage ||
      e == hipErrorSharedObjectInitFailed)
    return fail(SDIT_ERR_UNSUPPORTED, "%s: no gfx950 code object for the current device (%s)", what,
                hipGetErrorString(e));
  return fail(SDIT_ERR_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
}

// a >= 0, b > 0; no intermediate a + b - 1 that could pass INT32_MAX
int ceil_div(int a, int b) { return a / b + (a % b != 0); }

// a * b for a, b >= 0, saturated at INT64_MAX: size checks compare the
// result with limits far below that, so a saturated product is rejected
int64_t mul_sat(int64_t a, int64_t b) { return (a != 0 && b > INT64_MAX / a) ? INT64_MAX : a * b; }

// largest element count (n_tok * n_heads * head_dim) of any one tensor
constexpr int64_t kMaxElems = (int64_t)1 << 40;

bool valid_block(int b) { return b == 16 || b == 32 || b == 64 || b == 128; }

}  // namespace

SDIT_API int sdit_abi_version(void) { return SDIT_ABI_VERSION; }

SDIT_API const char* sdit_status_string(int status) {
  switch (status) {
    case SDIT_OK: return "SDIT_OK";
    case SDIT_ERR_INVALID: return "SDIT_ERR_INVALID";
    case SDIT_ERR_UNSUPPORTED: return "SDIT_ERR_UNSUPPORTED";
    case SDIT_ERR_DEVICE: return "SDIT_ERR_DEVICE";
    default: return "SDIT_UNKNOWN_STATUS";
  }
}

SDIT_API const char* sdit_last_error(void) { return g_err; }

// ------------------------------------------------------------------ qknorm_rope3d

SDIT_API int sdit_validate_qknorm_rope3d_args(const void* q_in, const void* k_in, void* q_out, void* k_out,
                                              const float* gamma_q, const float* gamma_k, int32_t T,
                                              int32_t Hl, int32_t Wl, int32_t t0, int32_t n_heads,
                                              int32_t head_dim, int32_t d_t, int32_t d_h, int32_t d_w,
                                              float theta, float eps) {
  if (head_dim != 64 && head_dim != 128)
    return fail(SDIT_ERR_UNSUPPORTED, "qknorm_rope3d: head_dim %d not in {64, 128}", head_dim);
  if (n_heads < 1) return fail(SDIT_ERR_INVALID, "qknorm_rope3d: n_heads %d < 1", n_heads);
  if (T < 0 || Hl < 0 || Wl < 0 || t0 < 0)
    return fail(SDIT_ERR_INVALID, "qknorm_rope3d: negative grid (T=%d Hl=%d Wl=%d t0=%d)", T, Hl, Wl, t0);
  if (d_t < 0 || d_h < 0 || d_w < 0 || (d_t | d_h | d_w) & 1 || d_t + d_h + d_w != head_dim)
    return fail(SDIT_ERR_INVALID, "qknorm_rope3d: axis split %d/%d/%d must be even and sum to %d", d_t, d_h,
                d_w, head_dim);
  if (!(theta > 0.f) || !isfinite(theta)) return fail(SDIT_ERR_INVALID, "qknorm_rope3d: theta must be > 0");
  if (!(eps >= 0.f) || !isfinite(eps)) return fail(SDIT_ERR_INVALID, "qknorm_rope3d: eps must be >= 0");
  const int64_t n_tok = mul_sat(mul_sat(T, Hl), Wl);
  if (n_tok > INT32_MAX) return fail(SDIT_ERR_INVALID, "qknorm_rope3d: too many tokens");
  if (n_tok * n_heads > kMaxElems / head_dim) return fail(SDIT_ERR_INVALID, "qknorm_rope3d: q/k too large");
  if ((int64_t)t0 + T > (1 << 24)) return fail(SDIT_ERR_INVALID, "qknorm_rope3d: t positions too large");
  if (n_tok == 0) return ok();
  const void* ptrs[4] = {q_in, k_in, q_out, k_out};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned(p, 16))
      return fail(SDIT_ERR_INVALID, "qknorm_rope3d: q/k pointers must be non-NULL and 16-byte aligned");
  if (gamma_q == nullptr || gamma_k == nullptr || !aligned(gamma_q, 16) || !aligned(gamma_k, 16))
    return fail(SDIT_ERR_INVALID, "qknorm_rope3d: gamma pointers must be non-NULL and 16-byte aligned");
  const int64_t bytes = n_tok * n_heads * head_dim * 2;
  if ((q_out != q_in && overlap(q_out, bytes, q_in, bytes)) || (k_out != k_in && overlap(k_out, bytes, k_in, bytes)) ||
      overlap(q_out, bytes, k_out, bytes) || overlap(q_out, bytes, k_in, bytes) || overlap(k_out, bytes, q_in, bytes))
    return fail(SDIT_ERR_INVALID, "qknorm_rope3d: outputs overlap inputs (only exact in-place is allowed)");
  if (overlap(q_out, bytes, gamma_q, head_dim * 4) || overlap(q_out, bytes, gamma_k, head_dim * 4) ||
      overlap(k_out, bytes, gamma_q, head_dim * 4) || overlap(k_out, bytes, gamma_k, head_dim * 4))
    return fail(SDIT_ERR_INVALID, "qknorm_rope3d: outputs overlap gamma");
  return ok();
}

namespace {

// Kernel arguments of a validated qknorm_rope3d call (no int8 outputs).
void fill_rope_params(sdit::RopeParams* P, const void* q_in, const void* k_in, void* q_out, void* k_out,
                      const float* gamma_q, const float* gamma_k, int32_t T, int32_t Hl, int32_t Wl, int32_t t0,
                      int32_t n_heads, int32_t d_t, int32_t d_h, int32_t d_w, float theta, float eps) {
  sdit::RopeParams& p = *P;
  memset(&p, 0, sizeof(p));
  p.q_in = (const uint16_t*)q_in;
  p.k_in = (const uint16_t*)k_in;
  p.q_out = (uint16_t*)q_out;
  p.k_out = (uint16_t*)k_out;
  p.gamma_q = gamma_q;
  p.gamma_k = gamma_k;
  p.n_tok = (int32_t)((int64_t)T * Hl * Wl);   // validated: at most INT32_MAX
  p.Hl = Hl;
  p.Wl = Wl;
  p.t0 = t0;
  p.n_heads = n_heads;
  p.d_t = d_t;
  p.d_h = d_h;
  p.d_w = d_w;
  // pair j of an axis of width d_a turns at theta^(-2j/d_a), in column order t | h | w
  int c = 0;
  for (int a = 0; a < 3; ++a) {
    const int da = a == 0 ? d_t : (a == 1 ? d_h : d_w);
    for (int j = 0; j < da / 2; ++j) p.omega[c++] = pow((double)theta, -2.0 * j / da);
  }
  for (; c < 64; ++c) p.omega[c] = 0.0;
  p.eps = eps;
}

}  // namespace

SDIT_API int sdit_qknorm_rope3d(const void* q_in, const void* k_in, void* q_out, void* k_out,
                                const float* gamma_q, const float* gamma_k, int32_t T, int32_t Hl, int32_t Wl,
                                int32_t t0, int32_t n_heads, int32_t head_dim, int32_t d_t, int32_t d_h,
                                int32_t d_w, float theta, float eps, void* stream) {
  int st = sdit_validate_qknorm_rope3d_args(q_in, k_in, q_out, k_out, gamma_q, gamma_k, T, Hl, Wl, t0, n_heads,
                                            head_dim, d_t, d_h, d_w, theta, eps);
  if (st != SDIT_OK) return st;
  sdit::RopeParams p;
  fill_rope_params(&p, q_in, k_in, q_out, k_out, gamma_q, gamma_k, T, Hl, Wl, t0, n_heads, d_t, d_h, d_w, theta, eps);
  if (p.n_tok == 0) return ok();
  return device_status(sdit::launch_qknorm_rope3d(p, head_dim, (hipStream_t)stream), "qknorm_rope3d");
}

SDIT_API int sdit_validate_qknorm_rope3d_kv_quant_int8_args(
    const void* q_in, const void* k_in, const void* v_in, void* q_out, void* k_out, const int8_t* k_codes,
    const float* k_scales, const int8_t* v_codes, const float* v_scales, const float* gamma_q,
    const float* gamma_k, int32_t T, int32_t Hl, int32_t Wl, int32_t t0, int32_t n_heads, int32_t head_dim,
    int32_t d_t, int32_t d_h, int32_t d_w, float theta, float eps) {
  int st = sdit_validate_qknorm_rope3d_args(q_in, k_in, q_out, k_out, gamma_q, gamma_k, T, Hl, Wl, t0, n_heads,
                                            head_dim, d_t, d_h, d_w, theta, eps);
  if (st != SDIT_OK) return st;
  const int64_t n_tok = (int64_t)T * Hl * Wl;
  if (n_tok == 0) return ok();
  if (v_in == nullptr || !aligned(v_in, 16))
    return fail(SDIT_ERR_INVALID, "qknorm_rope3d_kv_quant_int8: v_in must be non-NULL and 16-byte aligned");
  if (k_codes == nullptr || v_codes == nullptr || !aligned(k_codes, 16) || !aligned(v_codes, 16))
    return fail(SDIT_ERR_INVALID, "qknorm_rope3d_kv_quant_int8: codes must be non-NULL and 16-byte aligned");
  if (k_scales == nullptr || v_scales == nullptr || !aligned(k_scales, 4) || !aligned(v_scales, 4))
    return fail(SDIT_ERR_INVALID, "qknorm_rope3d_kv_quant_int8: scales must be non-NULL and 4-byte aligned");
  const int64_t rows = n_tok * n_heads, bytes = rows * head_dim * 2, cbytes = rows * head_dim, sbytes = rows * 4;
  // every output apart from each other and from every input (q_out/k_out may
  // equal q_in/k_in, already checked)
  const void* outs[4] = {k_codes, k_scales, v_codes, v_scales};
  const int64_t osz[4] = {cbytes, sbytes, cbytes, sbytes};
  const void* others[8] = {q_in, k_in, v_in, q_out, k_out, gamma_q, gamma_k, nullptr};
  const int64_t oth[8] = {bytes, bytes, bytes, bytes, bytes, head_dim * 4, head_dim * 4, 0};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 7; ++j)
      if (overlap(outs[i], osz[i], others[j], oth[j]))
        return fail(SDIT_ERR_INVALID, "qknorm_rope3d_kv_quant_int8: codes/scales overlap another argument");
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], osz[i], outs[j], osz[j]))
        return fail(SDIT_ERR_INVALID, "qknorm_rope3d_kv_quant_int8: codes/scales overlap each other");
  }
  if (overlap(v_in, bytes, q_out, bytes) || overlap(v_in, bytes, k_out, bytes))
    return fail(SDIT_ERR_INVALID, "qknorm_rope3d_kv_quant_int8: q_out/k_out overlap v_in");
  return ok();
}

SDIT_API int sdit_qknorm_rope3d_kv_quant_int8(const void* q_in, const void* k_in, const void* v_in, void* q_out,
                                              void* k_out, int8_t* k_codes, float* k_scales, int8_t* v_codes,
                                              float* v_scales, const float* gamma_q, const float* gamma_k,
                                              int32_t T, int32_t Hl, int32_t Wl, int32_t t0, int32_t n_heads,
                                              int32_t head_dim, int32_t d_t, int32_t d_h, int32_t d_w, float theta,
                                              float eps, void* stream) {
  int st = sdit_validate_qknorm_rope3d_kv_quant_int8_args(q_in, k_in, v_in, q_out, k_out, k_codes, k_scales,
                                                          v_codes, v_scales, gamma_q, gamma_k, T, Hl, Wl, t0,
                                                          n_heads, head_dim, d_t, d_h, d_w, theta, eps);
  if (st != SDIT_OK) return st;
  sdit::RopeParams p;
  fill_rope_params(&p, q_in, k_in, q_out, k_out, gamma_q, gamma_k, T, Hl, Wl, t0, n_heads, d_t, d_h, d_w, theta, eps);
  p.v_in = (const uint16_t*)v_in;
  p.k_codes = k_codes;
  p.k_scales = k_scales;
  p.v_codes = v_codes;
  p.v_scales = v_scales;
  if (p.n_tok == 0) return ok();
  return device_status(sdit::launch_qknorm_rope3d(p, head_dim, (hipStream_t)stream), "qknorm_rope3d_kv_quant_int8");
}

// ------------------------------------------------------------------ kv_quant_int8

SDIT_API int sdit_validate_kv_quant_args(const void* x, const int8_t* codes, const float* scales, int32_t n_tok,
                                         int32_t n_heads, int32_t head_dim) {
  if (head_dim != 64 && head_dim != 128)
    return fail(SDIT_ERR_UNSUPPORTED, "kv_quant_int8: head_dim %d not in {64, 128}", head_dim);
  if (n_heads < 1 || n_tok < 0) return fail(SDIT_ERR_INVALID, "kv_quant_int8: bad n_tok %d / n_heads %d", n_tok, n_heads);
  if (n_tok == 0) return ok();
  if (x == nullptr || codes == nullptr || scales == nullptr)
    return fail(SDIT_ERR_INVALID, "kv_quant_int8: NULL pointer");
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4))
    return fail(SDIT_ERR_INVALID, "kv_quant_int8: x/codes must be 16-byte and scales 4-byte aligned");
  const int64_t rows = (int64_t)n_tok * n_heads;
  if (rows > kMaxElems / head_dim) return fail(SDIT_ERR_INVALID, "kv_quant_int8: x too large");
  if (overlap(codes, rows * head_dim, x, rows * head_dim * 2) || overlap(scales, rows * 4, x, rows * head_dim * 2) ||
      overlap(scales, rows * 4, codes, rows * head_dim))
    return fail(SDIT_ERR_INVALID, "kv_quant_int8: buffers overlap");
  return ok();
}

SDIT_API int sdit_kv_quant_int8(const void* x, int8_t* codes, float* scales, int32_t n_tok, int32_t n_heads,
                                int32_t head_dim, void* stream) {
  int st = sdit_validate_kv_quant_args(x, codes, scales, n_tok, n_heads, head_dim);
  if (st != SDIT_OK) return st;
  if (n_tok == 0) return ok();
  sdit::QuantParams p;
  p.x = (const uint16_t*)x;
  p.codes = codes;
  p.scales = scales;
  p.n_rows = (int64_t)n_tok * n_heads;
  return device_status(sdit::launch_kv_quant_int8(p, head_dim, (hipStream_t)stream), "kv_quant_int8");
}

// ------------------------------------------------------------------ attn_fwd

namespace {

// out is bf16 [n_q][H][d], or fp32 when out_f32 (the partial form: lse
// then required).
int fill_attn_params(const void* q, int32_t n_q, const sdit_kv_segment* segs, int32_t n_segs,
                     const uint8_t* block_mask, int32_t block_q, int32_t block_k, int32_t n_heads,
                     int32_t head_dim, float softmax_scale, const void* out, const float* lse,
                     sdit::AttnParams* P, bool out_f32 = false) {
  const char* fn = out_f32 ? "attn_fwd_partial" : "attn_fwd";
  if (head_dim != 64 && head_dim != 128)
    return fail(SDIT_ERR_UNSUPPORTED, "attn_fwd: head_dim %d not in {64, 128}", head_dim);
  if (n_heads < 1) return fail(SDIT_ERR_INVALID, "attn_fwd: n_heads %d < 1", n_heads);
  // a key tile's rows are addressed with 32-bit offsets from its first row
  if (n_heads > 65536) return fail(SDIT_ERR_UNSUPPORTED, "attn_fwd: n_heads %d > 65536", n_heads);
  if (n_q < 0) return fail(SDIT_ERR_INVALID, "attn_fwd: n_q %d < 0", n_q);
  if (!valid_block(block_q) || !valid_block(block_k))
    return fail(SDIT_ERR_UNSUPPORTED, "attn_fwd: block sizes %d x %d not in {16, 32, 64, 128}", block_q, block_k);
  if (n_segs < 1 || n_segs > SDIT_MAX_SEGMENTS)
    return fail(SDIT_ERR_INVALID, "attn_fwd: n_segs %d not in [1, %d]", n_segs, SDIT_MAX_SEGMENTS);
  if (segs == nullptr) return fail(SDIT_ERR_INVALID, "attn_fwd: segs is NULL");
  if (!isfinite(softmax_scale)) return fail(SDIT_ERR_INVALID, "attn_fwd: softmax_scale not finite");
  // a masked key's -1e30 bias times the scale has to stay far below every
  // visible score (the kernel takes maxima under -1e15 as "nothing visible")
  if (softmax_scale > 0.f && softmax_scale < 0x1p-40f)
    return fail(SDIT_ERR_INVALID, "attn_fwd: softmax_scale %g below 2^-40", (double)softmax_scale);
  if ((int64_t)n_q * n_heads > kMaxElems / head_dim) return fail(SDIT_ERR_INVALID, "attn_fwd: q too large");
  int64_t tiles = 0, kbs = 0;
  for (int s = 0; s < n_segs; ++s) {
    const sdit_kv_segment& sg = segs[s];
    if (sg.len < 0) return fail(SDIT_ERR_INVALID, "attn_fwd: segment %d has len %d < 0", s, sg.len);
    if (sg.dtype != SDIT_BF16 && sg.dtype != SDIT_INT8)
      return fail(SDIT_ERR_INVALID, "attn_fwd: segment %d has unknown dtype %d", s, sg.dtype);
    if (sg.dtype == SDIT_BF16 && (sg.k_scale != nullptr || sg.v_scale != nullptr))
      return fail(SDIT_ERR_INVALID, "attn_fwd: bf16 segment %d must have NULL scales", s);
    if (sg.len > 0) {
      if (sg.k == nullptr || sg.v == nullptr || !aligned(sg.k, 16) || !aligned(sg.v, 16))
        return fail(SDIT_ERR_INVALID, "attn_fwd: segment %d k/v must be non-NULL and 16-byte aligned", s);
      if (sg.dtype == SDIT_INT8 && (sg.k_scale == nullptr || sg.v_scale == nullptr || !aligned(sg.k_scale, 4) ||
                                    !aligned(sg.v_scale, 4)))
        return fail(SDIT_ERR_INVALID, "attn_fwd: int8 segment %d needs 4-byte aligned k_scale and v_scale", s);
      const int64_t esz = sg.dtype == SDIT_INT8 ? 1 : 2;
      const int64_t seg_bytes = (int64_t)sg.len * n_heads * head_dim * esz;
      const int64_t out_bytes = (int64_t)n_q * n_heads * head_dim * (out_f32 ? 4 : 2);
      if (overlap(out, out_bytes, sg.k, seg_bytes) || overlap(out, out_bytes, sg.v, seg_bytes))
        return fail(SDIT_ERR_INVALID, "attn_fwd: out overlaps segment %d", s);
    }
    tiles += ceil_div(sg.len, sdit::kAttnBK);
    kbs += ceil_div(sg.len, block_k);
  }
  if (tiles > (1 << 24))
    return fail(SDIT_ERR_UNSUPPORTED, "attn_fwd: more than 2^24 key tiles of %d keys", sdit::kAttnBK);
  const int n_qb = ceil_div(n_q, block_q);
  const int n_qt = ceil_div(n_q, sdit::kAttnBQ);
  if ((int64_t)n_qt * n_heads > INT32_MAX / 2) return fail(SDIT_ERR_INVALID, "attn_fwd: grid too large");
  if (n_q > 0) {
    if (q == nullptr || !aligned(q, 16)) return fail(SDIT_ERR_INVALID, "attn_fwd: q must be non-NULL, 16-byte aligned");
    if (out == nullptr || !aligned(out, 16))
      return fail(SDIT_ERR_INVALID, "%s: out must be non-NULL, 16-byte aligned", fn);
    if (out_f32 && lse == nullptr) return fail(SDIT_ERR_INVALID, "%s: lse is required", fn);
    if (lse != nullptr && !aligned(lse, 4)) return fail(SDIT_ERR_INVALID, "%s: lse must be 4-byte aligned", fn);
    if (kbs > 0 && block_mask == nullptr) return fail(SDIT_ERR_INVALID, "attn_fwd: block_mask is NULL");
    const int64_t qbytes = (int64_t)n_q * n_heads * head_dim * 2;
    const int64_t obytes = out_f32 ? 2 * qbytes : qbytes;
    if (overlap(out, obytes, q, qbytes)) return fail(SDIT_ERR_INVALID, "%s: out overlaps q", fn);
    if (lse != nullptr && (overlap(lse, (int64_t)n_q * n_heads * 4, out, obytes) ||
                           overlap(lse, (int64_t)n_q * n_heads * 4, q, qbytes)))
      return fail(SDIT_ERR_INVALID, "%s: lse overlaps q or out", fn);
  }
  if (P != nullptr) {
    memset(P, 0, sizeof(*P));
    P->q = (const uint16_t*)q;
    P->out = out_f32 ? nullptr : (uint16_t*)out;
    P->out_f32 = out_f32 ? (float*)out : nullptr;
    P->lse = (float*)lse;
    P->mask = block_mask;
    int tile = 0, kb = 0;
    for (int s = 0; s < n_segs; ++s) {
      P->seg[s].k = segs[s].k;
      P->seg[s].v = segs[s].v;
      P->seg[s].k_scale = segs[s].k_scale;
      P->seg[s].v_scale = segs[s].v_scale;
      P->seg[s].len = segs[s].len;
      P->seg[s].is_int8 = segs[s].dtype == SDIT_INT8;
      P->seg[s].tile_start = tile;
      P->seg[s].kb_start = kb;
      tile += ceil_div(segs[s].len, sdit::kAttnBK);
      kb += ceil_div(segs[s].len, block_k);
    }
    P->n_segs = n_segs;
    P->n_q = n_q;
    P->n_heads = n_heads;
    P->n_qt = n_qt;
    P->n_tiles = tile;
    P->n_kb = kb;
    P->n_qb = n_qb;
    P->block_q = block_q;
    P->block_k = block_k;
    P->block_k_log2 = __builtin_ctz((unsigned)block_k);
    P->grid = n_qt * n_heads;   // one workgroup per unit; a balanced launch re-plans it
    P->cu_per_xcd = 1;
    const double scale = softmax_scale > 0.f ? (double)softmax_scale : 1.0 / sqrt((double)head_dim);
    P->scale_log2 = (float)(scale * 1.4426950408889634073599246810019);
  }
  return ok();
}

}  // namespace

SDIT_API int sdit_validate_attn_args(const void* q, int32_t n_q, const sdit_kv_segment* segs, int32_t n_segs,
                                     const uint8_t* block_mask, int32_t block_q, int32_t block_k, int32_t n_heads,
                                     int32_t head_dim, float softmax_scale, const void* out, const float* lse) {
  return fill_attn_params(q, n_q, segs, n_segs, block_mask, block_q, block_k, n_heads, head_dim, softmax_scale, out,
                          lse, nullptr);
}

SDIT_API int sdit_validate_attn_partial_args(const void* q, int32_t n_q, const sdit_kv_segment* segs,
                                             int32_t n_segs, const uint8_t* block_mask, int32_t block_q,
                                             int32_t block_k, int32_t n_heads, int32_t head_dim,
                                             float softmax_scale, const float* out, const float* lse) {
  return fill_attn_params(q, n_q, segs, n_segs, block_mask, block_q, block_k, n_heads, head_dim, softmax_scale, out,
                          lse, nullptr, true);
}

SDIT_API int sdit_attn_fwd_partial(const void* q, int32_t n_q, const sdit_kv_segment* segs, int32_t n_segs,
                                   const uint8_t* block_mask, int32_t block_q, int32_t block_k, int32_t n_heads,
                                   int32_t head_dim, float softmax_scale, float* out, float* lse, void* stream) {
  sdit::AttnParams P;
  int st = fill_attn_params(q, n_q, segs, n_segs, block_mask, block_q, block_k, n_heads, head_dim, softmax_scale,
                            out, lse, &P, true);
  if (st != SDIT_OK) return st;
  if (n_q == 0) return ok();
  return device_status(sdit::launch_attn_fwd(P, head_dim, (hipStream_t)stream), "attn_fwd_partial");
}

// ------------------------------------------------------------------ attn_merge

static_assert(SDIT_MAX_MERGE_PARTS == sdit::kMaxMergeParts, "merge part limit");

namespace {

int fill_merge_params(const float* const* o_parts, const float* const* lse_parts, int32_t n_parts, int32_t n_q,
                      int32_t n_heads, int32_t head_dim, const void* out, const float* lse_out,
                      sdit::MergeParams* P) {
  if (head_dim != 64 && head_dim != 128)
    return fail(SDIT_ERR_UNSUPPORTED, "attn_merge: head_dim %d not in {64, 128}", head_dim);
  if (n_heads < 1) return fail(SDIT_ERR_INVALID, "attn_merge: n_heads %d < 1", n_heads);
  if (n_q < 0) return fail(SDIT_ERR_INVALID, "attn_merge: n_q %d < 0", n_q);
  if (n_parts < 1 || n_parts > SDIT_MAX_MERGE_PARTS)
    return fail(SDIT_ERR_INVALID, "attn_merge: n_parts %d not in [1, %d]", n_parts, SDIT_MAX_MERGE_PARTS);
  if (o_parts == nullptr || lse_parts == nullptr) return fail(SDIT_ERR_INVALID, "attn_merge: part arrays are NULL");
  if ((int64_t)n_q * n_heads > kMaxElems / head_dim) return fail(SDIT_ERR_INVALID, "attn_merge: too large");
  const int64_t obytes = (int64_t)n_q * n_heads * head_dim * 2;
  const int64_t fbytes = 2 * obytes, lbytes = (int64_t)n_q * n_heads * 4;
  if (n_q > 0) {
    if (out == nullptr || !aligned(out, 16))
      return fail(SDIT_ERR_INVALID, "attn_merge: out must be non-NULL, 16-byte aligned");
    if (lse_out != nullptr && !aligned(lse_out, 4))
      return fail(SDIT_ERR_INVALID, "attn_merge: lse_out must be 4-byte aligned");
    if (lse_out != nullptr && overlap(lse_out, lbytes, out, obytes))
      return fail(SDIT_ERR_INVALID, "attn_merge: lse_out overlaps out");
    for (int i = 0; i < n_parts; ++i) {
      if (o_parts[i] == nullptr || !aligned(o_parts[i], 16))
        return fail(SDIT_ERR_INVALID, "attn_merge: part %d output must be non-NULL, 16-byte aligned", i);
      if (lse_parts[i] == nullptr || !aligned(lse_parts[i], 4))
        return fail(SDIT_ERR_INVALID, "attn_merge: part %d lse must be non-NULL, 4-byte aligned", i);
      if (overlap(out, obytes, o_parts[i], fbytes) || overlap(out, obytes, lse_parts[i], lbytes) ||
          (lse_out != nullptr && (overlap(lse_out, lbytes, o_parts[i], fbytes) ||
                                  overlap(lse_out, lbytes, lse_parts[i], lbytes))))
        return fail(SDIT_ERR_INVALID, "attn_merge: outputs overlap part %d", i);
    }
  }
  if (P != nullptr) {
    memset(P, 0, sizeof(*P));
    for (int i = 0; i < n_parts; ++i) {
      P->o[i] = o_parts[i];
      P->lse[i] = lse_parts[i];
    }
    P->n_parts = n_parts;
    P->n_q = n_q;
    P->n_heads = n_heads;
    P->out = (uint16_t*)out;
    P->lse_out = (float*)lse_out;
  }
  return ok();
}

}  // namespace

SDIT_API int sdit_validate_attn_merge_args(const float* const* o_parts, const float* const* lse_parts,
                                           int32_t n_parts, int32_t n_q, int32_t n_heads, int32_t head_dim,
                                           const void* out, const float* lse_out) {
  return fill_merge_params(o_parts, lse_parts, n_parts, n_q, n_heads, head_dim, out, lse_out, nullptr);
}

SDIT_API int sdit_attn_merge(const float* const* o_parts, const float* const* lse_parts, int32_t n_parts,
                             int32_t n_q, int32_t n_heads, int32_t head_dim, void* out, float* lse_out,
                             void* stream) {
  sdit::MergeParams P;
  int st = fill_merge_params(o_parts, lse_parts, n_parts, n_q, n_heads, head_dim, out, lse_out, &P);
  if (st != SDIT_OK) return st;
  if (n_q == 0) return ok();
  return device_status(sdit::launch_attn_merge(P, head_dim, (hipStream_t)stream), "attn_merge");
}

// ------------------------------------------------------------------ window_permute

namespace {

int fill_permute_params(const void* x, const void* y, int32_t T, int32_t Hl, int32_t Wl, int32_t n_heads,
                        int32_t head_dim, int32_t window, int32_t inverse, sdit::PermuteParams* P) {
  if (head_dim != 64 && head_dim != 128)
    return fail(SDIT_ERR_UNSUPPORTED, "window_permute: head_dim %d not in {64, 128}", head_dim);
  if (window != 2 && window != 4 && window != 8 && window != 16)
    return fail(SDIT_ERR_UNSUPPORTED, "window_permute: window %d not in {2, 4, 8, 16}", window);
  if (T < 0 || Hl < 0 || Wl < 0 || n_heads < 1)
    return fail(SDIT_ERR_INVALID, "window_permute: bad shape T=%d Hl=%d Wl=%d n_heads=%d", T, Hl, Wl, n_heads);
  if (Hl % window != 0 || Wl % window != 0)
    return fail(SDIT_ERR_INVALID, "window_permute: frame %d x %d is not whole %d x %d windows", Hl, Wl, window,
                window);
  if (inverse != 0 && inverse != 1) return fail(SDIT_ERR_INVALID, "window_permute: inverse must be 0 or 1");
  // a workgroup walks 8 rows of n_heads * head_dim / 8 16-byte chunks with 32-bit indices
  if ((int64_t)n_heads * head_dim > (1 << 24))
    return fail(SDIT_ERR_UNSUPPORTED, "window_permute: row of %d heads x %d too wide", n_heads, head_dim);
  const int64_t n_tok = mul_sat(mul_sat(T, Hl), Wl);
  if (n_tok > INT32_MAX / 2) return fail(SDIT_ERR_INVALID, "window_permute: too many tokens");
  if (n_tok * n_heads > kMaxElems / head_dim) return fail(SDIT_ERR_INVALID, "window_permute: x too large");
  const int64_t bytes = n_tok * n_heads * head_dim * 2;
  if (n_tok > 0) {
    if (x == nullptr || y == nullptr || !aligned(x, 16) || !aligned(y, 16))
      return fail(SDIT_ERR_INVALID, "window_permute: x and y must be non-NULL, 16-byte aligned");
    if (overlap(x, bytes, y, bytes)) return fail(SDIT_ERR_INVALID, "window_permute: x and y overlap");
  }
  if (P != nullptr) {
    P->x = (const uint16_t*)x;
    P->y = (uint16_t*)y;
    P->T = T;
    P->Hl = Hl;
    P->Wl = Wl;
    P->win = window;
    P->row_chunks = n_heads * head_dim / 8;
    P->inverse = inverse;
    P->n_tok = n_tok;
  }
  return ok();
}

}  // namespace

SDIT_API int sdit_validate_window_permute_args(const void* x, const void* y, int32_t T, int32_t Hl, int32_t Wl,
                                               int32_t n_heads, int32_t head_dim, int32_t window, int32_t inverse) {
  return fill_permute_params(x, y, T, Hl, Wl, n_heads, head_dim, window, inverse, nullptr);
}

SDIT_API int sdit_window_permute(const void* x, void* y, int32_t T, int32_t Hl, int32_t Wl, int32_t n_heads,
                                 int32_t head_dim, int32_t window, int32_t inverse, void* stream) {
  sdit::PermuteParams P;
  int st = fill_permute_params(x, y, T, Hl, Wl, n_heads, head_dim, window, inverse, &P);
  if (st != SDIT_OK) return st;
  if (P.n_tok == 0) return ok();
  return device_status(sdit::launch_window_permute(P, (hipStream_t)stream), "window_permute");
}

// ------------------------------------------------------------------ rmsnorm / layernorm_modulate

namespace {

// x, y bf16 [n_tok][dim]; vec[0..n_vec) fp32 [dim] each.
int fill_norm_params(const char* fn, const void* x, const void* y, const float* const* vec, int n_vec,
                     int64_t n_tok, int32_t dim, float eps, sdit::NormParams* P) {
  if (dim < 8 || dim > SDIT_MAX_NORM_DIM || dim % 8 != 0)
    return fail(SDIT_ERR_UNSUPPORTED, "%s: dim %d is not a multiple of 8 in [8, %d]", fn, dim, SDIT_MAX_NORM_DIM);
  // one 64-lane wave per token; a launch holds fewer than 2^32 threads
  if (n_tok < 0 || n_tok >= ((int64_t)1 << 26))
    return fail(SDIT_ERR_INVALID, "%s: n_tok %lld outside [0, 2^26)", fn, (long long)n_tok);
  if (!(eps >= 0.0f) || eps > 1.0f) return fail(SDIT_ERR_INVALID, "%s: eps must be in [0, 1]", fn);
  if (n_tok > 0) {
    const int64_t bytes = n_tok * dim * 2;
    if (x == nullptr || y == nullptr || !aligned(x, 16) || !aligned(y, 16))
      return fail(SDIT_ERR_INVALID, "%s: x and y must be non-NULL, 16-byte aligned", fn);
    if (y != x && overlap(x, bytes, y, bytes))
      return fail(SDIT_ERR_INVALID, "%s: y overlaps x (only exact in-place is allowed)", fn);
    for (int i = 0; i < n_vec; ++i) {
      if (vec[i] == nullptr || !aligned(vec[i], 16))
        return fail(SDIT_ERR_INVALID, "%s: parameter vectors must be non-NULL, 16-byte aligned", fn);
      if (overlap(y, bytes, vec[i], (int64_t)dim * 4))
        return fail(SDIT_ERR_INVALID, "%s: y overlaps a parameter vector", fn);
    }
  }
  if (P != nullptr) {
    P->x = (const uint16_t*)x;
    P->y = (uint16_t*)y;
    P->gamma = n_vec == 1 ? vec[0] : nullptr;
    P->scale = n_vec == 2 ? vec[0] : nullptr;
    P->shift = n_vec == 2 ? vec[1] : nullptr;
    P->n_tok = n_tok;
    P->dim = dim;
    P->eps = eps;
  }
  return ok();
}

}  // namespace

SDIT_API int sdit_validate_rmsnorm_args(const void* x, const void* y, const float* gamma, int64_t n_tok, int32_t dim,
                                        float eps) {
  const float* vec[1] = {gamma};
  return fill_norm_params("rmsnorm", x, y, vec, 1, n_tok, dim, eps, nullptr);
}

SDIT_API int sdit_rmsnorm(const void* x, void* y, const float* gamma, int64_t n_tok, int32_t dim, float eps,
                          void* stream) {
  const float* vec[1] = {gamma};
  sdit::NormParams P;
  int st = fill_norm_params("rmsnorm", x, y, vec, 1, n_tok, dim, eps, &P);
  if (st != SDIT_OK) return st;
  if (n_tok == 0) return ok();
  return device_status(sdit::launch_rmsnorm(P, (hipStream_t)stream), "rmsnorm");
}

SDIT_API int sdit_validate_layernorm_modulate_args(const void* x, const void* y, const float* scale,
                                                   const float* shift, int64_t n_tok, int32_t dim, float eps) {
  const float* vec[2] = {scale, shift};
  return fill_norm_params("layernorm_modulate", x, y, vec, 2, n_tok, dim, eps, nullptr);
}

SDIT_API int sdit_layernorm_modulate(const void* x, void* y, const float* scale, const float* shift, int64_t n_tok,
                                     int32_t dim, float eps, void* stream) {
  const float* vec[2] = {scale, shift};
  sdit::NormParams P;
  int st = fill_norm_params("layernorm_modulate", x, y, vec, 2, n_tok, dim, eps, &P);
  if (st != SDIT_OK) return st;
  if (n_tok == 0) return ok();
  return device_status(sdit::launch_layernorm_modulate(P, (hipStream_t)stream), "layernorm_modulate");
}

SDIT_API int sdit_attn_fwd(const void* q, int32_t n_q, const sdit_kv_segment* segs, int32_t n_segs,
                           const uint8_t* block_mask, int32_t block_q, int32_t block_k, int32_t n_heads,
                           int32_t head_dim, float softmax_scale, void* out, float* lse, void* stream) {
  sdit::AttnParams P;
  int st = fill_attn_params(q, n_q, segs, n_segs, block_mask, block_q, block_k, n_heads, head_dim, softmax_scale,
                            out, lse, &P);
  if (st != SDIT_OK) return st;
  if (n_q == 0) return ok();
  return device_status(sdit::launch_attn_fwd(P, head_dim, (hipStream_t)stream), "attn_fwd");
}

// ------------------------------------------------------------------ attn_fwd_balanced

namespace {

// Split units per XCD that the workspace bound covers (an XCD has at most 32 CUs).
constexpr int kMaxCuPerXcd = 32;
static_assert(SDIT_ATTN_WORKSPACE_BYTES(128) ==
                  (int64_t)sdit::kNumXcd * (kMaxCuPerXcd - 1) * 2 * sdit::kAttnBQ * (128 + 1) * 4,
              "workspace bound");

int64_t ws_o_floats(int rmax, int head_dim) { return (int64_t)sdit::kNumXcd * rmax * 2 * sdit::kAttnBQ * head_dim; }

// CUs per XCD of the current device (capped at kMaxCuPerXcd), cached per device.
int cu_per_xcd(int* c) {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, "attn_fwd_balanced");
  if (dev >= 0 && dev < 64 && cache[dev].load(std::memory_order_relaxed) > 0) {
    *c = cache[dev].load(std::memory_order_relaxed);
    return SDIT_OK;
  }
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return device_status(e, "attn_fwd_balanced");
  *c = std::max(1, std::min(kMaxCuPerXcd, cus / sdit::kNumXcd));
  if (dev >= 0 && dev < 64) cache[dev].store(*c, std::memory_order_relaxed);
  return SDIT_OK;
}

// The cut of a balanced launch. On an XCD with r units past its last full
// wave of C CUs, the r tail pieces queue on the C - r CUs the head pieces
// leave free, ceil(r / (C - r)) rounds of them; the head piece of t tiles
// has to outlast those rounds of n - t tiles each, plus a piece's fixed cost
// (loading its queries, writing its partial) of about kPieceCost tiles. The
// cut is kept only when it shortens the XCD's run by 5% or more and leaves
// tail pieces of at least 8 tiles, and not when the partial wave already
// keeps more than 3/4 of an XCD's CUs busy: measured on MI355X, filling the
// last few idle CUs does not shorten the run (the busy CUs run faster while
// the others idle) and the merge then only adds its cost. (Wan chunk, 29 of
// 32 CUs busy: 2.5% slower with the cut; Large-DiT, 20 of 32: 7% faster.)
struct BalancedPlan {
  int tile = 0, rmax = 0, grid = 0;
};

BalancedPlan plan_balanced(int n_units, int n, int C, int32_t split_tile) {
  constexpr int kPieceCost = 3;
  BalancedPlan bp;
  bp.grid = n_units;
  if (split_tile == 0 || C < 2 || n < 2) return bp;
  int rounds = 0, rmax = 0, blocks = 0, waves = 0;
  for (int x = 0; x < sdit::kNumXcd; ++x) {
    const sdit::XcdUnits u = sdit::xcd_units(n_units, x, C, true);
    blocks = std::max(blocks, u.n + u.r);
    waves = std::max(waves, u.n / C + (u.r > 0 ? 1 : 0));
    if (u.r == 0) continue;
    rmax = std::max(rmax, u.r);
    rounds = std::max(rounds, ceil_div(u.r, C - u.r));
  }
  if (rmax == 0) return bp;
  int t = split_tile;
  if (t < 0) {
    if (4 * rmax > 3 * C) return bp;
    t = (int)(((int64_t)rounds * (n + kPieceCost) + rounds) / (rounds + 1));
    const int saved = n - t;
    if (saved < 8 || 20 * (int64_t)saved < (int64_t)waves * n) return bp;
  }
  bp.tile = t;
  bp.rmax = rmax;
  bp.grid = sdit::kNumXcd * blocks;
  return bp;
}

int check_workspace(const void* q, int32_t n_q, const sdit_kv_segment* segs, int32_t n_segs,
                    const uint8_t* block_mask, int32_t block_q, int32_t block_k, int32_t n_heads,
                    int32_t head_dim, const void* out, const float* lse, const void* workspace,
                    int64_t workspace_bytes, int32_t split_tile) {
  int64_t tiles = 0, kbs = 0;
  for (int s = 0; s < n_segs; ++s) {
    tiles += ceil_div(segs[s].len, sdit::kAttnBK);
    kbs += ceil_div(segs[s].len, block_k);
  }
  if (split_tile < -1 || (split_tile > 0 && split_tile >= tiles))
    return fail(SDIT_ERR_INVALID, "attn_fwd_balanced: split_tile %d not -1, 0 or in [1, %lld)", split_tile,
                (long long)tiles);
  if (n_q == 0) return ok();
  if (workspace == nullptr || !aligned(workspace, 16))
    return fail(SDIT_ERR_INVALID, "attn_fwd_balanced: workspace must be non-NULL, 16-byte aligned");
  if (workspace_bytes < SDIT_ATTN_WORKSPACE_BYTES(head_dim))
    return fail(SDIT_ERR_INVALID, "attn_fwd_balanced: workspace of %lld bytes < %lld", (long long)workspace_bytes,
                (long long)SDIT_ATTN_WORKSPACE_BYTES(head_dim));
  const int64_t rows = (int64_t)n_q * n_heads;
  if (overlap(workspace, workspace_bytes, q, rows * head_dim * 2) ||
      overlap(workspace, workspace_bytes, out, rows * head_dim * 2) ||
      (lse != nullptr && overlap(workspace, workspace_bytes, lse, rows * 4)) ||
      overlap(workspace, workspace_bytes, block_mask, (int64_t)ceil_div(n_q, block_q) * kbs))
    return fail(SDIT_ERR_INVALID, "attn_fwd_balanced: workspace overlaps q, out, lse or block_mask");
  for (int s = 0; s < n_segs; ++s) {
    const sdit_kv_segment& sg = segs[s];
    if (sg.len == 0) continue;
    const int64_t kv = (int64_t)sg.len * n_heads * head_dim * (sg.dtype == SDIT_INT8 ? 1 : 2);
    const int64_t sc = (int64_t)sg.len * n_heads * 4;
    if (overlap(workspace, workspace_bytes, sg.k, kv) || overlap(workspace, workspace_bytes, sg.v, kv) ||
        (sg.k_scale != nullptr && overlap(workspace, workspace_bytes, sg.k_scale, sc)) ||
        (sg.v_scale != nullptr && overlap(workspace, workspace_bytes, sg.v_scale, sc)))
      return fail(SDIT_ERR_INVALID, "attn_fwd_balanced: workspace overlaps segment %d", s);
  }
  return ok();
}

}  // namespace

SDIT_API int sdit_attn_balanced_plan(int32_t n_q, int32_t n_heads, int32_t n_tiles, int32_t n_cus,
                                      int32_t split_tile, int32_t* tile, int32_t* grid) {
  if (n_q < 0 || n_heads < 1 || n_tiles < 0 || n_cus < 1 || split_tile < -1 || tile == nullptr || grid == nullptr)
    return fail(SDIT_ERR_INVALID, "attn_balanced_plan: bad arguments");
  if ((int64_t)ceil_div(n_q, sdit::kAttnBQ) * n_heads > INT32_MAX / 2)
    return fail(SDIT_ERR_INVALID, "attn_balanced_plan: grid too large");
  if (split_tile > 0 && split_tile >= n_tiles)
    return fail(SDIT_ERR_INVALID, "attn_balanced_plan: split_tile %d >= n_tiles %d", split_tile, n_tiles);
  const int C = std::max(1, std::min(kMaxCuPerXcd, n_cus / sdit::kNumXcd));
  const BalancedPlan bp = plan_balanced(ceil_div(n_q, sdit::kAttnBQ) * n_heads, n_tiles, C, split_tile);
  *tile = bp.tile;
  *grid = bp.grid;
  return ok();
}

SDIT_API int sdit_validate_attn_balanced_args(const void* q, int32_t n_q, const sdit_kv_segment* segs,
                                              int32_t n_segs, const uint8_t* block_mask, int32_t block_q,
                                              int32_t block_k, int32_t n_heads, int32_t head_dim,
                                              float softmax_scale, const void* out, const float* lse,
                                              const void* workspace, int64_t workspace_bytes, int32_t split_tile) {
  int st = fill_attn_params(q, n_q, segs, n_segs, block_mask, block_q, block_k, n_heads, head_dim, softmax_scale, out,
                            lse, nullptr);
  if (st != SDIT_OK) return st;
  return check_workspace(q, n_q, segs, n_segs, block_mask, block_q, block_k, n_heads, head_dim, out, lse, workspace,
                         workspace_bytes, split_tile);
}

namespace {

// The balanced launch with the workspace at ws (ws_bytes at least what its
// plan uses): attention kernel, then the merge of the cut pieces.
int launch_balanced(sdit::AttnParams& P, int head_dim, int32_t split_tile, void* ws, int64_t ws_bytes, void* out,
                    float* lse, hipStream_t stream, const char* fn) {
  int C = 1;
  if (split_tile != 0) {
    const int st = cu_per_xcd(&C);
    if (st != SDIT_OK) return st;
  }
  const BalancedPlan bp = plan_balanced(P.n_qt * P.n_heads, P.n_tiles, C, split_tile);
  const int64_t need = (ws_o_floats(bp.rmax, head_dim) + (int64_t)sdit::kNumXcd * bp.rmax * 2 * sdit::kAttnBQ) * 4;
  if (need > ws_bytes)
    return fail(SDIT_ERR_INVALID, "%s: the cut needs %lld bytes of scratch, %lld available", fn, (long long)need,
                (long long)ws_bytes);
  P.split_tile = bp.tile;
  P.split_rmax = bp.rmax;
  P.grid = bp.grid;
  P.cu_per_xcd = C;
  P.ws_o = (float*)ws;
  P.ws_lse = P.ws_o + ws_o_floats(P.split_rmax, head_dim);
  int st = device_status(sdit::launch_attn_fwd(P, head_dim, stream), fn);
  if (st != SDIT_OK) return st;
  return device_status(sdit::launch_attn_split_merge(P, (uint16_t*)out, lse, head_dim, stream), fn);
}

}  // namespace

SDIT_API int sdit_attn_fwd_balanced(const void* q, int32_t n_q, const sdit_kv_segment* segs, int32_t n_segs,
                                    const uint8_t* block_mask, int32_t block_q, int32_t block_k, int32_t n_heads,
                                    int32_t head_dim, float softmax_scale, void* out, float* lse, void* workspace,
                                    int64_t workspace_bytes, int32_t split_tile, void* stream) {
  sdit::AttnParams P;
  int st = fill_attn_params(q, n_q, segs, n_segs, block_mask, block_q, block_k, n_heads, head_dim, softmax_scale,
                            out, lse, &P);
  if (st != SDIT_OK) return st;
  st = check_workspace(q, n_q, segs, n_segs, block_mask, block_q, block_k, n_heads, head_dim, out, lse, workspace,
                       workspace_bytes, split_tile);
  if (st != SDIT_OK) return st;
  if (n_q == 0) return ok();
  return launch_balanced(P, head_dim, split_tile, workspace, workspace_bytes, out, lse, (hipStream_t)stream,
                         "attn_fwd_balanced");
}

SDIT_API int sdit_attn_fwd_balanced_static(const void* q, int32_t n_q, const sdit_kv_segment* segs, int32_t n_segs,
                                           const uint8_t* block_mask, int32_t block_q, int32_t block_k,
                                           int32_t n_heads, int32_t head_dim, float softmax_scale, void* out,
                                           float* lse, int32_t split_tile, void* stream) {
  sdit::AttnParams P;
  int st = fill_attn_params(q, n_q, segs, n_segs, block_mask, block_q, block_k, n_heads, head_dim, softmax_scale,
                            out, lse, &P);
  if (st != SDIT_OK) return st;
  if (split_tile < -1 || (split_tile > 0 && split_tile >= P.n_tiles))
    return fail(SDIT_ERR_INVALID, "attn_fwd_balanced_static: split_tile %d not -1, 0 or in [1, %d)", split_tile,
                P.n_tiles);
  if (n_q == 0) return ok();
  void* ws = nullptr;
  const hipError_t e = sdit::static_scratch(&ws);
  if (e != hipSuccess) return device_status(e, "attn_fwd_balanced_static (scratch address)");
  return launch_balanced(P, head_dim, split_tile, ws, SDIT_STATIC_SCRATCH_BYTES, out, lse, (hipStream_t)stream,
                         "attn_fwd_balanced_static");
}

static_assert(SDIT_STATIC_SCRATCH_BYTES == sdit::kStaticScratchBytes, "static scratch size");
static_assert(SDIT_STATIC_SCRATCH_BYTES >= SDIT_ATTN_WORKSPACE_BYTES(128), "static scratch covers every plan");
