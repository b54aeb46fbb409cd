// Merge of attention results over disjoint key sets, gfx950.
//
// Context-parallel attention (the Ulysses / Ring schemes that the Wave
// Forcing summary compares Wave Parallelism against) attends to one shard of
// the keys per step and combines the shards' results. For one query, with
// LSE_p the log-sum-exp of the scaled scores over shard p and o_p the
// softmax-weighted mean of V over it:
//   m = max_p LSE_p,  w_p = e^(LSE_p - m),
//   o = sum_p w_p o_p / sum_p w_p,  LSE = m + log sum_p w_p.
// A shard in which the query sees no key (LSE = -inf) adds nothing; a query
// that sees no key anywhere gets o = 0 and LSE = -inf, as in attn_fwd.
//
// HBM-bound: per (query, head) n_parts * (4 d + 4) bytes read and 2 d (+4)
// written. d/4 lanes own one (query, head) row, 4 columns each: 16-byte fp32
// loads, 8-byte bf16 stores, consecutive lane groups on consecutive heads of
// a query, so a wave reads and writes contiguous memory.
//
// The same identity merges the two pieces of each split unit of a balanced
// attn_fwd launch (workspace slots, 256 query rows of one head each).
#include "sdit_internal.h"

namespace sdit {
namespace {

constexpr int kThreads = 256;

// Combines n (<= NP) partial results of one (query, head) row at 4 columns:
// the merged bf16 quad, and the merged LSE in lse_out.
template <int NP>
__device__ __forceinline__ uint2 combine4(const float (&lse)[NP], const float4 (&v)[NP], float& lse_out) {
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NP; ++i) m = fmaxf(m, lse[i]);
  lse_out = -INFINITY;
  if (m == -INFINITY) return make_uint2(0u, 0u);   // +0 for a query that sees no key
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    if (lse[i] != -INFINITY) {
      const float w = expf(lse[i] - m);
      tot += w;
      acc.x += w * v[i].x;
      acc.y += w * v[i].y;
      acc.z += w * v[i].z;
      acc.w += w * v[i].w;
    }
  }
  const float inv = 1.0f / tot;
  const __bf16 b0 = (__bf16)(acc.x * inv), b1 = (__bf16)(acc.y * inv);
  const __bf16 b2 = (__bf16)(acc.z * inv), b3 = (__bf16)(acc.w * inv);
  lse_out = m + logf(tot);
  return make_uint2((uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16),
                    (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16));
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_merge_kernel(MergeParams p) {
  constexpr int LPR = D / 4;                 // lanes per (query, head)
  constexpr int PER_BLOCK = kThreads / LPR;
  const int64_t pair = (int64_t)blockIdx.x * PER_BLOCK + threadIdx.x / LPR;   // query * n_heads + head
  if (pair >= (int64_t)p.n_q * p.n_heads) return;
  const int c = (threadIdx.x % LPR) * 4;
  const int q = (int)(pair / p.n_heads), h = (int)(pair % p.n_heads);
  const int64_t li = (int64_t)h * p.n_q + q;
  const int64_t oi = pair * D + c;

  float lse[kMaxMergeParts];
  float4 v[kMaxMergeParts];
#pragma unroll
  for (int i = 0; i < kMaxMergeParts; ++i) {
    lse[i] = (i < p.n_parts) ? p.lse[i][li] : -INFINITY;
    v[i] = lse[i] != -INFINITY ? *reinterpret_cast<const float4*>(p.o[i] + oi) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float lse_out;
  *reinterpret_cast<uint2*>(p.out + oi) = combine4<kMaxMergeParts>(lse, v, lse_out);
  if (p.lse_out != nullptr && c == 0) p.lse_out[li] = lse_out;
}

// One block per PER_BLOCK rows of one split unit; blocks of slots an XCD
// does not use (j >= its r) and rows past n_q return at once.
template <int D>
__global__ __launch_bounds__(kThreads) void attn_split_merge_kernel(AttnParams p, uint16_t* out, float* lse_out) {
  constexpr int LPR = D / 4;
  constexpr int PER_BLOCK = kThreads / LPR;
  constexpr int BLOCKS_PER_UNIT = kAttnBQ / PER_BLOCK;
  const int unit_slot = blockIdx.x / BLOCKS_PER_UNIT;          // xcd * split_rmax + j
  const int xcd = unit_slot / p.split_rmax, j = unit_slot % p.split_rmax;
  const XcdUnits xu = xcd_units(p.n_qt * p.n_heads, xcd, p.cu_per_xcd, true);
  if (j >= xu.r) return;
  const int item = xu.u0 + xu.n - xu.r + j;
  const int head = item / p.n_qt, qt = item % p.n_qt;
  const int row = (blockIdx.x % BLOCKS_PER_UNIT) * PER_BLOCK + threadIdx.x / LPR;
  const int q_row = qt * kAttnBQ + row;
  if (q_row >= p.n_q) return;
  const int c = (threadIdx.x % LPR) * 4;
  float lse[2];
  float4 v[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t r = (int64_t)(2 * unit_slot + i) * kAttnBQ + row;
    lse[i] = p.ws_lse[r];
    v[i] = lse[i] != -INFINITY ? *reinterpret_cast<const float4*>(p.ws_o + r * D + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float l;
  *reinterpret_cast<uint2*>(out + ((int64_t)q_row * p.n_heads + head) * D + c) = combine4<2>(lse, v, l);
  if (lse_out != nullptr && c == 0) lse_out[(int64_t)head * p.n_q + q_row] = l;
}

template <int D>
hipError_t launch_split(const AttnParams& p, uint16_t* out, float* lse_out, hipStream_t stream) {
  constexpr int PER_BLOCK = kThreads / (D / 4);
  const int64_t blocks = (int64_t)kNumXcd * p.split_rmax * (kAttnBQ / PER_BLOCK);
  hipLaunchKernelGGL(attn_split_merge_kernel<D>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p, out, lse_out);
  return hipGetLastError();
}

template <int D>
hipError_t launch(const MergeParams& p, hipStream_t stream) {
  constexpr int PER_BLOCK = kThreads / (D / 4);
  const int64_t pairs = (int64_t)p.n_q * p.n_heads;
  const int64_t blocks = (pairs + PER_BLOCK - 1) / PER_BLOCK;
  hipLaunchKernelGGL(attn_merge_kernel<D>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_merge(const MergeParams& p, int head_dim, hipStream_t stream) {
  if (p.n_q == 0) return hipSuccess;
  return head_dim == 128 ? launch<128>(p, stream) : launch<64>(p, stream);
}

hipError_t launch_attn_split_merge(const AttnParams& p, uint16_t* out, float* lse_out, int head_dim,
                                   hipStream_t stream) {
  if (p.split_tile == 0 || p.split_rmax == 0) return hipSuccess;
  return head_dim == 128 ? launch_split<128>(p, out, lse_out, stream) : launch_split<64>(p, out, lse_out, stream);
}

}  // namespace sdit
