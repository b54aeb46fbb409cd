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
#include "sdit_internal.h"

namespace sdit {
namespace {

constexpr int kThreads = 256;

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
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxMergeParts; ++i) {
    lse[i] = (i < p.n_parts) ? p.lse[i][li] : -INFINITY;
    m = fmaxf(m, lse[i]);
  }
  uint2 packed = make_uint2(0u, 0u);          // +0 for a query that sees no key
  float lse_out = -INFINITY;
  if (m != -INFINITY) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxMergeParts; ++i) {
      if (i < p.n_parts && lse[i] != -INFINITY) {
        const float w = expf(lse[i] - m);
        const float4 v = *reinterpret_cast<const float4*>(p.o[i] + oi);
        tot += w;
        acc.x += w * v.x;
        acc.y += w * v.y;
        acc.z += w * v.z;
        acc.w += w * v.w;
      }
    }
    const float inv = 1.0f / tot;
    const __bf16 b0 = (__bf16)(acc.x * inv), b1 = (__bf16)(acc.y * inv);
    const __bf16 b2 = (__bf16)(acc.z * inv), b3 = (__bf16)(acc.w * inv);
    packed = make_uint2((uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16),
                        (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16));
    lse_out = m + logf(tot);
  }
  *reinterpret_cast<uint2*>(p.out + oi) = packed;
  if (p.lse_out != nullptr && c == 0) p.lse_out[li] = lse_out;
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

}  // namespace sdit
