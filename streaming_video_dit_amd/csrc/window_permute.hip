// Token reordering between raster order (t, h, w) and the window-major order
// of windowed sparse attention (t, h / win, w / win, h % win, w % win),
// gfx950. FlashVSR deployment notes, spatial tiling section: an attention
// block is a window of 8 x 8 tokens, so for a block of block-sparse attention
// to be a spatial window the tokens are grouped window by window.
//
// HBM-bound copy: every token's row of n_heads * head_dim bf16 moves once
// (2 * 2 * n_heads * head_dim bytes per token). Threads own 16-byte chunks;
// consecutive threads walk one row, so both the read of a source row and the
// write of a destination row are contiguous.
#include "sdit_internal.h"

namespace sdit {
namespace {

constexpr int kThreads = 256;
constexpr int kTokensPerBlock = 8;

__global__ __launch_bounds__(kThreads) void window_permute_kernel(PermuteParams p) {
  const int hw = p.Hl * p.Wl, ww = p.win * p.win, nwx = p.Wl / p.win;
  const int64_t tok0 = (int64_t)blockIdx.x * kTokensPerBlock;
  const int n = (int)min<int64_t>(kTokensPerBlock, p.n_tok - tok0);
  for (int i = threadIdx.x; i < n * p.row_chunks; i += kThreads) {
    const int j = (int)tok0 + i / p.row_chunks;   // destination token
    const int c = i % p.row_chunks;
    const int t = j / hw, rem = j % hw;
    int src;
    if (!p.inverse) {
      // j is window-major: the token of window rem / ww, position rem % ww inside it
      const int wi = rem / ww, pi = rem % ww;
      const int h = (wi / nwx) * p.win + pi / p.win;
      const int w = (wi % nwx) * p.win + pi % p.win;
      src = t * hw + h * p.Wl + w;
    } else {
      // j is raster: the window-major position of token (h, w)
      const int h = rem / p.Wl, w = rem % p.Wl;
      src = t * hw + ((h / p.win) * nwx + w / p.win) * ww + (h % p.win) * p.win + w % p.win;
    }
    const uint4* s = reinterpret_cast<const uint4*>(p.x) + (int64_t)src * p.row_chunks + c;
    uint4* d = reinterpret_cast<uint4*>(p.y) + (int64_t)j * p.row_chunks + c;
    *d = *s;
  }
}

}  // namespace

hipError_t launch_window_permute(const PermuteParams& p, hipStream_t stream) {
  if (p.n_tok == 0) return hipSuccess;
  const int64_t blocks = (p.n_tok + kTokensPerBlock - 1) / kTokensPerBlock;
  hipLaunchKernelGGL(window_permute_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sdit
