"""Windowed locality-sparse attention through the C ABI: the window
permutation against the oracle's index map (bit-exact, both directions), and
the chain raster -> window-major -> attention over 8 x 8-token blocks with
the locality mask -> raster against the oracle (tiny case on every element,
the page's clip geometry on sampled rows)."""
import numpy as np
import pytest

import workloads as W
from helpers import assert_attn_close, dev, empty_bf16, gpu_segments, host_u16
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print(*a, flush=True)


def _permute(x_bits, T, Hl, Wl, win, inverse):
    import torch
    import streaming_video_dit_amd as sdit
    n, H, d = x_bits.shape
    x = dev(x_bits)
    y = torch.full((n, H, d), -1, dtype=torch.int16, device="cuda")
    sdit.window_permute(x, y, T, Hl, Wl, H, d, win, inverse=inverse)
    torch.cuda.synchronize()
    return host_u16(y)


@pytest.mark.parametrize("shape", [(1, 8, 8, 8, 1, 64), (2, 16, 24, 4, 2, 64), (3, 8, 16, 2, 3, 128),
                                   (2, 96, 168, 8, 12, 128)])
def test_window_permute_bit_exact(shape):
    T, Hl, Wl, win, H, d = shape
    _say("window permute", shape)
    x = W.normal_bf16(sum(shape), 0, (T * Hl * Wl, H, d))
    order = oracle.window_order(T, Hl, Wl, win)
    y = _permute(x, T, Hl, Wl, win, False)
    assert np.array_equal(y, x[order])
    back = _permute(y, T, Hl, Wl, win, True)
    assert np.array_equal(back, x)


def _chain(cfg, inp, rows=None):
    """GPU: permute q, k, v -> attention -> inverse permute. Oracle: the same
    attention on the oracle-permuted inputs. Returns (gpu out, gpu lse, O, LSE)
    for the raster rows ``rows`` (all rows when None)."""
    import torch
    import streaming_video_dit_amd as sdit
    T, Hl, Wl, win, B = cfg.T, cfg.Hl, cfg.Wl, cfg.window, cfg.block
    n, H, d = inp.q.shape
    qw, kw, vw = (_permute(a, T, Hl, Wl, win, False) for a in (inp.q, inp.k, inp.v))
    segs, keep = gpu_segments([{"k": kw, "v": vw, "dtype": "bf16"}])
    m = dev(inp.mask)
    out_w = empty_bf16((n, H, d))
    lse_w = torch.full((H, n), float("nan"), dtype=torch.float32, device="cuda")
    sdit.attn_fwd(dev(qw), n, segs, m, B, B, H, d, out_w, lse_w)
    out = torch.full((n, H, d), -1, dtype=torch.int16, device="cuda")
    sdit.window_permute(out_w, out, T, Hl, Wl, H, d, win, inverse=True)
    torch.cuda.synchronize()
    out, lse_w = host_u16(out), lse_w.cpu().numpy()
    order = oracle.window_order(T, Hl, Wl, win)
    pos = np.empty_like(order)
    pos[order] = np.arange(n)                       # window-major position of every raster row
    rows = np.arange(n) if rows is None else np.asarray(rows)
    oseg = [{"k": inp.k[order], "v": inp.v[order], "dtype": "bf16"}]
    O, LSE = oracle.attention(inp.q[order], oseg, inp.mask, B, B, rows=pos[rows])
    return out[rows], lse_w[:, pos[rows]], O, LSE


def test_tiny_windowed_attention_every_element():
    cfg = W.WORKLOADS["tiny_local"]
    inp = W.make_inputs(cfg)
    _say("tiny windowed attention")
    out, lse, O, LSE = _chain(cfg, inp)
    e = assert_attn_close(out, lse, O, LSE, "tiny_local")
    _say(f"   max-abs {e[0]:.2e} ({e[2]:.2e} beyond half an ulp), rel-RMS {e[1]:.2e}")


def test_clip_windowed_attention_sampled():
    cfg = W.WORKLOADS["vsr_local"]
    inp = W.make_inputs(cfg)
    n = cfg.n_q
    rng = np.random.default_rng(cfg.seed)
    # corners and edges of both frames (windows with the fewest neighbours) and random rows
    hw = cfg.Hl * cfg.Wl
    fixed = {0, cfg.Wl - 1, hw - cfg.Wl, hw - 1, hw, n - 1, hw // 2 + cfg.Wl // 2}
    rows = np.array(sorted(fixed | set(rng.choice(n, size=24, replace=False).tolist())))
    _say("windowed attention, clip geometry", cfg.T, cfg.Hl, cfg.Wl, "rows", len(rows))
    out, lse, O, LSE = _chain(cfg, inp, rows)
    e = assert_attn_close(out, lse, O, LSE, "vsr_local")
    _say(f"   max-abs {e[0]:.2e} ({e[2]:.2e} beyond half an ulp), rel-RMS {e[1]:.2e}")
