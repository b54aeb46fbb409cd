"""Several query chunks in one forward (CPU only).

The chunk-causal block mask over [cache | chunk 0 | ... | chunk C-1] must give
every chunk exactly the attention it would get alone over the cache and the
chunks up to its own (Wave Forcing summary: block-causal attention, later
chunks read earlier ones); padding rows between chunks are extra queries whose
results are not used.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention


@pytest.mark.parametrize("name", ["tiny_chunks"])
def test_chunk_causal_mask_equals_per_chunk_attention(name):
    cfg = W.WORKLOADS[name]
    inp = W.make_inputs(cfg)
    segs = [{"k": k, "v": v, "dtype": "bf16"} for k, v in zip(inp.cache_k, inp.cache_v)]
    segs += [{"k": inp.k[W.chunk_rows(cfg, c)], "v": inp.v[W.chunk_rows(cfg, c)], "dtype": "bf16"}
             for c in range(cfg.n_chunks)]
    O, LSE = attention(inp.q, segs, inp.mask, cfg.block, cfg.block)
    for c in range(cfg.n_chunks):
        r = W.chunk_rows(cfg, c)
        own = segs[:cfg.n_cached + c + 1]
        n_kb = sum(-(-s["k"].shape[0] // cfg.block) for s in own)
        q = inp.q[r]
        dense = np.ones((-(-q.shape[0] // cfg.block), n_kb), np.uint8)
        Oc, Lc = attention(q, own, dense, cfg.block, cfg.block)
        np.testing.assert_allclose(O[r], Oc, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(LSE[:, r], Lc, rtol=1e-12)


def test_chunk_layout_and_mask_shape():
    cfg = W.WORKLOADS["wave_chunks"]
    assert cfg.chunk_tokens == 4680 and cfg.chunk_slot == 4736 and cfg.n_q == 4 * 4736
    assert cfg.n_cached == 2 and cfg.seg_lens[2:] == [4680] * 4
    m = W.make_mask(cfg)
    assert m.shape == (4 * 37, 4 + 110 + 4 * 37)
    # chunk c's q-blocks keep the cache and chunks 0..c, nothing later
    for c in range(4):
        rows = m[c * 37:(c + 1) * 37]
        assert np.all(rows[:, :114 + 37 * (c + 1)] == 1) and np.all(rows[:, 114 + 37 * (c + 1):] == 0)
    for c in range(4):
        r = W.chunk_rows(cfg, c)
        assert r.start % cfg.block == 0 and r.stop - r.start == 4680
