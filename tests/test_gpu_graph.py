"""The C-ABI calls allocate nothing, synchronise nothing and launch only on
the stream they are given, so a whole layer-chunk step (qknorm_rope3d,
kv_quant_int8 of a history cache, attn_fwd over [text bf16 | history int8 |
current bf16]) can be captured into a HIP graph. Each replay, with unrelated
eager work and synchronisations between replays, must reproduce the eager
results bit for bit (the kernels are deterministic). The attention runs
either as attn_fwd or as attn_fwd_balanced with a cut (attention kernel, then
the merge of the pieces through the caller's workspace)."""
import numpy as np
import pytest

import workloads as W
from helpers import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("launch", ["plain", "balanced"])
def test_step_captured_in_a_graph_replays_like_eager(launch):
    import torch
    import streaming_video_dit_amd as sdit

    T, Hl, Wl, t0, H, d = 2, 15, 20, 3, 2, 128
    n = T * Hl * Wl
    dt, dh, dw = W.rope_split(d)
    seed = 91
    q_in, k_in, v = (dev(W.normal_bf16(seed, i, (n, H, d))) for i in range(3))
    gq, gk = (dev(W.uniform_f32(seed, 3 + i, (d,), 0.5, 1.5)) for i in range(2))
    tk, tv = (dev(W.normal_bf16(seed, 5 + i, (64, H, d))) for i in range(2))
    L = 1200
    hk, hv = (dev(W.normal_bf16(seed, 7 + i, (L, H, d), outlier_p=0.01, outlier_tid=20 + i)) for i in range(2))
    q, k = torch.empty_like(q_in), torch.empty_like(k_in)
    ck, cv = (torch.empty((L, H, d), dtype=torch.int8, device="cuda") for _ in range(2))
    sk, sv = (torch.empty((L, H), dtype=torch.float32, device="cuda") for _ in range(2))
    out = torch.empty((n, H, d), dtype=torch.int16, device="cuda")
    lse = torch.empty((H, n), dtype=torch.float32, device="cuda")
    nkb = -(-64 // 128) + -(-L // 128) + -(-n // 128)
    mask = dev(np.ones((-(-n // 128), nkb), np.uint8))
    segs = sdit.make_segments([dict(k=tk, v=tv, len=64), dict(k=ck, v=cv, k_scale=sk, v_scale=sv, len=L,
                                                               dtype=sdit.SDIT_INT8), dict(k=k, v=v, len=n)])
    ws = torch.full((sdit.attn_workspace_bytes(d),), 0xFF, dtype=torch.uint8, device="cuda")

    def step():
        sdit.qknorm_rope3d(q_in, k_in, q, k, gq, gk, T, Hl, Wl, t0, H, d, dt, dh, dw)
        sdit.kv_quant_int8(hk, ck, sk, L, H, d)
        sdit.kv_quant_int8(hv, cv, sv, L, H, d)
        if launch == "plain":
            sdit.attn_fwd(q, n, segs, mask, 128, 128, H, d, out, lse)
        else:   # 30 key tiles, 6 units: every unit cut at tile 12
            sdit.attn_fwd_balanced(q, n, segs, mask, 128, 128, H, d, out, ws, lse, split_tile=12)

    outputs = (q, k, ck, cv, sk, sv, out, lse)
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outputs]

    graph = torch.cuda.CUDAGraph()
    capture = torch.cuda.Stream()
    capture.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(capture):
        with torch.cuda.graph(graph, stream=capture):
            step()
    torch.cuda.current_stream().wait_stream(capture)
    torch.cuda.synchronize()

    a = torch.randn(512, 512, device="cuda")
    for rep in range(3):
        for t in outputs:
            t.fill_(7)          # the replay has to write every output again
        a = a @ a.t() * 1e-3     # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("q", "k", "ck", "cv", "sk", "sv", "out", "lse"), outputs, eager):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager step"
