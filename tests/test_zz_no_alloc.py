"""sdit_attn_fwd_balanced_static (the allocation-free balanced attention, for
callers that cannot allocate device memory) against sdit_attn_fwd_balanced
with a caller workspace, through the C ABI: bit-identical outputs and LSE
(same kernels, same plan). Two calls in a row, the second with a smaller
input and a smaller cut, so that the library's scratch still holds the
first call's partials when the second one runs."""
import numpy as np
import pytest

import workloads as W
from helpers import dev, gpu_segments, host_u16
from test_gpu_parity import _rand_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print(*a, flush=True)


def _both(q_bits, oracle_segs, mask, bq, bk, split_tile):
    import torch
    import streaming_video_dit_amd as sdit
    n_q, H, d = q_bits.shape
    q = dev(q_bits)
    segs, keep = gpu_segments(oracle_segs)
    m = dev(mask.astype(np.uint8))
    res = []
    for form in ("workspace", "static"):
        out = torch.full((n_q, H, d), -1, dtype=torch.int16, device="cuda")
        lse = torch.full((H, n_q), float("nan"), dtype=torch.float32, device="cuda")
        if form == "workspace":
            ws = torch.full((sdit.attn_workspace_bytes(d),), 0xFF, dtype=torch.uint8, device="cuda")
            sdit.attn_fwd_balanced(q, n_q, segs, m, bq, bk, H, d, out, ws, lse, split_tile=split_tile)
        else:
            sdit.attn_fwd_balanced_static(q, n_q, segs, m, bq, bk, H, d, out, lse, split_tile=split_tile)
        torch.cuda.synchronize()
        res.append((host_u16(out), lse.cpu().numpy()))
    return res


def _check(res, what):
    (oa, la), (ob, lb) = res
    assert np.array_equal(oa, ob), f"{what}: {(oa != ob).sum()} outputs differ"
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)), f"{what}: LSE differs"
    assert np.all((oa & 0x7F80) != 0x7F80), f"{what}: non-finite output"


def test_static_scratch_matches_workspace_twice():
    # first call: the Large-DiT chunk through the library's plan (a cut on
    # every XCD, the largest scratch of the workloads)
    cfg = W.WORKLOADS["large_dit"]
    inp = W.make_inputs(cfg)
    segs = [{"k": k, "v": v, "dtype": "bf16"} for k, v in zip(inp.cache_k, inp.cache_v)]
    segs.append({"k": inp.k, "v": inp.v, "dtype": "bf16"})
    _say("static scratch: large_dit, library plan")
    _check(_both(inp.q, segs, inp.mask, cfg.block, cfg.block, -1), "large_dit")
    # second call, smaller: int8 + bf16 segments, 16-row blocks, forced cut
    q, segs2, mask = _rand_case(41, 300, 2, 128, [90, 300], ["int8", "bf16"], 16, 32, 0.6, (3,))
    _say("static scratch: small case, cut at tile 3")
    _check(_both(q, segs2, mask, 16, 32, 3), "small case")
