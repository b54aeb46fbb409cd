"""The online softmax's rare branches against the fp64 oracle, element by
element, and the pipelined schedule against the one-tile-at-a-time build.

The kernel takes a tile's exponentials with the running row max as it stands
and computes the tile's row max only when some lane's sum of P reaches 2^8
(only then may a P have passed the lazy-rescale threshold of 2^8), or while a
row has seen nothing. Scores here are laid out tile by tile (64 keys) so that
each branch runs on purpose, in log2 units of score * scale * log2(e):

  growing  every tile lifts the row max by 10: every tile rescales O and l and
           takes its exponentials again;
  crowded  one key of the first tile sets the max at 20, the next three tiles
           hold only keys at 27 (each P = 2^7, so a lane's 32 keys sum to 2^12
           without any P passing 2^8): the row max is computed and no rescale
           happens; a last tile at 29 then rescales;
  falling  scores fall by 12 per tile: the first tile's max stays, late P
           underflow toward 0.

Every case runs on bf16 and int8 caches, head_dim 64 and 128, and with
128-row and 16-row q-blocks (the kernel with the per-q-block bias)."""
import numpy as np
import pytest

import workloads as W
from helpers import assert_attn_close, run_attn
import oracle

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634

# per-tile score levels (log2 units) and the keys of the first tile that
# differ from the rest of it: (key index, level)
LAYOUTS = {
    "growing": ([0, 10, 20, 30, 40, 50], None),
    "crowded": ([0, 27, 27, 27, 29], (0, 20)),
    "falling": ([30, 18, 6, -6, -18, -30], None),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print(*a, flush=True)


def _case(layout: str, dtype: str, d: int, seed: int):
    levels, first = LAYOUTS[layout]
    n_q, H = 96, 2
    n_k = 64 * len(levels)
    rng = np.random.default_rng([seed, 1])
    # q near the all-ones direction, so q . k ~ d * y for a key row of y's
    q = 1.0 + 0.05 * rng.standard_normal((n_q, H, d))
    # key row values y such that sqrt(d) * log2(e) * y is the tile's level
    lev = np.repeat(np.asarray(levels, np.float64), 64)
    if first is not None:
        lev[first[0]] = first[1]
    y = lev / (np.sqrt(d) * LOG2E)
    k = y[:, None, None] * (1.0 + 0.02 * rng.standard_normal((n_k, H, d)))
    v = rng.standard_normal((n_k, H, d))
    qb = W._f32_to_bf16_bits(q.astype(np.float32))
    kb = W._f32_to_bf16_bits(k.astype(np.float32))
    vb = W._f32_to_bf16_bits(v.astype(np.float32))
    if dtype == "int8":
        ck, sk = oracle.kv_quant_int8(kb)
        cv, sv = oracle.kv_quant_int8(vb)
        segs = [{"k": ck, "v": cv, "k_scale": sk, "v_scale": sv, "dtype": "int8"}]
    else:
        segs = [{"k": kb, "v": vb, "dtype": "bf16"}]
    return qb, segs, n_q, n_k


@pytest.mark.parametrize("bq", [128, 16])
@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("dtype", ["bf16", "int8"])
@pytest.mark.parametrize("layout", sorted(LAYOUTS))
def test_softmax_branches_match_the_oracle(layout, dtype, d, bq):
    q, segs, n_q, n_k = _case(layout, dtype, d, seed=sum(map(ord, layout)) + d)
    mask = np.ones((-(-n_q // bq), -(-n_k // bq)), np.uint8)
    what = f"{layout} {dtype} d{d} bq{bq}"
    _say("softmax branches", what)
    out, lse = run_attn(q, segs, mask, bq, bq)
    O, LSE = oracle.attention(q, segs, mask, bq, bq)
    e = assert_attn_close(out, lse, O, LSE, what)
    _say(f"   max-abs {e[0]:.2e} ({e[2]:.2e} beyond half an ulp), rel-RMS {e[1]:.2e}")


@pytest.mark.parametrize("dtype", ["bf16", "int8"])
@pytest.mark.parametrize("layout", sorted(LAYOUTS))
def test_softmax_branches_single_stage_bit_identical(layout, dtype):
    import streaming_video_dit_amd as sdit
    single = sdit.load_library(sdit.SINGLE_STAGE_LIB_PATH)
    q, segs, n_q, n_k = _case(layout, dtype, 128, seed=7)
    mask = np.ones((-(-n_q // 128), -(-n_k // 128)), np.uint8)
    _say("softmax branches, single stage vs pipelined", layout, dtype)
    oa, la = run_attn(q, segs, mask, 128, 128)
    ob, lb = run_attn(q, segs, mask, 128, 128, library=single)
    assert np.array_equal(oa, ob), f"{(oa != ob).sum()} output elements differ"
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32))
