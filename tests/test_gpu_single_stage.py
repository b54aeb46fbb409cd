"""The prefetching attention schedule against a one-tile-at-a-time build.

libsdit_single_stage.so is the same library compiled with the attention
kernel's pipelined schedules (K double-buffered and V triple-buffered, tiles
loaded one or two steps ahead, half the waves a tile behind) replaced by a
schedule that loads one tile, waits, and computes it with every wave before
loading the next. Each wave does the same arithmetic on the same tiles in the
same order, so the two must agree bit for bit: any difference means a
prefetch read a tile buffer before it was complete or after it was
overwritten. (The Joy-face_change_optimized README, section 1.1, reports a
double-buffered prefetch that drifted from single buffering; this is the
guard against that failure.) bf16 and int8 caches, fine and coarse masks,
ragged and empty segments, V outside unit scale, several compaction passes,
and the balanced launch with a cut."""
import numpy as np
import pytest

from helpers import run_attn
from test_gpu_parity import CASES, _rand_case
from test_gpu_v_range import _case as v_range_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def single_stage():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import streaming_video_dit_amd as sdit
    return sdit.load_library(sdit.SINGLE_STAGE_LIB_PATH)


def _say(*a):
    print(*a, flush=True)


def _same(a, b, what):
    (oa, la), (ob, lb) = a, b
    assert np.array_equal(oa, ob), f"{what}: {(oa != ob).sum()} output elements differ"
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)), f"{what}: LSE differs"


@pytest.mark.parametrize("case", sorted(CASES))
def test_single_stage_bit_identical(case, single_stage):
    n_q, H, d, lens, dts, bq, bk, dens, empty = CASES[case]
    q, segs, mask = _rand_case(sum(map(ord, case)), n_q, H, d, lens, dts, bq, bk, dens, empty)
    _say("single stage vs pipelined", case)
    _same(run_attn(q, segs, mask, bq, bk), run_attn(q, segs, mask, bq, bk, library=single_stage), case)
    n_tiles = sum(-(-L // 64) for L in lens)
    if n_tiles >= 2:
        t = n_tiles // 2
        _same(run_attn(q, segs, mask, bq, bk, split_tile=t),
              run_attn(q, segs, mask, bq, bk, split_tile=t, library=single_stage), case + " cut")


@pytest.mark.parametrize("name", ["mixed_magnitudes", "int8_sigma_1e-5", "bf16_sigma_1e-6", "zero_tiles"])
def test_single_stage_bit_identical_v_range(name, single_stage):
    q, segs = v_range_case(name)
    lens = [s["k"].shape[0] for s in segs]
    mask = np.ones((-(-q.shape[0] // 128), sum(-(-L // 128) for L in lens)), np.uint8)
    _say("single stage vs pipelined, V range", name)
    _same(run_attn(q, segs, mask, 128, 128), run_attn(q, segs, mask, 128, 128, library=single_stage), name)


@pytest.mark.parametrize("dtype", ["bf16", "int8"])
def test_single_stage_bit_identical_several_passes(dtype, single_stage):
    lens = [1500, 67000] if dtype == "bf16" else [66000, 500]
    dts = ["bf16", "bf16"] if dtype == "bf16" else ["int8", "bf16"]
    q, segs, mask = _rand_case(73, 300, 2, 128, lens, dts, 128, 64, 0.6)
    _say("single stage vs pipelined, several passes", dtype)
    _same(run_attn(q, segs, mask, 128, 64), run_attn(q, segs, mask, 128, 64, library=single_stage), dtype)
