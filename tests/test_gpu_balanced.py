"""Parity of sdit_attn_fwd_balanced (the attention launch with its last
partial wave of work units cut into head and tail pieces) with the fp64
oracle, at the bars of the plain attention path: relative RMS 1e-2 of the
unrounded result, max-abs 4e-3 where |ref| < 1 and 4e-3 beyond half a bf16
ulp above that, LSE within 1e-3, rows without a visible key exactly +0 / -inf. The small cases force the cut at the first, a middle
and the last key tile (every unit of those cases is a piece: fewer units
than CUs); the full-size workloads run the library's own plan inside
test_full_size_hot_path_sampled."""
import numpy as np
import pytest

import oracle
from helpers import assert_attn_close, bf16_to_float, run_attn
from test_gpu_parity import CASES, _rand_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print(*a, flush=True)


def _n_tiles(segs):
    return sum(-(-s["k"].shape[0] // 64) for s in segs)


_ORACLE = {}


def _case(case):
    if case not in _ORACLE:
        n_q, H, d, lens, dts, bq, bk, dens, empty = CASES[case]
        q, segs, mask = _rand_case(sum(map(ord, case)), n_q, H, d, lens, dts, bq, bk, dens, empty)
        _ORACLE[case] = (q, segs, mask, oracle.attention(q, segs, mask, bq, bk))
    return _ORACLE[case]


@pytest.mark.parametrize("where", ["first", "middle", "last"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_balanced_small_cases(case, where):
    n_q, H, d, lens, dts, bq, bk, dens, empty = CASES[case]
    q, segs, mask, (O, LSE) = _case(case)
    n = _n_tiles(segs)
    if n < 2:
        pytest.skip("a single key tile cannot be cut")
    t = {"first": 1, "middle": n // 2, "last": n - 1}[where]
    _say("balanced", case, "cut at tile", t, "of", n)
    out, lse = run_attn(q, segs, mask, bq, bk, split_tile=t)
    e = assert_attn_close(out, lse, O, LSE, f"{case} cut {t}")
    _say(f"   max-abs {e[0]:.2e} ({e[2]:.2e} beyond half an ulp), rel-RMS {e[1]:.2e}")
    for r in empty:
        rows = slice(r * bq, min(n_q, (r + 1) * bq))
        assert np.all(out[rows] == 0)
        assert np.all(lse[:, rows] == -np.inf)


@pytest.mark.parametrize("t", [700, 1024, 1060])
def test_balanced_cut_inside_and_at_a_compaction_pass(t):
    """More than 1024 candidate tiles: the kept-tile list is built in passes
    of 1024 from the piece's first tile, so a cut inside the first pass, on
    its boundary and inside the second pass all start a pass mid-range."""
    q, segs, mask = _rand_case(71, 300, 2, 64, [1000, 69000], ["bf16", "bf16"], 128, 64, 0.6)
    assert _n_tiles(segs) == 1095
    O, LSE = oracle.attention(q, segs, mask, 128, 64)
    _say("balanced long cache, cut at", t, "of", _n_tiles(segs))
    out, lse = run_attn(q, segs, mask, 128, 64, split_tile=t)
    e = assert_attn_close(out, lse, O, LSE, f"long cache cut {t}")
    _say(f"   max-abs {e[0]:.2e} ({e[2]:.2e} beyond half an ulp), rel-RMS {e[1]:.2e}")


def test_balanced_without_a_cut_is_attn_fwd():
    """split_tile 0 (and a plan that finds nothing to cut) launch the plain
    kernel: bit-identical outputs and LSE."""
    q, segs, mask, _ = _case("d128_int8_mix")
    n_q, H, d, lens, dts, bq, bk, dens, empty = CASES["d128_int8_mix"]
    a, la = run_attn(q, segs, mask, bq, bk)
    b, lb = run_attn(q, segs, mask, bq, bk, split_tile=0)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_balanced_every_cut_position():
    """Every cut from the first to the last key tile of a three-segment case
    (cuts on both sides of each segment boundary) meets the oracle's bar.
    The cut regroups the sum over keys, and each piece rounds its
    probabilities to fp16 against its own running maximum, so results differ
    from the uncut kernel's by a few rounding steps; the differences are
    printed for reference."""
    q, segs, mask, (O, LSE) = _case("d128_ragged_3seg")
    n_q, H, d, lens, dts, bq, bk, dens, empty = CASES["d128_ragged_3seg"]
    a, la = run_attn(q, segs, mask, bq, bk)
    fa = bf16_to_float(a)
    for t in range(1, _n_tiles(segs)):
        b, lb = run_attn(q, segs, mask, bq, bk, split_tile=t)
        e = assert_attn_close(b, lb, O, LSE, f"cut {t}")
        d_o = float(np.abs(fa - bf16_to_float(b)).max())
        d_lse = float(np.abs(la - lb).max())
        _say(f"   cut {t}: beyond half an ulp {e[2]:.2e}; vs uncut: output {d_o:.2e}, LSE {d_lse:.2e}")


def test_balanced_workspace_reused_by_a_smaller_call():
    """Two calls in a row share one workspace; the second (fewer work units,
    a different cut) must not read what the first left behind."""
    import torch
    import streaming_video_dit_amd as sdit
    from helpers import dev, gpu_segments, host_u16
    ws = torch.full((sdit.attn_workspace_bytes(128),), 0xFF, dtype=torch.uint8, device="cuda")
    for case, t in (("d128_sparse", 3), ("d128_ragged_3seg", 5)):
        n_q, H, d, lens, dts, bq, bk, dens, empty = CASES[case]
        q, segs, mask, (O, LSE) = _case(case)
        gs, keep = gpu_segments(segs)
        out = torch.full((n_q, H, d), -1, dtype=torch.int16, device="cuda")
        lse = torch.full((H, n_q), float("nan"), dtype=torch.float32, device="cuda")
        sdit.attn_fwd_balanced(dev(q), n_q, gs, dev(mask), bq, bk, H, d, out, ws, lse, split_tile=t)
        torch.cuda.synchronize()
        assert_attn_close(host_u16(out), lse.cpu().numpy(), O, LSE, f"{case} after reuse")


def test_balanced_without_lse():
    q, segs, mask, (O, LSE) = _case("d64_b32_int8")
    n_q, H, d, lens, dts, bq, bk, dens, empty = CASES["d64_b32_int8"]
    out, _ = run_attn(q, segs, mask, bq, bk, lse=False, split_tile=2)
    out2, lse2 = run_attn(q, segs, mask, bq, bk, split_tile=2)
    assert np.array_equal(out, out2)
    assert_attn_close(out2, lse2, O, LSE, "d64_b32_int8 cut 2")
