"""Pins for the oracle's merge of attention results over disjoint key sets
(CPU only).

The merge is pinned against the definition of attention itself: attention
over a cache split into groups of segments, merged, must equal attention over
the whole cache (dense and block-sparse masks, ragged and int8 segments, rows
that see nothing in some part or in every part). Further: one part is the
identity, the order of the parts does not matter, and an empty part adds
nothing.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention, attention_merge, kv_quant_int8


def _segments(seed, lens, dtypes, H, d):
    segs = []
    for i, (L, dt) in enumerate(zip(lens, dtypes)):
        k = W.normal_bf16(seed, 10 + 2 * i, (L, H, d), outlier_p=0.01, outlier_tid=50 + i)
        v = W.normal_bf16(seed, 11 + 2 * i, (L, H, d), outlier_p=0.01, outlier_tid=60 + i)
        if dt == "int8":
            ck, sk = kv_quant_int8(k)
            cv, sv = kv_quant_int8(v)
            segs.append({"k": ck, "v": cv, "k_scale": sk, "v_scale": sv, "dtype": "int8"})
        else:
            segs.append({"k": k, "v": v, "dtype": "bf16"})
    return segs


def _columns(lens, bk, first, last):
    """Mask columns of segments first..last-1 (k-blocks restart per segment)."""
    starts = np.cumsum([0] + [-(-L // bk) for L in lens])
    return slice(int(starts[first]), int(starts[last]))


def _split_attention(q, segs, mask, bq, bk, cuts):
    lens = [s["k"].shape[0] for s in segs]
    bounds = [0] + list(cuts) + [len(segs)]
    parts = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        parts.append(attention(q, segs[a:b], mask[:, _columns(lens, bk, a, b)], bq, bk))
    return parts


CASES = [
    # seed, n_q, H, d, segment lengths, dtypes, block, density, cuts, empty q-block rows
    (1, 96, 2, 64, [40, 70, 33], ["bf16", "bf16", "bf16"], 16, 1.0, [1], ()),
    (2, 130, 2, 128, [64, 129, 5, 77], ["int8", "bf16", "int8", "bf16"], 32, 0.6, [1, 3], (2,)),
    (3, 64, 1, 64, [100, 60], ["bf16", "int8"], 16, 0.3, [1], (0, 3)),
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{c[0]}" for c in CASES])
def test_merged_parts_equal_attention_over_the_whole_cache(case):
    seed, n_q, H, d, lens, dts, B, dens, cuts, empty = case
    q = W.normal_bf16(seed, 0, (n_q, H, d))
    segs = _segments(seed, lens, dts, H, d)
    nqb, nkb = -(-n_q // B), sum(-(-L // B) for L in lens)
    mask = (np.random.default_rng([seed, 5]).random((nqb, nkb)) < dens).astype(np.uint8)
    for r in empty:
        mask[r] = 0
    O, LSE = attention(q, segs, mask, B, B)
    parts = _split_attention(q, segs, mask, B, B, cuts)
    # the split really separates rows: some row sees nothing in some part
    if dens < 1.0:
        assert any(np.isneginf(L).any() and np.isfinite(L).any() for _, L in parts)
    Om, Lm = attention_merge(parts)
    np.testing.assert_allclose(Om, O, rtol=1e-12, atol=1e-14)
    fin = np.isfinite(LSE)
    np.testing.assert_allclose(Lm[fin], LSE[fin], rtol=1e-12)
    assert np.array_equal(np.isneginf(Lm), np.isneginf(LSE))
    for r in empty:
        rows = slice(r * B, min(n_q, (r + 1) * B))
        assert np.all(Om[rows] == 0) and np.all(np.isneginf(Lm[:, rows]))


def test_one_part_is_the_identity_and_order_does_not_matter():
    q = W.normal_bf16(7, 0, (48, 2, 64))
    segs = _segments(7, [30, 50, 20], ["bf16", "int8", "bf16"], 2, 64)
    mask = np.ones((3, 2 + 4 + 2), np.uint8)
    mask[1, 2:6] = 0
    O, LSE = attention(q, segs, mask, 16, 16)
    O1, L1 = attention_merge([(O, LSE)])
    np.testing.assert_array_equal(O1, O)
    np.testing.assert_array_equal(L1, LSE)
    parts = _split_attention(q, segs, mask, 16, 16, [1, 2])
    Oa, La = attention_merge(parts)
    Ob, Lb = attention_merge(parts[::-1])
    np.testing.assert_allclose(Ob, Oa, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(Lb, La, rtol=1e-14)


def test_empty_part_adds_nothing():
    q = W.normal_bf16(8, 0, (32, 1, 64))
    segs = _segments(8, [40, 0, 24], ["bf16", "bf16", "bf16"], 1, 64)
    mask = np.ones((2, 3 + 0 + 2), np.uint8)
    O, LSE = attention(q, segs, mask, 16, 16)
    parts = _split_attention(q, segs, mask, 16, 16, [1, 2])
    assert np.all(parts[1][0] == 0) and np.all(np.isneginf(parts[1][1]))
    Om, Lm = attention_merge(parts)
    np.testing.assert_allclose(Om, O, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(Lm, LSE, rtol=1e-12)
    none = [(np.zeros_like(O), np.full_like(LSE, -np.inf))] * 2
    Oz, Lz = attention_merge(none)
    assert np.all(Oz == 0) and np.all(np.isneginf(Lz))
