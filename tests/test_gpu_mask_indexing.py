"""Mask and block indexing checked bit for bit.

With q = 0 every visible key scores 0 and gets the same weight, and a key the
mask drops gets none. Key j of k-block kb carries, in head kb // d, a one-hot
V on column kb % d (zero V in every other head). The output of query i at
(head h, column c) is then (visible keys of k-block h d + c) / (all visible
keys of i's q-block): nonzero exactly where the mask keeps that k-block for
qb(i). So the set of nonzero outputs is the mask expansion itself, and it is
compared bit for bit with the oracle's. This is the exact check of
mask/block indexing (a kept tile dropped, a dropped tile kept or a tile
shifted by one block changes the pattern); it follows the FlashVSR
deployment notes (Block-Sparse-Attention section), which prove the sparse
path runs by a lower-triangular block mask against brute force. The values
themselves, count ratios, must be within one bf16 ulp of the oracle's, and
LSE = ln(visible keys) within 1e-3.

Covers block sizes 16 to 128 for q-blocks and k-blocks, ragged and empty
segments, int8 + bf16 mixes, empty q-block rows, cuts of the balanced launch,
and more than 1024 candidate 64-key tiles per workgroup (several compaction
passes)."""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import ordered, run_attn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print(*a, flush=True)


def onehot_case(seed, n_q, d, lens, dtypes, bq, bk, density, empty_rows=()):
    """q = 0; K random; V one-hot by k-block as described above; a random
    block mask. Returns (q bits, oracle segments, mask, heads)."""
    n_kb = sum(-(-L // bk) for L in lens)
    H = max(1, -(-n_kb // d))
    q = np.zeros((n_q, H, d), np.uint16)
    segs, base = [], 0
    one = np.uint16(0x3F80)   # bf16 1.0
    for i, (L, dt) in enumerate(zip(lens, dtypes)):
        k = W.normal_bf16(seed, 10 + i, (L, H, d))
        v = np.zeros((L, H, d), np.uint16)
        kb = base + np.arange(L) // bk          # k-block of every key of this segment
        v[np.arange(L), kb // d, kb % d] = one
        base += -(-L // bk)
        if dt == "int8":
            ck, sk = oracle.kv_quant_int8(k)
            cv, sv = oracle.kv_quant_int8(v)
            segs.append({"k": ck, "v": cv, "k_scale": sk, "v_scale": sv, "dtype": "int8"})
        else:
            segs.append({"k": k, "v": v, "dtype": "bf16"})
    rng = np.random.default_rng([seed, 100])
    mask = (rng.random((-(-n_q // bq), n_kb)) < density).astype(np.uint8)
    for r in empty_rows:
        mask[r] = 0
    return q, segs, mask, H


CASES = {
    # name: (n_q, d, segment lengths, dtypes, block_q, block_k, density, empty q-block rows)
    "b128_three_segments": (300, 128, [77, 300, 130], ["bf16"] * 3, 128, 128, 0.6, ()),
    "b64_int8_mix": (257, 128, [64, 200, 257], ["int8", "int8", "bf16"], 64, 64, 0.5, (2,)),
    "b32_ragged_empty_segment": (200, 128, [50, 0, 150, 33], ["bf16", "bf16", "int8", "bf16"], 32, 32, 0.5, (1,)),
    "b16_sixteen_slots": (300, 128, [90, 300], ["bf16", "bf16"], 16, 16, 0.4, (3, 12)),
    "q16_k128": (270, 64, [100, 270], ["int8", "bf16"], 16, 128, 0.5, (0,)),
    "q128_k16_two_heads": (256, 128, [1000, 2000], ["bf16", "int8"], 128, 16, 0.3, ()),
    "eight_segments": (130, 128, [1, 63, 64, 65, 0, 128, 3, 130], ["bf16", "int8"] * 4, 128, 64, 0.7, ()),
    "d64_b32": (190, 64, [33, 190, 64], ["bf16", "bf16", "int8"], 32, 32, 0.6, ()),
}


def _check(case, out, lse, O, LSE):
    got_nz = (out & 0x7FFF) != 0
    ref_nz = O != 0
    bad = int((got_nz != ref_nz).sum())
    assert bad == 0, f"{case}: {bad} outputs differ from the mask expansion in being zero"
    ref_bits = oracle.f64_to_bf16(O)
    ulps = np.abs(ordered(out) - ordered(ref_bits))
    assert int(ulps.max()) <= 1, f"{case}: count ratio off by {int(ulps.max())} ulp"
    fin = np.isfinite(LSE)
    assert np.array_equal(np.isfinite(lse), fin) and np.all(np.isneginf(lse[~fin]))
    if fin.any():
        assert float(np.abs(lse[fin] - LSE[fin]).max()) <= 1e-3
    return int(ref_nz.sum()), int(ulps.max())


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("launch", ["plain", "cut"])
def test_mask_expansion_bit_exact(case, launch):
    n_q, d, lens, dts, bq, bk, dens, empty = CASES[case]
    q, segs, mask, H = onehot_case(sum(map(ord, case)), n_q, d, lens, dts, bq, bk, dens, empty)
    n_tiles = sum(-(-L // 64) for L in lens)
    split = None if launch == "plain" else max(1, n_tiles // 2)
    _say("mask indexing", case, launch, "heads", H, "mask", mask.shape, "kept", int(mask.sum()))
    out, lse = run_attn(q, segs, mask, bq, bk, split_tile=split)
    O, LSE = oracle.attention(q, segs, mask, bq, bk)
    nz, u = _check(case, out, lse, O, LSE)
    _say(f"   {nz} nonzero outputs match the mask expansion; values within {u} ulp")


@pytest.mark.parametrize("launch", ["plain", "cut"])
def test_mask_expansion_over_several_compaction_passes(launch):
    # 70000 keys = 1094 candidate 64-key tiles: two compaction passes per
    # workgroup; 547 k-blocks of 128 keys spread over 5 heads of d = 128
    q, segs, mask, H = onehot_case(97, 256, 128, [70000], ["bf16"], 128, 128, 0.7)
    split = None if launch == "plain" else 700
    _say("mask indexing, several passes", launch, "heads", H, "mask", mask.shape)
    out, lse = run_attn(q, segs, mask, 128, 128, split_tile=split)
    O, LSE = oracle.attention(q, segs, mask, 128, 128)
    nz, u = _check("passes", out, lse, O, LSE)
    _say(f"   {nz} nonzero outputs match the mask expansion; values within {u} ulp")


def test_lower_triangular_block_mask_bit_exact():
    # the pages' own check of the sparse path: a lower-triangular block mask
    n, bq = 640, 64
    q, segs, _, H = onehot_case(98, n, 128, [n], ["bf16"], bq, bq, 1.0)
    nb = -(-n // bq)
    mask = np.tril(np.ones((nb, nb), np.uint8))
    out, lse = run_attn(q, segs, mask, bq, bq)
    O, LSE = oracle.attention(q, segs, mask, bq, bq)
    _check("lower triangular", out, lse, O, LSE)
    # row block r sees exactly blocks 0..r
    for r in range(nb):
        rows = slice(r * bq, min(n, (r + 1) * bq))
        nz = (out[rows, 0, :nb] & 0x7FFF) != 0
        assert np.all(nz[:, :r + 1]) and not np.any(nz[:, r + 1:])
