"""Attention with V far from unit scale, against the fp64 oracle.

The probability-weighted sum of V runs as an fp16 product; each staged 64-key
V tile carries a power-of-two exponent so that fp16 holds it. These cases
put V where a fixed fp16 staging would lose it: int8 rows whose scales sit
below fp16's normal range (V of standard deviation 1e-3 .. 1e-5), bf16 V
below fp16's subnormal step (1e-6, 1e-9), bf16 V near the fp16 ceiling
(|v| up to 65280) and past it (1e6, 1e30), segments whose magnitudes differ by
many orders (the exponent changes from tile to tile inside one row), and
all-zero V tiles. Bars: relative RMS 1e-2 and LSE within 1e-3 as everywhere;
the max-abs bar (4e-3 where |ref| < 1, 4e-3 beyond half a bf16 ulp above) is
stated for unit-scale V, and since attention is linear in V it is applied
here times the RMS of the case's V (an output that cancels to nearly 0 among
values of 6e4 still carries errors of the size 6e4 x 2^-11); each case
through the unscaled kernel (bf16 only) or the scaled one (int8 present),
with 128-token blocks and with 16-token blocks (the per-q-block bias path),
and through the balanced launch with a forced cut."""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import assert_attn_close, run_attn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print(*a, flush=True)


# name: list of (segment length, dtype, V kind, V parameter); K is N(0,1) everywhere
CASES = {
    "int8_sigma_1e-3": [(300, "int8", "normal", 1e-3), (200, "bf16", "normal", 1e-3)],
    "int8_sigma_1e-4": [(300, "int8", "normal", 1e-4), (200, "bf16", "normal", 1e-4)],
    "int8_sigma_1e-5": [(300, "int8", "normal", 1e-5), (200, "bf16", "normal", 1e-5)],
    "bf16_sigma_1e-6": [(300, "bf16", "normal", 1e-6), (200, "bf16", "normal", 1e-6)],
    "bf16_sigma_1e-9": [(500, "bf16", "normal", 1e-9)],
    "bf16_near_6e4": [(300, "bf16", "uniform", (5.0e4, 6.5e4)), (200, "bf16", "uniform", (5.0e4, 6.5e4))],
    "bf16_sigma_1e6": [(500, "bf16", "normal", 1e6)],
    "bf16_sigma_1e30": [(260, "bf16", "normal", 1e30), (130, "int8", "normal", 1e30)],
    "mixed_magnitudes": [(200, "int8", "normal", 1e-5), (150, "bf16", "normal", 1.0), (130, "bf16", "normal", 1e-6),
                         (100, "int8", "normal", 1.0), (120, "bf16", "normal", 1e5)],
    "zero_tiles": [(130, "bf16", "zero", None), (200, "bf16", "normal", 1.0), (70, "int8", "zero", None)],
}


def _case(name, H=2, d=128, n_q=200):
    seed = sum(map(ord, name))
    q = W.normal_bf16(seed, 0, (n_q, H, d))
    segs = []
    for i, (L, dt, kind, arg) in enumerate(CASES[name]):
        k = W.normal_bf16(seed, 10 + i, (L, H, d))
        if kind == "normal":
            v = W.normal_bf16(seed, 20 + i, (L, H, d), sigma=arg)
        elif kind == "uniform":
            v = W.signed_uniform_bf16(seed, 20 + i, (L, H, d), *arg)
            assert np.abs(oracle.bf16_to_f64(v)).max() <= 65280.0
        else:
            v = np.zeros((L, H, d), np.uint16)
        if dt == "int8":
            ck, sk = oracle.kv_quant_int8(k)
            cv, sv = oracle.kv_quant_int8(v)
            segs.append({"k": ck, "v": cv, "k_scale": sk, "v_scale": sv, "dtype": "int8"})
        else:
            segs.append({"k": k, "v": v, "dtype": "bf16"})
    return q, segs


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("block,launch", [(128, "plain"), (16, "plain"), (128, "cut")])
def test_v_far_from_unit_scale(name, block, launch):
    q, segs = _case(name)
    n_q = q.shape[0]
    lens = [s["k"].shape[0] for s in segs]
    nkb = sum(-(-L // block) for L in lens)
    nqb = -(-n_q // block)
    rng = np.random.default_rng([sum(map(ord, name)), 100])
    mask = np.ones((nqb, nkb), np.uint8) if block == 128 else (rng.random((nqb, nkb)) < 0.7).astype(np.uint8)
    split = None if launch == "plain" else max(1, sum(-(-L // 64) for L in lens) // 2)
    _say("V range", name, "block", block, launch)
    out, lse = run_attn(q, segs, mask, block, block, split_tile=split)
    O, LSE = oracle.attention(q, segs, mask, block, block)
    vals = np.concatenate([oracle.segment_values(s)[1].ravel() for s in segs])
    v_rms = float(np.sqrt(np.mean(vals * vals))) or 1.0
    e = assert_attn_close(out, lse, O, LSE, f"{name} block {block} {launch}", v_scale=v_rms)
    _say(f"   V rms {v_rms:.3e}, |O| up to {np.abs(O).max():.3e}: max-abs {e[0]:.2e}, rel-RMS {e[1]:.2e}")
