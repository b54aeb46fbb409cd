"""RMSNorm and LayerNorm + modulate through the C ABI against the fp64
oracle: every output within one bf16 ulp of the oracle's correctly rounded
value (both sides compute in fp64 and round once, so nearly all outputs are
identical), over ragged hidden sizes (idle lanes, every chunks-per-lane
count up to the 8192 maximum), ragged token counts, in place, degenerate
rows, and the DiT hidden-state shapes of the attention workloads on sampled
rows."""
import numpy as np
import pytest

import workloads as W
from helpers import dev, host_u16, ordered
import oracle

pytestmark = pytest.mark.gpu

EPS = float(np.float32(1e-6))   # the fp32 eps the kernel receives, also given to the oracle


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print(*a, flush=True)


def _run(op, inp, eps=EPS, in_place=False):
    import torch
    import streaming_video_dit_amd as sdit
    n, d = inp.x.shape
    x = dev(inp.x)
    y = x if in_place else torch.full((n, d), -1, dtype=torch.int16, device="cuda")
    if op == "rmsnorm":
        g = dev(inp.gamma)
        sdit.rmsnorm(x, y, g, n, d, eps)
    else:
        sc, sh = dev(inp.scale), dev(inp.shift)
        sdit.layernorm_modulate(x, y, sc, sh, n, d, eps)
    torch.cuda.synchronize()
    return host_u16(y)


def _ref(op, inp, rows=slice(None), eps=EPS):
    if op == "rmsnorm":
        return oracle.rmsnorm(inp.x[rows], inp.gamma, eps)
    return oracle.layernorm_modulate(inp.x[rows], inp.scale, inp.shift, eps)


def _check(got, ref, min_same=0.999):
    ulps = np.abs(ordered(got) - ordered(ref))
    same = float((ulps == 0).mean())
    _say(f"   max ulp {int(ulps.max())}, identical {100 * same:.4f}%")
    assert ulps.max() <= 1
    assert same >= min_same


OPS = ["rmsnorm", "layernorm_modulate"]


# (n_tok, dim): 8 is one chunk on one lane; 520 and 1000 leave lanes of the
# last chunk idle; 8192 is 16 chunks per lane; token counts are not multiples
# of the 4 rows of a workgroup.
@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("n_tok,dim", [(37, 8), (37, 520), (45, 1000), (64, 1536), (9, 5120), (5, 8192),
                                       (130, 3072), (1, 4096)])
def test_norm_within_one_ulp(op, n_tok, dim):
    inp = W.make_norm_inputs(40, n_tok, dim, offset=2.0)
    _say(op, n_tok, dim)
    _check(_run(op, inp), _ref(op, inp))


# Above 2048 columns each wave walks several rows (one workgroup per 4 rows up
# to 2048 workgroups): 16421 rows = 2.005 rows per wave, so most waves take
# two rows and a few take three; every row is checked.
@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("dim", [2560, 8192])
def test_norm_rows_walked_per_wave(op, dim):
    n = 2 * 8192 + 37 if dim == 2560 else 8192 + 5
    inp = W.make_norm_inputs(46, n, dim, offset=1.0)
    _say(op, n, dim)
    _check(_run(op, inp), _ref(op, inp))


@pytest.mark.parametrize("op", OPS)
def test_norm_in_place_equals_out_of_place(op):
    for n, d in ((77, 1536), (8200, 4096)):
        inp = W.make_norm_inputs(41, n, d)
        assert np.array_equal(_run(op, inp), _run(op, inp, in_place=True))


@pytest.mark.parametrize("op", OPS)
def test_norm_degenerate_rows(op):
    """A zero row, a constant row, a row far from zero with a small spread
    (x - mean must keep its bits) and a row of one large value among zeros."""
    d = 2048
    inp = W.make_norm_inputs(42, 6, d)
    x = inp.x.copy()
    x[0] = 0
    x[1] = W.normal_bf16(42, 50, (1,))[0]
    big = W.make_norm_inputs(43, 1, d).x[0]
    # 256 + small bf16 values: bf16 near 256 has a step of 2, so draw integers
    x[2] = W._f32_to_bf16_bits(np.float32(256.0) + 2.0 * np.random.default_rng(44).integers(-4, 5, d).astype(
        np.float32))
    x[3] = 0
    x[3, 17] = W._f32_to_bf16_bits(np.float32([1000.0]))[0]
    x[4] = big
    x[5] = W._f32_to_bf16_bits(np.full(d, -3.5, np.float32))
    inp.x = x
    got = _run(op, inp)
    ref = _ref(op, inp)
    _check(got, ref, min_same=0.99)
    if op == "layernorm_modulate":
        # zero spread: (x - mean) is exactly 0, so the output is the shift rounded to bf16
        want = W._f32_to_bf16_bits(inp.shift)
        assert np.array_equal(ordered(got[0]), ordered(want))
        assert np.array_equal(ordered(got[5]), ordered(want))
    else:
        assert np.all(ordered(got[0]) == 0)


@pytest.mark.parametrize("op", OPS)
def test_norm_eps_zero(op):
    inp = W.make_norm_inputs(45, 33, 1024, offset=1.0)
    _check(_run(op, inp, eps=0.0), _ref(op, inp, eps=0.0))


@pytest.mark.parametrize("op", OPS)
def test_norm_zero_tokens_is_a_no_op(op):
    import torch
    import streaming_video_dit_amd as sdit
    y = torch.full((4, 64), 7, dtype=torch.int16, device="cuda")
    g = torch.ones(64, dtype=torch.float32, device="cuda")
    if op == "rmsnorm":
        sdit.rmsnorm(y, y, g, 0, 64)
    else:
        sdit.layernorm_modulate(y, y, g, g, 0, 64)
    torch.cuda.synchronize()
    assert bool((y == 7).all())


# The hidden state of each attention workload's query tokens, hidden size
# n_heads * head_dim, checked on sampled rows.
@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("name", ["wan13b", "large_dit", "bsa_sr"])
def test_norm_workload_shapes_sampled(op, name):
    cfg = W.WORKLOADS[name]
    n, d = cfg.n_q, cfg.n_heads * cfg.head_dim
    inp = W.make_norm_inputs(cfg.seed, n, d, offset=1.0)
    _say(op, name, n, d)
    got = _run(op, inp)
    rows = np.unique(np.concatenate([np.arange(4), n - 1 - np.arange(4),
                                     np.random.default_rng(cfg.seed).integers(0, n, 256)]))
    _check(got[rows], _ref(op, inp, rows))
