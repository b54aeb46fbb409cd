"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Bars: int8 codes and fp32 scales bit-exact; qknorm_rope3d within one bf16
ulp of the oracle's single rounding (at least 99.9% bit-identical);
attention within relative RMS 1e-2 of the unrounded fp64 result and, element
by element, within max-abs 4e-3 where |ref| < 1 (a correctly rounded bf16
output is then within 2e-3) and within 4e-3 beyond half a bf16 ulp of ref
above that (where the output's own rounding alone may exceed 4e-3); LSE
within 1e-3. Small cases are compared element by element; the full-size
workloads run in the same launch configuration as the benchmark and are
compared on every row of two whole heads (one of them holding units that the
balanced launch cuts) and on sampled query rows of every head
(first/last/ragged q-tiles)."""
import numpy as np
import pytest

import workloads as W
from helpers import (assert_attn_close, dev, empty_bf16, gpu_segments, host_u16, ordered, run_attn,
                     segments_for_oracle)
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ kv_quant_int8

def _gpu_quant(x_bits):
    import torch
    import streaming_video_dit_amd as sdit
    n, H, d = x_bits.shape
    x = dev(x_bits)
    codes = torch.full((n, H, d), 99, dtype=torch.int8, device="cuda")
    scales = torch.full((n, H), float("nan"), dtype=torch.float32, device="cuda")
    sdit.kv_quant_int8(x, codes, scales, n, H, d)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def test_kv_quant_bit_exact_on_the_int8_cache_workload():
    cfg = W.WORKLOADS["wan13b_int8"]
    inp = W.make_inputs(cfg)
    for name, x in [("text K", inp.cache_k[0]), ("text V", inp.cache_v[0]),
                    ("history K", inp.cache_k[1]), ("history V", inp.cache_v[1]), ("chunk K", inp.k)]:
        _say("kv_quant", name, x.shape)
        c, s = _gpu_quant(x)
        rc, rs = oracle.kv_quant_int8(x)
        assert np.array_equal(s.view(np.uint32), rs.view(np.uint32)), name
        assert np.array_equal(c, rc), f"{name}: {(c != rc).sum()} codes differ"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_tok,H", [(1, 1), (3, 5), (1000, 12)])
def test_kv_quant_edge_cases(d, n_tok, H):
    rng = np.random.default_rng(n_tok * 7 + d)
    x = W.normal_bf16(n_tok + d, 1, (n_tok, H, d), outlier_p=0.05, outlier_tid=2)
    x[0, 0, :] = 0                                   # all-zero row
    if n_tok > 1:
        x[1, 0, :] = 0
        x[1, 0, d // 2] = 0xBF80                     # single nonzero (-1.0)
    if n_tok > 2:
        # amax = 127 * 2^-3 makes the scale a power of two: exact half-way quotients
        vals = (np.arange(d) - d // 2 + 0.5).astype(np.float32) * np.float32(0.125)
        vals[0] = 127 * 0.125
        x[2, H - 1, :] = (vals.view(np.uint32) >> 16).astype(np.uint16)
    _say("kv_quant edge", d, n_tok, H)
    c, s = _gpu_quant(x)
    rc, rs = oracle.kv_quant_int8(x)
    assert np.array_equal(s.view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(c, rc)


# ------------------------------------------------------------------ qknorm_rope3d

def _gpu_rope(cfg_like, q_bits, k_bits, gq, gk, in_place=False):
    import torch
    import streaming_video_dit_amd as sdit
    T, Hl, Wl, t0, (dt, dh, dw) = cfg_like
    n, H, d = q_bits.shape
    qi, ki = dev(q_bits), dev(k_bits)
    qo, ko = (qi, ki) if in_place else (empty_bf16((n, H, d)), empty_bf16((n, H, d)))
    sdit.qknorm_rope3d(qi, ki, qo, ko, dev(gq), dev(gk), T, Hl, Wl, t0, H, d, dt, dh, dw, 1.0e4, 1.0e-6)
    torch.cuda.synchronize()
    return host_u16(qo), host_u16(ko)


def _check_rope(got, x_bits, g, geo):
    T, Hl, Wl, t0, (dt, dh, dw) = geo
    ref = oracle.qknorm_rope3d(x_bits, g, T, Hl, Wl, t0, dt, dh, dw)
    ulps = np.abs(ordered(got) - ordered(ref))
    same = float((ulps == 0).mean())
    _say(f"   max ulp {int(ulps.max())}, identical {100 * same:.4f}%")
    assert ulps.max() <= 1
    assert same >= 0.999
    return same


@pytest.mark.parametrize("name", ["tiny", "wan13b", "large_dit"])
def test_qknorm_rope3d_within_one_ulp(name):
    cfg = W.WORKLOADS[name]
    inp = W.make_inputs(cfg)
    geo = (cfg.T, cfg.Hl, cfg.Wl, cfg.t0, cfg.split)
    _say("qknorm_rope3d", name, inp.q.shape)
    gq, gk = _gpu_rope(geo, inp.q, inp.k, inp.gamma_q, inp.gamma_k)
    _check_rope(gq, inp.q, inp.gamma_q, geo)
    _check_rope(gk, inp.k, inp.gamma_k, geo)


def test_qknorm_rope3d_in_place_equals_out_of_place():
    cfg = W.WORKLOADS["wan13b"]
    inp = W.make_inputs(cfg, n_heads=3)
    geo = (cfg.T, cfg.Hl, cfg.Wl, cfg.t0, cfg.split)
    a = _gpu_rope(geo, inp.q, inp.k, inp.gamma_q, inp.gamma_k)
    b = _gpu_rope(geo, inp.q, inp.k, inp.gamma_q, inp.gamma_k, in_place=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# Far frame positions: rotation angles up to ~7e4 rad go through the
# kernel's own argument reduction, and past 2^20 rad through the fallback.
@pytest.mark.parametrize("t0", [70000, 1 << 21])
def test_qknorm_rope3d_far_positions(t0):
    geo = (2, 3, 5, t0, W.rope_split(128))
    n, H, d = 2 * 3 * 5, 4, 128
    q = W.normal_bf16(32, 0, (n, H, d))
    k = W.normal_bf16(32, 1, (n, H, d))
    gq = W.uniform_f32(32, 2, (d,), 0.5, 1.5)
    gk = W.uniform_f32(32, 3, (d,), 0.5, 1.5)
    _say("qknorm_rope3d t0", t0)
    a, b = _gpu_rope(geo, q, k, gq, gk)
    _check_rope(a, q, gq, geo)
    _check_rope(b, k, gk, geo)


@pytest.mark.parametrize("split,d", [((64, 0, 0), 64), ((0, 0, 64), 64), ((20, 24, 20), 64), ((0, 128, 0), 128)])
def test_qknorm_rope3d_other_splits(split, d):
    geo = (2, 3, 5, 7, split)
    n, H = 2 * 3 * 5, 3
    q = W.normal_bf16(31, 0, (n, H, d))
    k = W.normal_bf16(31, 1, (n, H, d))
    gq = W.uniform_f32(31, 2, (d,), 0.5, 1.5)
    gk = W.uniform_f32(31, 3, (d,), 0.5, 1.5)
    a, b = _gpu_rope(geo, q, k, gq, gk)
    _check_rope(a, q, gq, geo)
    _check_rope(b, k, gk, geo)


# ------------------------------------------------------------------ qknorm_rope3d + int8 cache entries, fused

def _gpu_rope_quant(geo, q_bits, k_bits, v_bits, gq, gk, in_place=False):
    import torch
    import streaming_video_dit_amd as sdit
    T, Hl, Wl, t0, (dt, dh, dw) = geo
    n, H, d = q_bits.shape
    qi, ki, vi = dev(q_bits), dev(k_bits), dev(v_bits)
    qo, ko = (qi, ki) if in_place else (empty_bf16((n, H, d)), empty_bf16((n, H, d)))
    kc = torch.full((n, H, d), 99, dtype=torch.int8, device="cuda")
    vc = torch.full((n, H, d), 99, dtype=torch.int8, device="cuda")
    ks = torch.full((n, H), float("nan"), dtype=torch.float32, device="cuda")
    vs = torch.full((n, H), float("nan"), dtype=torch.float32, device="cuda")
    sdit.qknorm_rope3d_kv_quant_int8(qi, ki, vi, qo, ko, kc, ks, vc, vs, dev(gq), dev(gk), T, Hl, Wl, t0, H, d,
                                     dt, dh, dw, 1.0e4, 1.0e-6)
    torch.cuda.synchronize()
    return host_u16(qo), host_u16(ko), kc.cpu().numpy(), ks.cpu().numpy(), vc.cpu().numpy(), vs.cpu().numpy()


@pytest.mark.parametrize("case", ["tiny", "wan13b_int8", "five_heads_d128", "three_heads_d64_in_place"])
def test_qknorm_rope3d_with_int8_cache_entries(case):
    """One pass writing the rotated q, k and the int8 cache entries of k and
    v: q/k bit for bit as sdit_qknorm_rope3d (within one ulp of the oracle),
    codes and scales bit for bit as the oracle's quantisation of that k and of
    v (head groups of 4 with a ragged last group: 5 and 3 heads)."""
    if case in ("tiny", "wan13b_int8"):
        cfg = W.WORKLOADS[case]
        inp = W.make_inputs(cfg)
        r = W.chunk_rows(cfg, 0)
        q, k, v, gq, gk = inp.q[r], inp.k[r], inp.v[r], inp.gamma_q, inp.gamma_k
        geo = (cfg.T, cfg.Hl, cfg.Wl, cfg.t0, cfg.split)
    else:
        H, d = (5, 128) if case == "five_heads_d128" else (3, 64)
        geo = (3, 5, 7, 4, W.rope_split(d))
        n = 3 * 5 * 7
        q = W.normal_bf16(61, 0, (n, H, d))
        k = W.normal_bf16(61, 1, (n, H, d), outlier_p=0.02, outlier_tid=5)
        v = W.normal_bf16(61, 2, (n, H, d), outlier_p=0.02, outlier_tid=6)
        v[0, 0, :] = 0                      # an all-zero v row
        gq = W.uniform_f32(61, 3, (d,), 0.5, 1.5)
        gk = W.uniform_f32(61, 4, (d,), 0.5, 1.5)
    _say("qknorm_rope3d + int8 cache entries", case, q.shape)
    qo, ko, kc, ks, vc, vs = _gpu_rope_quant(geo, q, k, v, gq, gk, in_place=case.endswith("in_place"))
    pq, pk = _gpu_rope(geo, q, k, gq, gk)
    assert np.array_equal(qo, pq) and np.array_equal(ko, pk), "q/k differ from sdit_qknorm_rope3d"
    _check_rope(qo, q, gq, geo)
    _check_rope(ko, k, gk, geo)
    rkc, rks = oracle.kv_quant_int8(ko)
    rvc, rvs = oracle.kv_quant_int8(v)
    assert np.array_equal(ks.view(np.uint32), rks.view(np.uint32)) and np.array_equal(kc, rkc), "k codes/scales"
    assert np.array_equal(vs.view(np.uint32), rvs.view(np.uint32)) and np.array_equal(vc, rvc), "v codes/scales"


# ------------------------------------------------------------------ attention: tiny workload end to end

@pytest.mark.parametrize("name", ["tiny", "tiny_dense"])
def test_tiny_workload_end_to_end(name):
    cfg = W.WORKLOADS[name]
    inp = W.make_inputs(cfg)
    geo = (cfg.T, cfg.Hl, cfg.Wl, cfg.t0, cfg.split)
    _say("tiny end to end", name)
    gq, gk = _gpu_rope(geo, inp.q, inp.k, inp.gamma_q, inp.gamma_k)
    dt, dh, dw = cfg.split
    rq = oracle.qknorm_rope3d(inp.q, inp.gamma_q, cfg.T, cfg.Hl, cfg.Wl, cfg.t0, dt, dh, dw)
    rk = oracle.qknorm_rope3d(inp.k, inp.gamma_k, cfg.T, cfg.Hl, cfg.Wl, cfg.t0, dt, dh, dw)
    assert np.abs(ordered(gq) - ordered(rq)).max() <= 1
    # each side runs its own chain: GPU rope -> GPU attention, oracle rope -> oracle attention
    out, lse = run_attn(gq, segments_for_oracle(inp, gk), inp.mask, cfg.block, cfg.block)
    O, LSE = oracle.attention(rq, segments_for_oracle(inp, rk), inp.mask, cfg.block, cfg.block)
    e = assert_attn_close(out, lse, O, LSE, name)
    _say(f"   max-abs {e[0]:.2e} ({e[2]:.2e} beyond half an ulp), rel-RMS {e[1]:.2e}")


def test_tiny_chunks_end_to_end():
    """Two query chunks in one forward, RoPE per chunk, chunk-causal mask."""
    cfg = W.WORKLOADS["tiny_chunks"]
    inp = W.make_inputs(cfg)
    dt, dh, dw = cfg.split
    gq, gk, rq, rk = inp.q.copy(), inp.k.copy(), inp.q.copy(), inp.k.copy()
    for c in range(cfg.n_chunks):
        r = W.chunk_rows(cfg, c)
        t0 = cfg.t0 + c * cfg.T
        gq[r], gk[r] = _gpu_rope((cfg.T, cfg.Hl, cfg.Wl, t0, cfg.split), inp.q[r], inp.k[r], inp.gamma_q,
                                 inp.gamma_k)
        rq[r] = oracle.qknorm_rope3d(inp.q[r], inp.gamma_q, cfg.T, cfg.Hl, cfg.Wl, t0, dt, dh, dw)
        rk[r] = oracle.qknorm_rope3d(inp.k[r], inp.gamma_k, cfg.T, cfg.Hl, cfg.Wl, t0, dt, dh, dw)
    _say("tiny chunks end to end")
    out, lse = run_attn(gq, segments_for_oracle(inp, gk), inp.mask, cfg.block, cfg.block)
    O, LSE = oracle.attention(rq, segments_for_oracle(inp, rk), inp.mask, cfg.block, cfg.block)
    e = assert_attn_close(out, lse, O, LSE, "tiny_chunks")
    _say(f"   max-abs {e[0]:.2e} ({e[2]:.2e} beyond half an ulp), rel-RMS {e[1]:.2e}")


def test_tiny_mask_readings_differ_on_gpu():
    cfg = W.WORKLOADS["tiny"]
    inp = W.make_inputs(cfg)
    segs = segments_for_oracle(inp, inp.k)
    a, _ = run_attn(inp.q, segs, W.make_mask(cfg), 16, 16)
    b, _ = run_attn(inp.q, segs, W.make_mask(W.WORKLOADS["tiny_dense"]), 16, 16)
    assert np.array_equal(a[16:], b[16:])
    assert not np.array_equal(a[:16], b[:16])


# ------------------------------------------------------------------ attention: small cases, every element

def _rand_case(seed, n_q, H, d, lens, dtypes, bq, bk, density=1.0, empty_rows=()):
    q = W.normal_bf16(seed, 0, (n_q, H, d))
    segs = []
    for i, (L, dt) in enumerate(zip(lens, dtypes)):
        k = W.normal_bf16(seed, 10 + 2 * i, (L, H, d), outlier_p=0.01, outlier_tid=50 + i)
        v = W.normal_bf16(seed, 11 + 2 * i, (L, H, d), outlier_p=0.01, outlier_tid=60 + i)
        if dt == "int8":
            ck, sk = oracle.kv_quant_int8(k)
            cv, sv = oracle.kv_quant_int8(v)
            segs.append({"k": ck, "v": cv, "k_scale": sk, "v_scale": sv, "dtype": "int8"})
        else:
            segs.append({"k": k, "v": v, "dtype": "bf16"})
    nqb = -(-n_q // bq)
    nkb = sum(-(-L // bk) for L in lens)
    rng = np.random.default_rng([seed, 100])
    mask = (rng.random((nqb, nkb)) < density).astype(np.uint8)
    for r in empty_rows:
        mask[r] = 0
    return q, segs, mask


CASES = {
    # name: (n_q, H, d, segment lengths, dtypes, block_q, block_k, density, empty q-block rows)
    "d128_ragged_3seg": (300, 2, 128, [77, 300, 130], ["bf16"] * 3, 128, 128, 1.0, ()),
    "d128_int8_mix": (257, 3, 128, [64, 200, 257], ["int8", "int8", "bf16"], 128, 128, 1.0, ()),
    "d128_sparse": (640, 2, 128, [640], ["bf16"], 128, 128, 0.35, (2,)),
    "d128_small_blocks": (200, 2, 128, [50, 150, 200], ["bf16", "int8", "bf16"], 32, 16, 0.6, (0,)),
    "d64_b64": (190, 2, 64, [33, 190], ["bf16", "bf16"], 64, 64, 0.7, ()),
    "d64_b32_int8": (100, 1, 64, [129, 100], ["int8", "bf16"], 32, 32, 0.5, (1,)),
    "one_query": (1, 4, 128, [5, 1], ["bf16", "bf16"], 16, 16, 1.0, ()),
    "eight_segments": (130, 2, 128, [1, 63, 64, 65, 0, 128, 3, 130], ["bf16", "int8"] * 4, 128, 64, 0.8, ()),
    # 16-row q-blocks: all 16 bias slots of a 256-row workgroup, a ragged second one
    "d128_b16_sixteen_slots": (300, 2, 128, [90, 300], ["bf16", "bf16"], 16, 32, 0.5, (3, 12)),
    "d64_b16_int8_slots": (270, 2, 64, [100, 270], ["int8", "bf16"], 16, 64, 0.6, (9,)),
    # 32-row q-blocks: waves skip the tiles their rows drop, no bias needed
    "d128_b32_wave_skip": (520, 2, 128, [256, 520], ["bf16", "bf16"], 32, 64, 0.3, (5,)),
    "d128_b32_int8_wave_skip": (333, 2, 128, [160, 333], ["int8", "bf16"], 32, 128, 0.4, (0, 7)),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_attention_small_cases(case):
    n_q, H, d, lens, dts, bq, bk, dens, empty = CASES[case]
    q, segs, mask = _rand_case(sum(map(ord, case)), n_q, H, d, lens, dts, bq, bk, dens, empty)
    _say("attention", case)
    out, lse = run_attn(q, segs, mask, bq, bk)
    O, LSE = oracle.attention(q, segs, mask, bq, bk)
    e = assert_attn_close(out, lse, O, LSE, case)
    _say(f"   max-abs {e[0]:.2e} ({e[2]:.2e} beyond half an ulp), rel-RMS {e[1]:.2e}")
    for r in empty:
        rows = slice(r * bq, min(n_q, (r + 1) * bq))
        assert np.all(out[rows] == 0)


# More than 1024 kept 64-key tiles per workgroup: the kept-tile list is built
# and walked in passes of 1024 candidates (the second pass starts after the
# first one's last P.V), in the unscaled and the scaled kernel, with a
# first pass that keeps nothing.
@pytest.mark.parametrize("case", ["bf16_two_passes", "int8_empty_first_pass"])
def test_attention_long_cache_several_passes(case):
    if case == "bf16_two_passes":
        q, segs, mask = _rand_case(71, 300, 2, 64, [1000, 69000], ["bf16", "bf16"], 128, 64, 0.6)
    else:
        q, segs, mask = _rand_case(72, 200, 1, 128, [66000, 500], ["int8", "bf16"], 128, 64, 0.5)
        mask[:, :1024] = 0
    bq, bk = 128, 64
    assert mask.shape[1] * bk > 1024 * 64
    _say("attention", case, mask.shape)
    out, lse = run_attn(q, segs, mask, bq, bk)
    O, LSE = oracle.attention(q, segs, mask, bq, bk)
    e = assert_attn_close(out, lse, O, LSE, case)
    _say(f"   max-abs {e[0]:.2e} ({e[2]:.2e} beyond half an ulp), rel-RMS {e[1]:.2e}")


def test_attention_maximum_head_count():
    """The largest head count the library accepts (65536, so that a 64-key
    tile's rows, n_heads * head_dim elements apart, stay within 32-bit
    offsets: 2^29 elements at d = 128), with a full and a ragged key tile:
    65536 workgroups, K and V of 1.1 GB each. The oracle computes sampled
    heads (first, last and some between); every head's output is finite."""
    H, d, L = 65536, 128, 65
    _say("attention at the maximum head count: generating inputs")
    q = W.normal_bf16(83, 0, (1, H, d))
    k = W.normal_bf16(83, 1, (L, H, d))
    v = W.normal_bf16(83, 2, (L, H, d))
    segs = [{"k": k, "v": v, "dtype": "bf16"}]
    mask = np.ones((1, 1), np.uint8)
    _say("   running", H, "heads")
    out, lse = run_attn(q, segs, mask, 128, 128)
    assert np.all((out & 0x7F80) != 0x7F80) and np.all(np.isfinite(lse))
    heads = [0, 1, 4097, 32768, 65534, 65535]
    # heads are independent: the oracle runs on the sampled heads' slices
    sub = [{"k": np.ascontiguousarray(k[:, heads]), "v": np.ascontiguousarray(v[:, heads]), "dtype": "bf16"}]
    O, LSE = oracle.attention(np.ascontiguousarray(q[:, heads]), sub, mask, 128, 128)
    e = assert_attn_close(out[:, heads], lse[heads], O, LSE, "maximum head count")
    _say(f"   {len(heads)} heads: max-abs {e[0]:.2e} ({e[2]:.2e} beyond half an ulp), rel-RMS {e[1]:.2e}")


def test_dense_block_mask_matches_sdpa_within_the_pages_figure():
    """FlashVSR deployment notes (Block-Sparse-Attention on Ada): with a dense
    mask the block-sparse kernel has to reproduce scaled_dot_product_attention,
    and the page measured a bf16 max-abs difference of 1.16e-3
    (tests/golden/bsa_dense_vs_sdpa.json). The same check here, in the SR
    layout (one self-attention segment, 128-token blocks, N(0,1) q/k/v)
    against torch SDPA in fp64: the part of the error beyond the bf16 output's
    own rounding stays under the page's figure."""
    import json
    import os
    import torch
    from helpers import attn_errors
    fx = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "bsa_dense_vs_sdpa.json")))
    n, H, d = 1000, 2, 128
    q, k, v = (W.normal_bf16(81, t, (n, H, d)) for t in range(3))
    mask = np.ones((-(-n // 128), -(-n // 128)), np.uint8)
    out, _ = run_attn(q, [{"k": k, "v": v, "dtype": "bf16"}], mask, 128, 128)
    t = [torch.from_numpy(oracle.bf16_to_f64(a)).permute(1, 0, 2) for a in (q, k, v)]
    ref = torch.nn.functional.scaled_dot_product_attention(*t).permute(1, 0, 2).numpy()
    max_abs, rrms, beyond, _ = attn_errors(out, ref)
    _say(f"   dense vs SDPA: max-abs {max_abs:.2e}, beyond half an ulp {beyond:.2e}, page {fx['bf16_max_abs_error']}")
    assert beyond <= fx["bf16_max_abs_error"]
    assert rrms <= 1e-2


def test_attention_custom_softmax_scale():
    q, segs, mask = _rand_case(5, 200, 2, 128, [100, 200], ["bf16", "bf16"], 128, 128)
    out, lse = run_attn(q, segs, mask, 128, 128, softmax_scale=0.03)
    O, LSE = oracle.attention(q, segs, mask, 128, 128, softmax_scale=0.03)
    assert_attn_close(out, lse, O, LSE, "scale 0.03")


@pytest.mark.parametrize("dtypes", [["bf16", "bf16"], ["int8", "bf16"]])
def test_smallest_softmax_scale_keeps_masked_keys_out(dtypes):
    """At the smallest accepted scale (2^-40) every visible score is ~0, so each
    row averages V over its visible keys; a masked key's -1e30 bias, scaled,
    must still rank as invisible (fine 16-token blocks, int8 and bf16 tiles)."""
    q, segs, mask = _rand_case(23, 160, 2, 128, [96, 160], dtypes, 16, 16, 0.5, (3,))
    out, lse = run_attn(q, segs, mask, 16, 16, softmax_scale=2.0 ** -40)
    O, LSE = oracle.attention(q, segs, mask, 16, 16, softmax_scale=2.0 ** -40)
    assert_attn_close(out, lse, O, LSE, "scale 2^-40")


def test_attention_all_segments_empty_gives_zero_and_minus_inf():
    q = W.normal_bf16(1, 0, (40, 2, 64))
    segs = [{"k": np.zeros((0, 2, 64), np.uint16), "v": np.zeros((0, 2, 64), np.uint16), "dtype": "bf16"}]
    out, lse = run_attn(q, segs, np.zeros((3, 0), np.uint8), 16, 16)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_nan_in_skipped_tiles_never_reaches_the_output():
    q, segs, mask = _rand_case(9, 512, 2, 128, [512], ["bf16"], 128, 128, 0.4)
    mask[:, 1] = 0
    mask[np.arange(4), np.arange(4)] = 1
    mask[1, 1] = 0
    out_clean, lse_clean = run_attn(q, segs, mask, 128, 128)
    poisoned = {"k": segs[0]["k"].copy(), "v": segs[0]["v"].copy(), "dtype": "bf16"}
    poisoned["k"][128:256] = 0x7FC0
    poisoned["v"][128:256] = 0x7FC0
    out_p, lse_p = run_attn(q, [poisoned], mask, 128, 128)
    assert np.array_equal(out_p, out_clean)
    assert np.array_equal(lse_p.view(np.uint32), lse_clean.view(np.uint32))
    assert not np.isnan(lse_p).any()
    # q-block 1 keeps no tile at all: zero output, LSE -inf
    assert np.all(out_p[128:256] == 0) and np.all(np.isneginf(lse_p[:, 128:256]))
    O, LSE = oracle.attention(q, segs, mask, 128, 128)
    assert_attn_close(out_p, lse_p, O, LSE, "poisoned")


@pytest.mark.parametrize("bq", [32, 16])
def test_rows_whose_first_tiles_are_fully_masked(bq):
    # q-block 0 drops the first three 64-key tiles that its neighbours keep.
    # With 32-row q-blocks the wave holding those rows skips the tiles; with
    # 16-row q-blocks the same wave also holds rows that keep them, so the
    # rows of q-block 0 meet whole tiles of -1e30-biased scores before any
    # visible key. Either way their output must be the attention over the
    # later keys only (no overflow from the bias).
    q, segs, mask = _rand_case(21, 128, 2, 128, [512], ["bf16"], bq, 64)
    mask[0, :3] = 0
    mask[2, 5:] = 0
    out, lse = run_attn(q, segs, mask, bq, 64)
    O, LSE = oracle.attention(q, segs, mask, bq, 64)
    assert not np.isnan(lse).any()
    assert_attn_close(out, lse, O, LSE, "first tiles masked")


def test_all_zero_int8_key_in_a_masked_block_stays_masked():
    # An all-zero key quantises to scale 0; the mask bias must still remove it
    # when its block is dropped for a q-block (its score multiplier is floored
    # above 0), and it must count (score 0) where its block is kept.
    q, segs, mask = _rand_case(22, 96, 2, 128, [200, 64], ["int8", "bf16"], 32, 32)
    s = segs[0]
    s["k"][40:48] = 0
    s["k_scale"][40:48] = 0.0
    mask[:] = 1
    mask[1, 1] = 0          # keys 32..63 (holding the zero keys) dropped for rows 32..63
    out, lse = run_attn(q, segs, mask, 32, 32)
    O, LSE = oracle.attention(q, segs, mask, 32, 32)
    assert_attn_close(out, lse, O, LSE, "zero int8 key")


def test_attention_is_deterministic():
    q, segs, mask = _rand_case(3, 700, 3, 128, [300, 700], ["int8", "bf16"], 128, 128, 0.9)
    a = run_attn(q, segs, mask, 128, 128)
    b = run_attn(q, segs, mask, 128, 128)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


# ------------------------------------------------------------------ full-size workloads, sampled rows

def _sample_rows(n_q, rng, k=24):
    rows = set(range(0, 3)) | set(range(n_q - 3, n_q))
    for tile in (128, 256):   # first rows of the last half and whole 256-row workgroup tile
        last_tile = (n_q - 1) // tile * tile
        rows |= {last_tile, min(n_q - 1, last_tile + 1)}
    rows |= set(rng.choice(n_q, size=k, replace=False).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", ["wan13b", "wan13b_int8", "large_dit", "bsa_sr", "wave_chunks"])
def test_full_size_hot_path_sampled(name):
    """The benchmark's step at full size: [qknorm_rope3d] -> [kv_quant_int8 of the
    cache] -> attention on the GPU, both through attn_fwd and through
    attn_fwd_balanced with the library's plan (the benchmark's launch); the
    oracle runs the same chain on the CPU and computes the sampled rows of
    every head and every row of two whole heads."""
    import torch
    import streaming_video_dit_amd as sdit
    cfg = W.WORKLOADS[name]
    inp = W.make_inputs(cfg)
    H, d, n_q = cfg.n_heads, cfg.head_dim, cfg.n_q
    _say("full size", name, "n_q", n_q, "keys", sum(cfg.seg_lens))
    # --- GPU chain (RoPE per query chunk; padding rows between chunks stay raw)
    gq, gk = inp.q.copy(), inp.k.copy()
    if cfg.rope:
        for c in range(cfg.n_chunks):
            r = W.chunk_rows(cfg, c)
            geo = (cfg.T, cfg.Hl, cfg.Wl, cfg.t0 + c * cfg.T, cfg.split)
            gq[r], gk[r] = _gpu_rope(geo, inp.q[r], inp.k[r], inp.gamma_q, inp.gamma_k)
    gpu_quant = {}
    for i, is8 in enumerate(cfg.seg_int8[:cfg.n_cached]):
        if is8:
            ck, sk = _gpu_quant(inp.cache_k[i])
            cv, sv = _gpu_quant(inp.cache_v[i])
            gpu_quant[i] = (ck, sk, cv, sv)
    gsegs = segments_for_oracle(inp, gk, gpu_quant)
    out, lse = run_attn(gq, gsegs, inp.mask, cfg.block, cfg.block)
    out_b, lse_b = run_attn(gq, gsegs, inp.mask, cfg.block, cfg.block, split_tile=-1)
    # --- oracle chain
    rq, rk = inp.q.copy(), inp.k.copy()
    if cfg.rope:
        dt, dh, dw = cfg.split
        for c in range(cfg.n_chunks):
            r = W.chunk_rows(cfg, c)
            t0 = cfg.t0 + c * cfg.T
            rq[r] = oracle.qknorm_rope3d(inp.q[r], inp.gamma_q, cfg.T, cfg.Hl, cfg.Wl, t0, dt, dh, dw)
            rk[r] = oracle.qknorm_rope3d(inp.k[r], inp.gamma_k, cfg.T, cfg.Hl, cfg.Wl, t0, dt, dh, dw)
    ref_quant = {}
    for i, is8 in enumerate(cfg.seg_int8[:cfg.n_cached]):
        if is8:
            ck, sk = oracle.kv_quant_int8(inp.cache_k[i])
            cv, sv = oracle.kv_quant_int8(inp.cache_v[i])
            ref_quant[i] = (ck, sk, cv, sv)
            assert np.array_equal(ck, gpu_quant[i][0]) and np.array_equal(cv, gpu_quant[i][2])
    rows = _sample_rows(n_q, np.random.default_rng(cfg.seed))
    O, LSE = oracle.attention(rq, segments_for_oracle(inp, rk, ref_quant), inp.mask, cfg.block, cfg.block,
                              rows=rows)
    e = assert_attn_close(out[rows], lse[:, rows], O, LSE, name)
    _say(f"   {len(rows)} rows x {H} heads: max-abs {e[0]:.2e} ({e[2]:.2e} beyond half an ulp), rel-RMS {e[1]:.2e}")
    e = assert_attn_close(out_b[rows], lse_b[:, rows], O, LSE, name + " balanced")
    _say(f"   balanced: max-abs {e[0]:.2e} ({e[2]:.2e} beyond half an ulp), rel-RMS {e[1]:.2e}")
    # every row of two whole heads: head 0 and the head of XCD 0's last work
    # unit, which the balanced launch cuts into pieces whenever it cuts at all
    osegs = segments_for_oracle(inp, rk, ref_quant)
    n_qt = -(-n_q // 256)
    heads = sorted({0, min(H - 1, ((H * n_qt) // 8 - 1) // n_qt)})
    Of, LSEf = oracle.attention(rq, osegs, inp.mask, cfg.block, cfg.block, heads=heads)
    for o_x, l_x, label in ((out, lse, name), (out_b, lse_b, name + " balanced")):
        e = assert_attn_close(o_x[:, heads], l_x[heads], Of, LSEf, f"{label}, heads {heads}")
        _say(f"   {label}: every row of heads {heads}: max-abs {e[0]:.2e} ({e[2]:.2e} beyond half an ulp), "
             f"rel-RMS {e[1]:.2e}")
    # every row, every head: finite output, and LSE finite where a key is visible
    assert np.all((out & 0x7F80) != 0x7F80)
    assert np.all((out_b & 0x7F80) != 0x7F80)
    assert np.array_equal(np.isfinite(lse), np.isfinite(lse_b))
