"""Parity of split-KV attention (sdit_attn_fwd_partial + sdit_attn_merge)
with the fp64 oracle, through the C ABI.

  * the fp32 partial output over a group of segments against the oracle's
    attention over that group, with the bars of the bf16 output it becomes
    (max-abs 4e-3 where |ref| < 1, else 4e-3 beyond half a bf16 ulp;
    relative RMS 1e-2; LSE 1e-3; rows that see nothing: exact 0 and -inf);
  * the merge alone, fed the oracle's partials in fp32, against the oracle's
    merge of the same fp32 values: within one bf16 ulp, LSE within 1e-5;
  * the whole split path (partials on the GPU, merge on the GPU) against the
    oracle's attention over the whole cache, small cases and the Wan-chunk
    shape split into cache | current chunk (sampled rows)."""
import numpy as np
import pytest

import workloads as W
from helpers import ATOL_LSE, ATOL_O, RRMS_O, assert_attn_close, attn_tolerance, bf16_to_float, dev, gpu_segments, \
    half_ulp_bf16, host_u16, run_attn
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print(*a, flush=True)


def _segments(seed, lens, dtypes, H, d):
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
    return segs


def _columns(lens, bk, first, last):
    starts = np.cumsum([0] + [-(-L // bk) for L in lens])
    return slice(int(starts[first]), int(starts[last]))


def _groups(n_segs, cuts):
    b = [0] + list(cuts) + [n_segs]
    return list(zip(b[:-1], b[1:]))


def run_partial(q_bits, segs, mask, bq, bk):
    """sdit_attn_fwd_partial; returns (O fp32 [n_q,H,d], LSE [H,n_q]) on the host."""
    import torch
    import streaming_video_dit_amd as sdit
    n_q, H, d = q_bits.shape
    q = dev(q_bits)
    gs, keep = gpu_segments(segs)
    m = dev(mask.astype(np.uint8))
    out = torch.full((n_q, H, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((H, n_q), float("nan"), dtype=torch.float32, device="cuda")
    sdit.attn_fwd_partial(q, n_q, gs, m, bq, bk, H, d, out, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def run_merge(parts, n_q, H, d):
    """sdit_attn_merge of host fp32 partials; returns (out bits, lse)."""
    import torch
    import streaming_video_dit_amd as sdit
    os_ = [dev(np.ascontiguousarray(O, dtype=np.float32)) for O, _ in parts]
    ls_ = [dev(np.ascontiguousarray(L, dtype=np.float32)) for _, L in parts]
    out = torch.full((n_q, H, d), -1, dtype=torch.int16, device="cuda")
    lse = torch.full((H, n_q), float("nan"), dtype=torch.float32, device="cuda")
    sdit.attn_merge(os_, ls_, n_q, H, d, out, lse)
    torch.cuda.synchronize()
    return host_u16(out), lse.cpu().numpy()


def _assert_paths_agree(out_a, out_b, what):
    """Two bf16 results that are each within ATOL_O plus half an ulp of the
    exact value differ by at most 2 ATOL_O plus one ulp."""
    a, b = bf16_to_float(out_a), bf16_to_float(out_b)
    bound = 2 * ATOL_O + 2 * half_ulp_bf16(np.maximum(np.abs(a), np.abs(b)))
    assert np.all(np.abs(a - b) <= bound), f"{what}: paths differ by {np.abs(a - b).max():.3e}"


def _assert_partial_close(O, L, O_ref, L_ref, what):
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isneginf(L), ~fin), what
    empty_rows = ~fin.T                                   # [n_q, H]
    assert np.all(O[empty_rows] == 0), what
    # the fp32 partial is an intermediate of a bf16 result: same bar as the bf16 output
    diff = O - O_ref
    worst = float((np.abs(diff) / attn_tolerance(O_ref)).max())
    assert worst <= 1.0, f"{what}: error {worst:.3f} x the per-element bar (max-abs {np.abs(diff).max():.3e})"
    denom = float(np.sqrt((O_ref ** 2).sum()))
    if denom > 0:
        assert float(np.sqrt((diff ** 2).sum())) / denom <= RRMS_O, what
    if fin.any():
        assert float(np.abs(L[fin] - L_ref[fin]).max()) <= ATOL_LSE, what


CASES = {
    # name: (n_q, H, d, lens, dtypes, block, density, cuts, empty q-block rows)
    "d128_two_groups": (300, 2, 128, [77, 300, 130], ["bf16", "bf16", "bf16"], 128, 1.0, [2], ()),
    "d128_int8_three_groups": (257, 3, 128, [64, 200, 257], ["int8", "int8", "bf16"], 32, 0.6, [1, 2], (3,)),
    "d64_sparse": (190, 2, 64, [33, 190, 64], ["bf16", "int8", "bf16"], 16, 0.4, [1], (0,)),
    "empty_group": (96, 1, 128, [100, 0, 60], ["bf16", "bf16", "bf16"], 32, 1.0, [1, 2], ()),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_split_kv_matches_whole_cache_attention(name):
    n_q, H, d, lens, dts, B, dens, cuts, empty = CASES[name]
    seed = sum(map(ord, name))
    q = W.normal_bf16(seed, 0, (n_q, H, d))
    segs = _segments(seed, lens, dts, H, d)
    nqb, nkb = -(-n_q // B), sum(-(-L // B) for L in lens)
    mask = (np.random.default_rng([seed, 5]).random((nqb, nkb)) < dens).astype(np.uint8)
    for r in empty:
        mask[r] = 0
    _say("split-kv", name)
    parts = []
    for a, b in _groups(len(segs), cuts):
        sub_mask = np.ascontiguousarray(mask[:, _columns(lens, B, a, b)])
        O, L = run_partial(q, segs[a:b], sub_mask, B, B)
        O_ref, L_ref = oracle.attention(q, segs[a:b], sub_mask, B, B)
        _assert_partial_close(O, L, O_ref, L_ref, f"{name} part {a}:{b}")
        parts.append((O, L))
    out, lse = run_merge(parts, n_q, H, d)
    O_all, L_all = oracle.attention(q, segs, mask, B, B)
    e = assert_attn_close(out, lse, O_all, L_all, name)
    _say(f"   merged vs whole cache: max-abs {e[0]:.2e} ({e[2]:.2e} beyond half an ulp), rel-RMS {e[1]:.2e}")
    # and against the single-launch path on the same inputs
    out1, _ = run_attn(q, segs, mask, B, B)
    _assert_paths_agree(out, out1, name)


@pytest.mark.parametrize("n_parts", [1, 3, 8])
def test_merge_alone_within_one_ulp(n_parts):
    """The merge kernel on oracle partials (cast to fp32) against the oracle's
    merge of the same fp32 values; some rows see nothing in some parts, one
    row sees nothing in any part."""
    rng = np.random.default_rng(n_parts)
    n_q, H, d = 77, 3, 128
    parts = []
    for p in range(n_parts):
        O = rng.normal(size=(n_q, H, d)).astype(np.float32)
        L = (rng.normal(size=(H, n_q)) * 4).astype(np.float32)
        drop = rng.random((H, n_q)) < 0.3
        L[drop] = -np.inf
        O[drop.T] = 0.0
        parts.append((O, L))
    for O, L in parts:           # query 5 sees nothing anywhere
        L[:, 5] = -np.inf
        O[5] = 0.0
    out, lse = run_merge(parts, n_q, H, d)
    O_ref, L_ref = oracle.attention_merge([(O.astype(np.float64), L.astype(np.float64)) for O, L in parts])
    g = bf16_to_float(out)
    ulp = np.maximum(np.abs(O_ref), 2.0 ** -126)
    ulp = 2.0 ** (np.floor(np.log2(ulp)) - 7)
    assert np.all(np.abs(g - O_ref) <= ulp)
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isneginf(lse), ~fin)
    assert float(np.abs(lse[fin] - L_ref[fin]).max()) <= 1e-5
    assert np.all(out[5] == 0)


def test_wan_chunk_split_cache_and_current_sampled():
    """Wan-chunk shape at full size, keys split into the cache (text +
    history) and the current chunk: GPU partials and merge against the
    oracle's whole-cache attention on sampled rows, and against the
    single-launch GPU path on every row."""
    cfg = W.WORKLOADS["wan13b"]
    inp = W.make_inputs(cfg)
    H, d, n_q, B = cfg.n_heads, cfg.head_dim, cfg.n_q, cfg.block
    segs = [{"k": k, "v": v, "dtype": "bf16"} for k, v in zip(inp.cache_k, inp.cache_v)]
    segs.append({"k": inp.k, "v": inp.v, "dtype": "bf16"})
    lens = [s["k"].shape[0] for s in segs]
    _say("split-kv full size wan13b", lens)
    parts = []
    for a, b in [(0, len(segs) - 1), (len(segs) - 1, len(segs))]:
        sub_mask = np.ascontiguousarray(inp.mask[:, _columns(lens, B, a, b)])
        parts.append(run_partial(inp.q, segs[a:b], sub_mask, B, B))
    out, lse = run_merge(parts, n_q, H, d)
    rng = np.random.default_rng(cfg.seed)
    rows = np.array(sorted(set(rng.choice(n_q, size=24, replace=False).tolist()) | {0, 255, 256, n_q - 1}))
    O, LSE = oracle.attention(inp.q, segs, inp.mask, B, B, rows=rows)
    e = assert_attn_close(out[rows], lse[:, rows], O, LSE, "wan13b split")
    _say(f"   {len(rows)} rows: max-abs {e[0]:.2e} ({e[2]:.2e} beyond half an ulp), rel-RMS {e[1]:.2e}")
    out1, _ = run_attn(inp.q, segs, inp.mask, B, B)
    _assert_paths_agree(out, out1, "wan13b split")
