"""Shared test helpers: moving seeded inputs to the GPU, calling the HIP path
through the C ABI, and comparing against the oracle. Nothing here computes
any part of the method."""
from __future__ import annotations

import numpy as np

import workloads as W

ATOL_O = 4e-3     # max-abs on bf16 attention outputs vs the unrounded fp64 oracle:
                  # |gpu - ref| <= ATOL_O wherever a correctly rounded bf16 output
                  # is within HALF_ULP_CAP of ref (|ref| < 1); above that the bar
                  # applies to the error beyond the output's own rounding,
                  # |gpu - ref| <= ATOL_O + ulp_bf16(ref) / 2
HALF_ULP_CAP = 2e-3
RRMS_O = 1e-2     # relative RMS, ||gpu - ref||_2 / ||ref||_2
ATOL_LSE = 1e-3   # natural-log LSE, absolute


def dev(a: np.ndarray):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host_u16(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def empty_bf16(shape):
    import torch
    return torch.empty(shape, dtype=torch.int16, device="cuda")


def ordered(bits: np.ndarray) -> np.ndarray:
    """bf16 bits -> integers that increase with the value (one step = one ulp)."""
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def segments_for_oracle(inp: W.Inputs, k_cur_bits: np.ndarray, quant=None):
    """Oracle segment list [cached..., current chunk(s)]. ``quant`` maps a
    cached segment index to (codes_k, scale_k, codes_v, scale_v)."""
    segs = []
    for i, (k, v) in enumerate(zip(inp.cache_k, inp.cache_v)):
        if quant is not None and i in quant:
            ck, sk, cv, sv = quant[i]
            segs.append({"k": ck, "v": cv, "k_scale": sk, "v_scale": sv, "dtype": "int8"})
        else:
            segs.append({"k": k, "v": v, "dtype": "bf16"})
    for c in range(inp.cfg.n_chunks):
        r = W.chunk_rows(inp.cfg, c)
        segs.append({"k": k_cur_bits[r], "v": inp.v[r], "dtype": "bf16"})
    return segs


def gpu_segments(oracle_segs):
    """Upload an oracle-style segment list; returns (dicts for the binding, keepalive)."""
    import streaming_video_dit_amd as sdit
    out, keep = [], []
    for s in oracle_segs:
        if s["dtype"] == "int8":
            t = [dev(s["k"]), dev(s["v"]), dev(s["k_scale"]), dev(s["v_scale"])]
            keep += t
            out.append(dict(k=t[0], v=t[1], k_scale=t[2], v_scale=t[3], len=s["k"].shape[0], dtype=sdit.SDIT_INT8))
        else:
            t = [dev(s["k"]), dev(s["v"])]
            keep += t
            out.append(dict(k=t[0], v=t[1], len=s["k"].shape[0], dtype=sdit.SDIT_BF16))
    return out, keep


def run_attn(q_bits, oracle_segs, mask, bq, bk, softmax_scale=0.0, lse=True, split_tile=None, library=None):
    """HIP attention via the C ABI; returns (out bits [n_q,H,d], lse [H,n_q] or None).
    split_tile None: sdit_attn_fwd; else sdit_attn_fwd_balanced with that
    split_tile (-1 = the library's plan) and a NaN-filled workspace.
    library: another build of the library (streaming_video_dit_amd.load_library)."""
    import torch
    import streaming_video_dit_amd as sdit
    n_q, H, d = q_bits.shape
    q = dev(q_bits)
    segs, keep = gpu_segments(oracle_segs)
    m = dev(mask.astype(np.uint8))
    out = torch.full((n_q, H, d), -1, dtype=torch.int16, device="cuda")   # NaN-ish fill (0xFFFF)
    l = torch.full((H, n_q), float("nan"), dtype=torch.float32, device="cuda") if lse else None
    if split_tile is None:
        sdit.attn_fwd(q, n_q, segs, m, bq, bk, H, d, out, l, softmax_scale=softmax_scale, library=library)
    else:
        ws = torch.full((sdit.attn_workspace_bytes(d),), 0xFF, dtype=torch.uint8, device="cuda")
        sdit.attn_fwd_balanced(q, n_q, segs, m, bq, bk, H, d, out, ws, l, softmax_scale=softmax_scale,
                               split_tile=split_tile, library=library)
    torch.cuda.synchronize()
    return host_u16(out), (l.cpu().numpy() if lse else None)


def bf16_to_float(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def half_ulp_bf16(ref: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at each value: the error of the correctly rounded output."""
    e = np.frexp(np.abs(ref))[1]
    return np.ldexp(1.0, e - 9)


def attn_tolerance(ref: np.ndarray, v_scale: float = 1.0) -> np.ndarray:
    """Per-element max-abs bar: ATOL_O, plus half a bf16 ulp of ref where that
    half ulp exceeds HALF_ULP_CAP (|ref| >= 1: a correctly rounded bf16 output
    alone may then be more than 4e-3 away; at |ref| >= 2 it always can be).
    The bar is stated for unit-scale V (the workloads' V is N(0, 1));
    attention is linear in V, so for V of RMS v_scale both absolute terms
    scale with it (v_scale = 1 for every workload)."""
    h = half_ulp_bf16(ref)
    return ATOL_O * v_scale + np.where(h > HALF_ULP_CAP * v_scale, h, 0.0)


def attn_errors(out_bits, ref, v_scale: float = 1.0):
    """(max-abs error, relative RMS error, max-abs error beyond half a bf16 ulp
    of ref, largest error / per-element bar)."""
    g = bf16_to_float(out_bits)
    diff = g - ref
    if not diff.size:
        return 0.0, 0.0, 0.0, 0.0
    max_abs = float(np.abs(diff).max())
    beyond = float((np.abs(diff) - half_ulp_bf16(ref)).max())
    worst = float((np.abs(diff) / attn_tolerance(ref, v_scale)).max())
    denom = float(np.sqrt((ref * ref).sum()))
    rrms = float(np.sqrt((diff * diff).sum()) / denom) if denom > 0 else float(np.sqrt((diff * diff).sum()))
    return max_abs, rrms, beyond, worst


def assert_attn_close(out_bits, lse, O_ref, LSE_ref, what="", v_scale: float = 1.0):
    """max-abs within attn_tolerance(ref, v_scale) element by element (plain
    4e-3 for |ref| < 1 at unit-scale V), rel-RMS within RRMS_O, LSE within
    ATOL_LSE, empty rows -inf. Returns (max-abs, rel-RMS, max-abs beyond half
    an ulp)."""
    assert np.all(np.isfinite(bf16_to_float(out_bits))), f"{what}: non-finite output"
    max_abs, rrms, beyond, worst = attn_errors(out_bits, O_ref, v_scale)
    assert worst <= 1.0, (f"{what}: error {worst:.3f} x the per-element bar (max-abs {max_abs:.3e}, "
                          f"{beyond:.3e} beyond half an ulp)")
    assert rrms <= RRMS_O, f"{what}: rel-RMS {rrms:.3e} > {RRMS_O}"
    if lse is not None:
        fin = np.isfinite(LSE_ref)
        assert np.array_equal(np.isfinite(lse), fin), f"{what}: LSE finiteness differs"
        assert np.all(lse[~fin] == -np.inf), f"{what}: empty rows must give LSE = -inf"
        if fin.any():
            err = float(np.abs(lse[fin] - LSE_ref[fin]).max())
            assert err <= ATOL_LSE, f"{what}: LSE error {err:.3e}"
    return max_abs, rrms, beyond
