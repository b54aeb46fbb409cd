#!/usr/bin/env python3
"""Benchmark of the streaming-video-DiT attention core on one MI355X.

One step = one layer-chunk of the hot path on seeded synthetic inputs already
resident in HBM:
    qknorm_rope3d(chunk q, k)            (skipped by the self-attention SR workload)
    kv_quant_int8(chunk K), (chunk V)    (int8-cache workload: the steady-state cache write;
                                          fused with the line above into one
                                          qknorm_rope3d_kv_quant_int8 pass unless
                                          --unfused-cache-write)
    attn_fwd_balanced(q, [cache segments..., current chunk])

The attention call is sdit_attn_fwd_balanced with the library's own plan:
on each XCD the work units of the grid's last partial wave are cut at one
key tile into head and tail pieces, and a second kernel merges the two
pieces (both launches are inside the timed attention). --launch plain times
sdit_attn_fwd instead (one workgroup per unit, no cut, no merge).

With --kv-parts N (N > 1) the attention is the split-KV form instead: the
segments are cut into N groups of consecutive segments, attn_fwd_partial
runs once per group (fp32 partial O and LSE) and attn_merge combines them;
the line then also reports the merge kernel against the HBM roofline.

With --with-norms the line also carries a "norms" object: RMSNorm and
LayerNorm + modulate over the hidden state of the workload's query tokens
(n_q x n_heads*head_dim bf16), each timed alone after the attention steps
against the HBM roofline. They are not part of the step and do not change
``value``.

Prints ONE JSON line. ``value`` is effective attention TFLOP/s of the whole
step (kept-tile FLOPs 4*d*H*sum rows*cols / step time); ``ms_per_step`` is
the ms/layer/chunk. ``roofline`` reports the attention kernel alone, timed
with HIP events around each launch on the stream it runs on.
The attention time covers both launches of the balanced call.
``cpu_baseline`` times the fp64 oracle on the host (heads processed one by
one until about 10 s have elapsed, scaled to TFLOP/s).

By default the line also carries a ``configs`` object with one record per
main workload (tiny, Wan chunk, Wan chunk with an int8 cache, Large-DiT,
block-sparse SR), each timed the same way after the headline workload:
attention ms (mean, median, p10-p90), step ms, effective TFLOP/s and the
fraction of the bf16 peak (the tiny one, which is launch-latency bound,
against its algorithmic bytes instead), HBM traffic where a profile of the
current kernel sources exists, and the oracle's seconds on a bounded sample.
``clocks`` holds the engine and memory clock levels read before and after
the timed work.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "attention ms/layer/chunk + effective TFLOP/s (% bf16 MFMA peak), 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# Q.K^T runs as a bf16 MFMA; P.V multiplies fp16 probabilities with V staged
# in fp16 (same MFMA rate, 3 more mantissa bits for P); accumulation fp32.
DTYPE = "bf16 (P.V in fp16)"


def _dev(a, torch):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


class Step:
    """Device buffers and the launch sequence of one layer-chunk."""

    def __init__(self, cfg: W.Config, torch, sdit, kv_parts: int = 1, launch: str = "balanced",
                 split_tile: int = -1, fused_cache_write: bool = True):
        self.cfg, self.torch, self.sdit = cfg, torch, sdit
        inp = W.make_inputs(cfg)
        self.inp = inp
        H, d, n = cfg.n_heads, cfg.head_dim, cfg.n_q
        self.q_in, self.k_in, self.v = _dev(inp.q, torch), _dev(inp.k, torch), _dev(inp.v, torch)
        self.gq, self.gk = _dev(inp.gamma_q, torch), _dev(inp.gamma_k, torch)
        # padding rows between chunks keep their raw values
        self.q = self.q_in.clone()
        self.k = self.k_in.clone()
        self.out = torch.empty((n, H, d), dtype=torch.int16, device="cuda")
        self.lse = torch.empty((H, n), dtype=torch.float32, device="cuda")
        self.mask = _dev(inp.mask, torch)
        self.keep = []
        segs = []
        for i, (kc, vc) in enumerate(zip(inp.cache_k, inp.cache_v)):
            kd, vd = _dev(kc, torch), _dev(vc, torch)
            L = kc.shape[0]
            if cfg.seg_int8[i]:
                ck = torch.empty((L, H, d), dtype=torch.int8, device="cuda")
                cv = torch.empty((L, H, d), dtype=torch.int8, device="cuda")
                sk = torch.empty((L, H), dtype=torch.float32, device="cuda")
                sv = torch.empty((L, H), dtype=torch.float32, device="cuda")
                sdit.kv_quant_int8(kd, ck, sk, L, H, d)
                sdit.kv_quant_int8(vd, cv, sv, L, H, d)
                self.keep += [ck, cv, sk, sv]
                segs.append(dict(k=ck, v=cv, k_scale=sk, v_scale=sv, len=L, dtype=sdit.SDIT_INT8))
            else:
                self.keep += [kd, vd]
                segs.append(dict(k=kd, v=vd, len=L, dtype=sdit.SDIT_BF16))
        cur_k, cur_v = (self.k if cfg.rope else self.k_in), self.v
        if cfg.window:
            # windowed attention runs on window-major copies; the output is put back in raster order
            self.q_w, self.k_w, self.v_w = (torch.empty_like(self.q_in) for _ in range(3))
            self.out_w = torch.empty_like(self.out)
            cur_k, cur_v = self.k_w, self.v_w
        for c in range(cfg.n_chunks):
            rows = W.chunk_rows(cfg, c)
            segs.append(dict(k=cur_k[rows], v=cur_v[rows], len=cfg.chunk_tokens, dtype=sdit.SDIT_BF16))
        self.segs = sdit.make_segments(segs)
        self.n_segs = len(segs)
        # split-KV form: groups of consecutive segments, each with its own mask columns
        self.kv_parts = kv_parts
        if kv_parts > 1:
            if kv_parts > len(segs):
                raise ValueError(f"--kv-parts {kv_parts} > {len(segs)} segments")
            cuts = np.linspace(0, len(segs), kv_parts + 1).round().astype(int)
            starts = np.cumsum([0] + [-(-int(sg["len"]) // cfg.block) for sg in segs])
            self.groups = []
            for a, b in zip(cuts[:-1], cuts[1:]):
                cols = np.ascontiguousarray(inp.mask[:, starts[a]:starts[b]])
                o = torch.empty((n, H, d), dtype=torch.float32, device="cuda")
                ls = torch.empty((H, n), dtype=torch.float32, device="cuda")
                self.groups.append((sdit.make_segments(segs[a:b]), b - a, _dev(cols, torch), o, ls))
            self.merge_bytes = (kv_parts * (4 * d + 4) + 2 * d + 4) * n * H
        self.q_attn = self.q_w if cfg.window else (self.q if cfg.rope else self.q_in)
        self.launch = launch
        self.n_tiles = sum(-(-int(sg["len"]) // 64) for sg in segs)
        self.plan = (0, cfg.n_heads * -(-n // 256))
        if launch == "balanced":
            self.ws = torch.empty((sdit.attn_workspace_bytes(d),), dtype=torch.uint8, device="cuda")
            cus = torch.cuda.get_device_properties(0).multi_processor_count
            self.split_tile = split_tile
            self.plan = sdit.attn_balanced_plan(n, H, self.n_tiles, cus, split_tile)
        self.quant_chunk = any(cfg.seg_int8)
        self.fused = fused_cache_write and self.quant_chunk and cfg.rope and cfg.n_chunks == 1
        if self.quant_chunk:
            self.ck = torch.empty((n, H, d), dtype=torch.int8, device="cuda")
            self.cv = torch.empty((n, H, d), dtype=torch.int8, device="cuda")
            self.sk = torch.empty((n, H), dtype=torch.float32, device="cuda")
            self.sv = torch.empty((n, H), dtype=torch.float32, device="cuda")
        self.flops = W.attn_flops(cfg, inp.mask)
        torch.cuda.synchronize()

    def run(self, ev_before=None, ev_after=None, ev_merge=None):
        cfg, sdit = self.cfg, self.sdit
        H, d, n = cfg.n_heads, cfg.head_dim, cfg.n_q
        if self.fused:
            # rotated q, k and the chunk's int8 cache entries in one pass
            dt, dh, dw = cfg.split
            sdit.qknorm_rope3d_kv_quant_int8(self.q_in, self.k_in, self.v, self.q, self.k, self.ck, self.sk, self.cv,
                                             self.sv, self.gq, self.gk, cfg.T, cfg.Hl, cfg.Wl, cfg.t0, H, d, dt, dh,
                                             dw, cfg.theta, cfg.eps)
        else:
            if cfg.rope:
                dt, dh, dw = cfg.split
                for c in range(cfg.n_chunks):
                    r = W.chunk_rows(cfg, c)
                    sdit.qknorm_rope3d(self.q_in[r], self.k_in[r], self.q[r], self.k[r], self.gq, self.gk, cfg.T,
                                       cfg.Hl, cfg.Wl, cfg.t0 + c * cfg.T, H, d, dt, dh, dw, cfg.theta, cfg.eps)
            if self.quant_chunk:   # single-chunk workloads only
                sdit.kv_quant_int8(self.k, self.ck, self.sk, n, H, d)
                sdit.kv_quant_int8(self.v, self.cv, self.sv, n, H, d)
        if cfg.window:
            for src, dst in ((self.q_in, self.q_w), (self.k_in, self.k_w), (self.v, self.v_w)):
                sdit.window_permute(src, dst, cfg.T, cfg.Hl, cfg.Wl, H, d, cfg.window)
        out = self.out_w if cfg.window else self.out
        if ev_before is not None:
            ev_before.record()
        if self.kv_parts > 1:
            for segs, n_segs, mask, o, ls in self.groups:
                sdit.attn_fwd_partial(self.q_attn, n, segs, mask, cfg.block, cfg.block, H, d, o, ls)
            if ev_merge is not None:
                ev_merge.record()
            sdit.attn_merge([g[3] for g in self.groups], [g[4] for g in self.groups], n, H, d, out, self.lse)
        elif self.launch == "balanced":
            sdit.attn_fwd_balanced(self.q_attn, n, self.segs, self.mask, cfg.block, cfg.block, H, d, out, self.ws,
                                   self.lse, split_tile=self.split_tile)
        else:
            sdit.attn_fwd(self.q_attn, n, self.segs, self.mask, cfg.block, cfg.block, H, d, out, self.lse)
        if ev_after is not None:
            ev_after.record()
        if cfg.window:
            sdit.window_permute(self.out_w, self.out, cfg.T, cfg.Hl, cfg.Wl, H, d, cfg.window, inverse=True)


def attn_algorithmic_bytes(cfg: W.Config, mask) -> int:
    """One pass over every operand of one attention call: q, each segment's K
    and V (int8 codes plus their fp32 scales, or bf16), the bf16 output, the
    fp32 LSE and the mask."""
    H, d, n = cfg.n_heads, cfg.head_dim, cfg.n_q
    b = 2 * n * H * d * 2 + 4 * H * n + int(np.asarray(mask).size)
    for L, i8 in zip(cfg.seg_lens, cfg.seg_int8):
        b += 2 * L * H * d * (1 if i8 else 2) + (2 * L * H * 4 if i8 else 0)
    return b


def read_clocks():
    """Current engine (sclk) and memory (mclk) clock levels in MHz from the
    driver's sysfs files (the line marked '*'), or None where unreadable."""
    import glob
    out = {}
    for key in ("sclk", "mclk"):
        val = None
        for f in sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{key}")):
            try:
                for line in open(f):
                    if line.rstrip().endswith("*"):
                        val = int("".join(ch for ch in line.split(":", 1)[1] if ch.isdigit()))
            except (OSError, ValueError, IndexError):
                continue
            if val is not None:
                break
        out[key + "_mhz"] = val
    return out


def device_info(torch):
    """What the peak figure rests on: the device's compute-unit count (one
    bf16 32x32x16 MFMA per 32 cycles per SIMD, 4 SIMDs per CU, at the
    published 2.4 GHz peak engine clock)."""
    pr = torch.cuda.get_device_properties(0)
    cus = int(pr.multi_processor_count)
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", ""), "compute_units": cus,
            "peak_bf16_tflops_from_cus": round(cus * 4 * 32768 / 32 * 2.4e9 / 1e12, 1)}


def measure_norms(cfg: W.Config, torch, sdit, steps: int, warmup: int):
    """Average launch time and HBM rate of the two per-token norms on the
    workload's hidden-state shape (algorithmic bytes: x read and y written
    once, 2 + 2 bytes per element, plus the fp32 parameter vectors once)."""
    n, d = cfg.n_q, cfg.n_heads * cfg.head_dim
    inp = W.make_norm_inputs(cfg.seed, n, d, offset=1.0)
    # successive launches cycle through enough input/output sets to exceed the
    # 256 MB last-level cache, so the figures are HBM rates
    n_sets = max(2, -(-768 * 2**20 // (4 * n * d)))
    xs = [_dev(inp.x, torch) for _ in range(n_sets)]
    ys = [torch.empty_like(xs[0]) for _ in range(n_sets)]
    g, sc, sh = _dev(inp.gamma, torch), _dev(inp.scale, torch), _dev(inp.shift, torch)
    launches = {
        "rmsnorm": (lambda i: sdit.rmsnorm(xs[i], ys[i], g, n, d), 4 * n * d + 4 * d),
        "layernorm_modulate": (lambda i: sdit.layernorm_modulate(xs[i], ys[i], sc, sh, n, d), 4 * n * d + 8 * d),
    }
    res = {"shape": [n, d], "input_sets": n_sets}
    stream = torch.cuda.current_stream()
    for name, (fn, nbytes) in launches.items():
        for i in range(warmup):
            fn(i % n_sets)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            fn(i % n_sets)
            b.record(stream)
        torch.cuda.synchronize()
        us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = {"kernel": f"norm_kernel<{(d // 8 + 63) // 64}, {'true' if name != 'rmsnorm' else 'false'}>",
                     "bound": "hbm", "us": round(us, 2), "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": nbytes}
    return res


def _time_rotating(torch, fn, n_sets: int, steps: int, warmup: int, settle_s: float = 0.2):
    """Median, p10 and p90 (us) of single launches fn(i), timed with HIP
    events on the current stream, cycling through n_sets buffer sets (after
    about settle_s seconds of untimed launches and the warmup ones)."""
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < settle_s:
        fn(i % n_sets)
        i += 1
    for i in range(warmup):
        fn(i % n_sets)
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        fn(i % n_sets)
        b.record(stream)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
    return float(np.median(us)), float(np.percentile(us, 10)), float(np.percentile(us, 90))


def _hbm_entry(kernel: str, shape, nbytes: int, n_sets: int, t):
    med, p10, p90 = t
    gbs = nbytes / (med * 1e-6) / 1e9
    return {"kernel": kernel, "shape": list(shape), "bound": "hbm", "us_median": round(med, 2),
            "us_p10_p90": [round(p10, 2), round(p90, 2)], "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": nbytes, "input_sets": n_sets}


def measure_hbm_kernels(cfg: W.Config, torch, sdit, steps: int, warmup: int):
    """The HBM-bound kernels of the step, each launch timed alone: qknorm_rope3d
    of the chunk's q and k (2 * 2 * 2 bytes per element: q and k read and
    written, plus the two fp32 gamma vectors), and kv_quant_int8 (2 bytes read,
    1 written per element, 4 per (token, head) scale) of the chunk's K and of
    the cached segments' K. Successive launches cycle through enough buffer
    sets to exceed 768 MB, so the 256 MB last-level cache does not serve them."""
    H, d, n = cfg.n_heads, cfg.head_dim, cfg.n_q
    res = {}

    def sets_for(nbytes):
        return max(3, -(-768 * 2**20 // nbytes))

    if cfg.rope:
        inp = W.make_inputs(cfg)
        r = W.chunk_rows(cfg, 0)
        q0, k0 = inp.q[r], inp.k[r]
        m = q0.shape[0]
        dt, dh, dw = cfg.split
        nbytes = 2 * 2 * 2 * m * H * d + 2 * 4 * d
        ns = sets_for(nbytes)
        qs = [_dev(q0, torch) for _ in range(ns)]
        ks = [_dev(k0, torch) for _ in range(ns)]
        qo = [torch.empty_like(qs[0]) for _ in range(ns)]
        ko = [torch.empty_like(ks[0]) for _ in range(ns)]
        gq, gk = _dev(inp.gamma_q, torch), _dev(inp.gamma_k, torch)
        t = _time_rotating(torch, lambda i: sdit.qknorm_rope3d(qs[i], ks[i], qo[i], ko[i], gq, gk, cfg.T, cfg.Hl, cfg.Wl,
                                                               cfg.t0, H, d, dt, dh, dw, cfg.theta, cfg.eps),
                           ns, steps, warmup)
        res["qknorm_rope3d_chunk"] = _hbm_entry(f"qknorm_rope3d_kernel<{d}, false>", (m, H, d), nbytes, ns, t)
        del qs, ks, qo, ko
        if any(cfg.seg_int8):
            # the fused pass: q, k, v read, q and k written, int8 codes + fp32 scales of k and v written
            v0 = inp.v[r]
            nbytes = 3 * 2 * m * H * d + 2 * 2 * m * H * d + 2 * (m * H * d + 4 * m * H) + 2 * 4 * d
            ns = sets_for(nbytes)
            qs = [_dev(q0, torch) for _ in range(ns)]
            ks = [_dev(k0, torch) for _ in range(ns)]
            vs = [_dev(v0, torch) for _ in range(ns)]
            qo = [torch.empty_like(qs[0]) for _ in range(ns)]
            ko = [torch.empty_like(ks[0]) for _ in range(ns)]
            kc = [torch.empty((m, H, d), dtype=torch.int8, device="cuda") for _ in range(ns)]
            vc = [torch.empty((m, H, d), dtype=torch.int8, device="cuda") for _ in range(ns)]
            ksc = [torch.empty((m, H), dtype=torch.float32, device="cuda") for _ in range(ns)]
            vsc = [torch.empty((m, H), dtype=torch.float32, device="cuda") for _ in range(ns)]
            t = _time_rotating(torch, lambda i: sdit.qknorm_rope3d_kv_quant_int8(
                qs[i], ks[i], vs[i], qo[i], ko[i], kc[i], ksc[i], vc[i], vsc[i], gq, gk, cfg.T, cfg.Hl, cfg.Wl,
                cfg.t0, H, d, dt, dh, dw, cfg.theta, cfg.eps), ns, steps, warmup)
            res["qknorm_rope3d_kv_quant_int8_chunk"] = _hbm_entry(f"qknorm_rope3d_kernel<{d}, true>", (m, H, d),
                                                                  nbytes, ns, t)
            del qs, ks, vs, qo, ko, kc, vc, ksc, vsc
    n_cache = sum(cfg.seg_lens[:cfg.n_cached])
    for label, n_tok in (("kv_quant_int8_chunk", cfg.chunk_tokens), ("kv_quant_int8_cache", n_cache)):
        if n_tok == 0:
            continue
        nbytes = n_tok * H * d * 3 + n_tok * H * 4
        ns = sets_for(nbytes)
        x = W.normal_bf16(cfg.seed, 90, (n_tok, H, d))
        xs = [_dev(x, torch) for _ in range(ns)]
        cs = [torch.empty((n_tok, H, d), dtype=torch.int8, device="cuda") for _ in range(ns)]
        ss = [torch.empty((n_tok, H), dtype=torch.float32, device="cuda") for _ in range(ns)]
        t = _time_rotating(torch, lambda i: sdit.kv_quant_int8(xs[i], cs[i], ss[i], n_tok, H, d), ns, steps, warmup)
        res[label] = _hbm_entry(f"kv_quant_int8_kernel<{d}>", (n_tok, H, d), nbytes, ns, t)
        del xs, cs, ss
    return res


def attn_src_hash() -> str:
    """sha256 prefix of the attention kernels' sources (attn_fwd.hip, then
    attn_merge.hip, which holds the merge of a balanced launch)."""
    h = hashlib.sha256()
    for f in ("attn_fwd.hip", "attn_merge.hip"):
        h.update(open(os.path.join(ROOT, "streaming_video_dit_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per attention call (the attention kernel, plus the merge
    kernel when the balanced plan cuts) from the rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs summarised under profiles/ (calibrated against a plain
    copy). The figures belong to one version of the kernel sources: once
    they have changed they no longer describe them and None is returned."""
    f = os.path.join(ROOT, "profiles", "attn_fwd_traffic.json")
    if not os.path.exists(f):
        return None
    t = json.load(open(f))
    if attn_src_hash() != t.get("attn_src_sha256_16"):
        return None
    w = t["workloads"].get(workload)
    return None if w is None else int(w["fetch_bytes"] + w["write_bytes"])


def cpu_baseline(cfg: W.Config, budget_s: float = 10.0):
    """The oracle as it stands, on the host: qknorm_rope3d of the chunk (and
    the int8 quantisation of the cache for the int8 workload) once, then
    attention head by head until ``budget_s`` has elapsed. Scaled to TFLOP/s
    over the heads done, with the one-off work charged in full."""
    import oracle
    try:
        import threadpoolctl
        threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    inp = W.make_inputs(cfg)
    t0 = time.perf_counter()
    rq, rk = inp.q.copy(), inp.k.copy()
    if cfg.rope:
        dt, dh, dw = cfg.split
        for c in range(cfg.n_chunks):
            r = W.chunk_rows(cfg, c)
            f0 = cfg.t0 + c * cfg.T   # the chunk's first frame position
            rq[r] = oracle.qknorm_rope3d(inp.q[r], inp.gamma_q, cfg.T, cfg.Hl, cfg.Wl, f0, dt, dh, dw)
            rk[r] = oracle.qknorm_rope3d(inp.k[r], inp.gamma_k, cfg.T, cfg.Hl, cfg.Wl, f0, dt, dh, dw)
    segs = []
    for i, (k, v) in enumerate(zip(inp.cache_k, inp.cache_v)):
        if cfg.seg_int8[i]:
            ck, sk = oracle.kv_quant_int8(k)
            cv, sv = oracle.kv_quant_int8(v)
            segs.append({"k": ck, "v": cv, "k_scale": sk, "v_scale": sv, "dtype": "int8"})
        else:
            segs.append({"k": k, "v": v, "dtype": "bf16"})
    v = inp.v
    if cfg.window:
        order = oracle.window_order(cfg.T, cfg.Hl, cfg.Wl, cfg.window)
        rq, rk, v = rq[order], rk[order], v[order]
    for c in range(cfg.n_chunks):
        r = W.chunk_rows(cfg, c)
        segs.append({"k": rk[r], "v": v[r], "dtype": "bf16"})
    heads = 0
    while heads < cfg.n_heads:
        oracle.attention(rq, segs, inp.mask, cfg.block, cfg.block, heads=[heads])
        heads += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    flops = W.attn_flops(cfg, inp.mask) * heads / cfg.n_heads
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "seconds": el,
            "sample": f"{cfg.name}: " + " + ".join(
                (["qknorm_rope3d of the whole chunk"] if cfg.rope else [])
                + (["int8 quantisation of the cache"] if any(cfg.seg_int8) else [])
                + [f"attention for {heads} of {cfg.n_heads} heads"]) + f", fp64 numpy, {el:.1f} s"}


# Untimed steps run back to back before the warmup steps, for at least this
# long: from idle the engine clock needs a few hundred milliseconds of
# continuous load to reach its sustained level (measured on MI355X: ~1.1 GHz
# at the start of a Wan-chunk run, ~2.2 GHz after 0.3-0.5 s, the attention
# call 0.69 ms over the first 20 steps and 0.60 ms from step ~50 on).
SETTLE_S = 0.5


def settle_clock(step: "Step", torch, seconds: float):
    """Run untimed steps back to back for about ``seconds`` (step count from a
    short timed probe), so that the timed steps run at the sustained clock.
    Returns (steps run, wall seconds)."""
    if seconds <= 0:
        return 0, 0.0
    t0 = time.perf_counter()
    for _ in range(3):
        step.run()
    torch.cuda.synchronize()
    per = max((time.perf_counter() - t0) / 3, 1e-5)
    n = int(min(20000, max(1, seconds / per)))
    for _ in range(n):
        step.run()
    torch.cuda.synchronize()
    return n + 3, time.perf_counter() - t0


def time_step(step: "Step", torch, steps: int, warmup: int, with_merge: bool = False,
              settle_s: float = SETTLE_S):
    """Clock settling (untimed steps for settle_s seconds), W untimed steps,
    then K steps bracketed by events; per-step attention events on the launch
    stream. The events exist before the untimed steps start, so nothing but a
    synchronisation separates the last untimed step from the first timed one.
    Returns (ms per step, attention ms per call list, events, wall seconds,
    (settle steps, settle seconds))."""
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3 if with_merge else 2)) for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    settle = settle_clock(step, torch, settle_s)
    for _ in range(warmup):
        step.run()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for i in range(steps):
        step.run(*evs[i])
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    return start.elapsed_time(end) / steps, [e[0].elapsed_time(e[1]) for e in evs], evs, t_wall, settle


def config_record(cfg: W.Config, torch, sdit, steps: int, warmup: int, cpu_budget: float, step=None, timing=None,
                  cpu=None, settle_s: float = SETTLE_S):
    """One workload's record for the ``configs`` object: the balanced
    attention call of the library's plan inside the full step (``step`` and
    ``timing`` reuse the headline measurement, ``cpu`` its oracle timing)."""
    if step is None:
        step = Step(cfg, torch, sdit)
    ms_step, attn_ms, _, _, _ = (timing if timing is not None
                                 else time_step(step, torch, steps, warmup, settle_s=settle_s))
    a = np.asarray(attn_ms)
    med = float(np.median(a))
    rec = {"description": cfg.description, "n_heads": cfg.n_heads, "head_dim": cfg.head_dim, "n_q": cfg.n_q,
           "segments": cfg.seg_lens, "int8_segments": cfg.seg_int8, "block": cfg.block,
           "kept_tiles": int(step.inp.mask.sum()), "mask_tiles": int(step.inp.mask.size),
           "effective_gflop": round(step.flops / 1e9, 6), "cut_at_tile": step.plan[0],
           "attn_workgroups": step.plan[1],
           "attn_ms": round(float(a.mean()), 5), "attn_ms_median": round(med, 5),
           "attn_ms_p10_p90": [round(float(np.percentile(a, 10)), 5), round(float(np.percentile(a, 90)), 5)],
           "step_ms": round(ms_step, 5)}
    tflops = step.flops / (float(a.mean()) * 1e-3) / 1e12
    nbytes = attn_algorithmic_bytes(cfg, step.inp.mask)
    rec["tflops"] = round(tflops, 3)
    rec["pct_bf16_peak"] = round(100 * tflops / PEAK_BF16_TFLOPS, 2)
    if cfg.name == "tiny":
        gbs = nbytes / (float(a.mean()) * 1e-3) / 1e9
        rec["roofline"] = {"bound": "latency", "achieved": round(gbs, 3), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": round(gbs / PEAK_HBM_GBS, 6), "algorithmic_bytes": nbytes,
                           "traffic": measured_traffic(cfg.name)}
    else:
        rec["roofline"] = {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "algorithmic_bytes": nbytes,
                           "traffic": measured_traffic(cfg.name)}
    if cpu is not None or cpu_budget > 0:
        cb = cpu if cpu is not None else cpu_baseline(cfg, cpu_budget)
        rec["cpu_baseline"] = {"seconds": round(cb["seconds"], 3), "value": cb["value"], "unit": cb["unit"],
                               "cores": cb["cores"], "sample": cb["sample"]}
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-s", type=float, default=SETTLE_S,
                    help="seconds of untimed steps before the warmup steps (engine clock ramp; 0: none)")
    ap.add_argument("--workload", default="wan13b", choices=sorted(W.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--kv-parts", type=int, default=1,
                    help="split-KV form: attention over this many groups of segments, then the merge")
    ap.add_argument("--launch", choices=["balanced", "plain"], default="balanced",
                    help="attention entry point: sdit_attn_fwd_balanced (library plan) or sdit_attn_fwd")
    ap.add_argument("--split-tile", type=int, default=-1,
                    help="balanced launch: key tile of the cut (-1: the library's plan, 0: none)")
    ap.add_argument("--unfused-cache-write", action="store_true",
                    help="int8-cache workload: qknorm_rope3d and two kv_quant_int8 launches instead of the fused pass")
    ap.add_argument("--with-hbm", action="store_true",
                    help="also time qknorm_rope3d and kv_quant_int8 alone (rotated input sets) against 8 TB/s")
    ap.add_argument("--with-norms", action="store_true",
                    help="also time RMSNorm and LayerNorm + modulate on the workload's hidden-state shape")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (calibrates HBM byte counters)")
    ap.add_argument("--configs", default=",".join(W.WORKLOAD_ORDER),
                    help="comma-separated workloads timed after the headline one for the 'configs' object "
                         "('none' to skip)")
    ap.add_argument("--config-cpu-budget", type=float, default=3.0,
                    help="seconds of oracle time per entry of the 'configs' object (0: none)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the kernel runs on one GPU's share; sharding is described in the design notes).",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import streaming_video_dit_amd as sdit
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": max(1, args.steps)}), flush=True)
        return

    cfg = W.WORKLOADS[args.workload]
    clocks = {"before": read_clocks()}
    step = Step(cfg, torch, sdit, args.kv_parts, args.launch, args.split_tile,
                fused_cache_write=not args.unfused_cache_write)
    # determinism: the output of two identical steps must be bit-identical
    # (checked first: the host-side hashing leaves the GPU idle)
    step.run()
    torch.cuda.synchronize()
    h1 = hashlib.md5(step.out.cpu().numpy().tobytes()).hexdigest()
    step.run()
    torch.cuda.synchronize()
    h2 = hashlib.md5(step.out.cpu().numpy().tobytes()).hexdigest()

    timing = time_step(step, torch, args.steps, args.warmup, with_merge=args.kv_parts > 1,
                       settle_s=args.settle_s)
    ms_step, attn_ms, evs, t_wall, settle = timing
    clocks["after"] = read_clocks()
    attn_avg = float(np.mean(attn_ms))
    value = step.flops / (ms_step * 1e-3) / 1e12
    attn_tflops = step.flops / (attn_avg * 1e-3) / 1e12

    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "data": "synthetic",
        "config": {"workload": cfg.name, "description": cfg.description, "n_heads": cfg.n_heads,
                   "head_dim": cfg.head_dim, "n_q": cfg.n_q, "segments": cfg.seg_lens,
                   "int8_segments": cfg.seg_int8, "block": cfg.block,
                   "kept_tiles": int(step.inp.mask.sum()), "mask_tiles": int(step.inp.mask.size),
                   "effective_gflop": round(step.flops / 1e9, 3), "parallelism": "none (1 GPU)",
                   "launch": args.launch if args.kv_parts == 1 else "split-kv",
                   "key_tiles": step.n_tiles, "cut_at_tile": step.plan[0], "attn_workgroups": step.plan[1],
                   "cache_write": "fused" if step.fused else ("separate" if step.quant_chunk else "none")},
        "attn_ms": round(attn_avg, 5),
        "attn_ms_median": round(float(np.median(attn_ms)), 5),
        "attn_ms_p10_p90": [round(float(np.percentile(attn_ms, 10)), 5), round(float(np.percentile(attn_ms, 90)), 5)],
        "pct_bf16_peak_step": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "pct_bf16_peak_attn": round(100 * attn_tflops / PEAK_BF16_TFLOPS, 2),
        "deterministic": h1 == h2,
        "device": device_info(torch),
        "clocks": clocks,
        "wall_s_timed": round(t_wall, 3),
        "clock_settle": {"untimed_steps": settle[0], "seconds": round(settle[1], 3),
                         "note": "untimed steps run back to back before the warmup steps, so that the "
                                 "timed steps see the sustained engine clock"},
        "roofline": {"kernel": (f"attn_fwd_kernel<{cfg.head_dim}>"
                               + (f" + attn_split_merge_kernel<{cfg.head_dim}>" if step.plan[0] > 0 else "")),
                     "bound": "mfma", "achieved": round(attn_tflops, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(cfg.name)},
    }
    if args.kv_parts > 1:
        merge_ms = float(np.mean([e[2].elapsed_time(e[1]) for e in evs]))
        gbs = step.merge_bytes / (merge_ms * 1e-3) / 1e9
        rec["config"]["kv_parts"] = args.kv_parts
        rec["merge"] = {"kernel": "attn_merge_kernel", "bound": "hbm", "us": round(merge_ms * 1e3, 2),
                        "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": step.merge_bytes}
        rec["roofline"]["traffic"] = None
    if args.with_hbm:
        rec["hbm_kernels"] = measure_hbm_kernels(cfg, torch, sdit, args.steps, args.warmup)
    if args.with_norms:
        rec["norms"] = measure_norms(cfg, torch, sdit, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget)
    names = [] if args.configs in ("", "none") else [n for n in args.configs.split(",") if n]
    if names:
        configs = {}
        headline_plain = args.kv_parts == 1 and args.launch == "balanced" and args.split_tile == -1
        cpu_budget = 0.0 if args.no_cpu_baseline else args.config_cpu_budget
        for name in names:
            if name == cfg.name and headline_plain:
                configs[name] = config_record(cfg, torch, sdit, args.steps, args.warmup, cpu_budget, step=step,
                                              timing=timing, cpu=rec.get("cpu_baseline"))
            else:
                c = W.WORKLOADS[name]
                configs[name] = config_record(c, torch, sdit, args.steps, args.warmup, cpu_budget,
                                              settle_s=args.settle_s)
                torch.cuda.empty_cache()
        rec["configs"] = configs
        rec["clocks"]["after_configs"] = read_clocks()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
