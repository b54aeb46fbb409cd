"""The synthetic workloads have the token geometry the pages state
(tests/golden/token_geometry.json, each value with its source): 16 px per
token, Wan chunks of 3 latent frames of 480 x 832 px, the SR clip of
1056 x 1056 px, the windowed clip of 2688 x 1536 px in 8 x 8-token windows
with local_range 11. Inputs only: no part of the method is computed here."""
import json
import os

import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "token_geometry.json")
G = json.load(open(GOLDEN))


def test_px_per_token_is_vae_times_patch():
    assert G["vae_downsample"] * G["patch_hw"] == G["px_per_token"]
    assert G["block_tokens_side"] * G["px_per_token"] == G["block_px"]
    # local_range counts windows around the query window: (11 - 1) / 2 windows of 128 px either side
    assert (G["local_range_blocks"] - 1) // 2 * G["block_px"] == G["local_range_px"]


def test_wan_chunk_geometry():
    for name in ("wan13b", "wan13b_int8", "wave_chunks"):
        cfg = W.WORKLOADS[name]
        assert cfg.Hl == G["wan_height_px"] // G["px_per_token"]
        assert cfg.Wl == G["wan_width_px"] // G["px_per_token"]
        assert cfg.T % G["latent_frames_per_chunk_divisor"] == 0
        assert cfg.chunk_tokens == cfg.T * cfg.Hl * cfg.Wl
        # history = whole previous chunks; the last segment(s) are the current chunk(s)
        hist = cfg.seg_lens[1]
        assert hist % cfg.chunk_tokens == 0 and cfg.seg_lens[-1] == cfg.chunk_tokens


def test_sr_clip_geometry():
    cfg = W.WORKLOADS["bsa_sr"]
    side = G["sr_clip_px"] // G["px_per_token"]
    assert (cfg.Hl, cfg.Wl) == (side, side)
    assert cfg.seg_lens == [cfg.T * side * side] and cfg.n_q == cfg.seg_lens[0]


def test_windowed_clip_geometry():
    cfg = W.WORKLOADS["vsr_local"]
    w_px, h_px = G["vsr_timing_clip_px"]
    assert (cfg.Hl, cfg.Wl) == (h_px // G["px_per_token"], w_px // G["px_per_token"])
    assert cfg.window == G["block_tokens_side"] and cfg.block == cfg.window ** 2
    assert cfg.local_range == G["local_range_blocks"]
    assert cfg.Hl % cfg.window == 0 and cfg.Wl % cfg.window == 0
