"""Seeded synthetic inputs for the streaming-video-DiT attention core.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic (no normalisation, rotation, quantisation or attention),
so both the oracle-side tests and the HIP-side tests/bench may import it.

Shapes follow the pages' workloads:
  * latent token geometry: 8x VAE downsampling and a [1,2,2] patch give one
    token per 16x16 pixels (FlashVSR deployment notes, spatial tiling section);
    Wan2.1 at 832x480 gives 30x52 tokens per latent frame and chunks of three
    latent frames (Wave Forcing summary, usage section);
  * the K/V cache is [cached text | history chunks or reference image |
    current chunk] (Joy-face_change_optimized README, section 1, item 1);
  * the int8 cache has one scale per (token, head) (same README, section 1,
    int8 K/V bullet);
  * block-sparse attention takes a (q-block, k-block) keep mask
    (FlashVSR deployment notes, Block-Sparse-Attention kernel section).

Every tensor has its own stream ``np.random.default_rng([seed, tid])``.
Normals are drawn in fp64, rounded to fp32, then to bf16 (round to nearest
even on the bit pattern); bf16 tensors are returned as ``uint16`` bit arrays.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

# Stream ids, one per generated tensor.
TID_Q, TID_K, TID_V = 0, 1, 2
TID_TEXT_K, TID_TEXT_V = 3, 4
TID_HIST_K, TID_HIST_V = 5, 6
TID_GAMMA_Q, TID_GAMMA_K = 7, 8
TID_K_OUTLIER, TID_V_OUTLIER = 9, 10
TID_HIDDEN, TID_CH_SCALE, TID_TOK_OFFSET, TID_GAMMA, TID_MOD_SCALE, TID_MOD_SHIFT = 11, 12, 13, 14, 15, 16
TID_TILE_MASK = 100


def _f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the bits."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def normal_bf16(seed: int, tid: int, shape, outlier_p: float = 0.0,
                outlier_mult: float = 8.0, outlier_tid: Optional[int] = None, sigma: float = 1.0) -> np.ndarray:
    """N(0, sigma^2) samples as bf16 bits (sigma scales the fp64 draw before
    the roundings). With ``outlier_p`` > 0 each element is, independently,
    multiplied by ``outlier_mult`` with that probability (the multiplication
    by a power of two happens before the bf16 rounding and is exact)."""
    rng = np.random.default_rng([seed, tid])
    x = rng.standard_normal(size=shape) * sigma
    if outlier_p > 0.0:
        assert outlier_tid is not None
        orng = np.random.default_rng([seed, outlier_tid])
        hit = orng.random(size=shape) < outlier_p
        x = np.where(hit, x * outlier_mult, x)
    return _f32_to_bf16_bits(x.astype(np.float32))


def signed_uniform_bf16(seed: int, tid: int, shape, lo: float, hi: float) -> np.ndarray:
    """Magnitudes U(lo, hi) with random signs, as bf16 bits (rounded through
    fp32; choose hi so that the rounding stays below any limit of interest)."""
    rng = np.random.default_rng([seed, tid])
    x = rng.uniform(lo, hi, size=shape) * np.where(rng.random(size=shape) < 0.5, -1.0, 1.0)
    return _f32_to_bf16_bits(x.astype(np.float32))


def uniform_f32(seed: int, tid: int, shape, lo: float, hi: float) -> np.ndarray:
    rng = np.random.default_rng([seed, tid])
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def rope_split(head_dim: int):
    """Per-axis rotary widths (t, h, w): d_h = d_w = 2*floor(d/6), d_t the rest
    (128 -> 44/42/42, 64 -> 24/20/20)."""
    dh = 2 * (head_dim // 6)
    return head_dim - 2 * dh, dh, dh


@dataclass
class Config:
    name: str
    n_heads: int
    head_dim: int
    T: int                 # latent frames in the query chunk
    Hl: int                # tokens per frame, vertical
    Wl: int                # tokens per frame, horizontal
    t0: int                # latent frames that precede the chunk
    seg_lens: List[int]    # K/V segments in cache order; the last is the current chunk
    seg_int8: List[bool]   # which segments are stored int8
    block: int             # block_q == block_k
    mask_kind: str         # "ones" | "frame_causal" | "bsa"
    seed: int
    rope: bool = True      # False: q/k/v are used as they are (one self-attention segment)
    outlier_p: float = 0.0
    theta: float = 1.0e4
    eps: float = 1.0e-6
    bsa_density: float = 0.2
    bsa_frame_tokens: int = 0
    n_chunks: int = 1      # query chunks in one forward (the last n_chunks segments)
    window: int = 0        # > 0: windowed attention, tokens reordered window by window (block = window^2)
    local_range: int = 0   # windows kept around a query window (mask kind "local")
    description: str = ""

    @property
    def chunk_tokens(self) -> int:
        return self.T * self.Hl * self.Wl

    @property
    def chunk_slot(self) -> int:
        """Query rows per chunk: the chunk's tokens, rounded up to whole
        blocks when several chunks share one forward (so that no q-block
        straddles two chunks; the extra rows are padding queries)."""
        n = self.chunk_tokens
        return n if self.n_chunks == 1 else -(-n // self.block) * self.block

    @property
    def n_q(self) -> int:
        return self.n_chunks * self.chunk_slot

    @property
    def n_cached(self) -> int:
        """Number of cached segments (before the chunk segments)."""
        return len(self.seg_lens) - self.n_chunks

    @property
    def split(self):
        return rope_split(self.head_dim)

    def n_qb(self) -> int:
        return -(-self.n_q // self.block)

    def n_kb(self) -> int:
        return sum(-(-L // self.block) for L in self.seg_lens)


WORKLOADS: Dict[str, Config] = {
    # Tiny: 1 head x d64, 2 latent frames of 4x4 tokens, cache 16 text + 32
    # history (two frames) + 32 current, block 16.
    "tiny": Config("tiny", 1, 64, 2, 4, 4, 2, [16, 32, 32], [False, False, False], 16,
                   "frame_causal", 0, description="tiny, frame-level block-causal mask"),
    "tiny_dense": Config("tiny_dense", 1, 64, 2, 4, 4, 2, [16, 32, 32], [False, False, False], 16,
                         "ones", 0, description="tiny, chunk-granularity (all-ones) mask"),
    # Wan2.1-1.3B-shaped chunk: 12 heads x d128, 3 latent frames of 30x52,
    # 512 text + 3 history chunks + the current chunk.
    "wan13b": Config("wan13b", 12, 128, 3, 30, 52, 9, [512, 14040, 4680], [False, False, False], 128,
                     "ones", 1, description="Wan-1.3B-shaped chunk, bf16 cache"),
    "wan13b_int8": Config("wan13b_int8", 12, 128, 3, 30, 52, 9, [512, 14040, 4680], [True, True, False], 128,
                          "ones", 2, outlier_p=0.01,
                          description="Wan-1.3B-shaped chunk, int8 text+history cache"),
    # Large-DiT chunk: 32 heads x d128, 2 latent frames of 30x52, 256 text +
    # one reference-image frame + the current chunk.
    "large_dit": Config("large_dit", 32, 128, 2, 30, 52, 1, [256, 1560, 3120], [False, False, False], 128,
                        "ones", 3, description="Large-DiT chunk, reference-image cache"),
    # Block-sparse video SR: 8 latent frames of 66x66 tokens, self-attention,
    # 128x128 tiles, random 20% tiles plus diagonal and same-frame tiles.
    "bsa_sr": Config("bsa_sr", 12, 128, 8, 66, 66, 0, [34848], [False], 128,
                     "bsa", 4, rope=False, bsa_frame_tokens=66 * 66,
                     description="block-sparse video SR self-attention"),
    # The same clip and mask rule at 32-token blocks (a fine mask: 64-key
    # tiles hold two k-blocks, 256-row workgroups eight q-blocks), for timing
    # the per-q-block masking path.
    "bsa_sr_b32": Config("bsa_sr_b32", 12, 128, 8, 66, 66, 0, [34848], [False], 32,
                         "bsa", 9, rope=False, bsa_frame_tokens=66 * 66,
                         description="block-sparse video SR self-attention, 32-token blocks"),
    # Staggered chunks in one forward (Wave Forcing summary: block-causal
    # attention, later chunks read earlier ones): four Wan-1.3B chunks of
    # 3 x 30 x 52 tokens attend to the text cache, three history chunks and
    # every chunk up to their own.
    "wave_chunks": Config("wave_chunks", 12, 128, 3, 30, 52, 9, [512, 14040, 4680, 4680, 4680, 4680],
                          [False] * 6, 128, "chunk_causal", 5, n_chunks=4,
                          description="four staggered Wan chunks, chunk-level block-causal mask"),
    # Windowed locality-sparse SR self-attention (FlashVSR deployment notes,
    # spatial tiling section): the page's 2688 x 1536 clip is 168 x 96 tokens
    # per frame, attention blocks are 8 x 8-token windows (64 tokens), and
    # local_range = 11 windows; two latent frames.
    "vsr_local": Config("vsr_local", 12, 128, 2, 96, 168, 0, [2 * 96 * 168], [False], 64, "local", 7,
                        rope=False, window=8, local_range=11,
                        description="windowed locality-sparse SR self-attention, 2 frames of 96 x 168 tokens"),
    "tiny_local": Config("tiny_local", 2, 64, 2, 16, 24, 0, [2 * 16 * 24], [False], 16, "local", 8,
                         rope=False, window=4, local_range=3,
                         description="tiny windowed locality-sparse self-attention"),
    # Tiny version: 2 chunks of 2 x 4 x 5 tokens (40, padded to 48 rows), block 16.
    "tiny_chunks": Config("tiny_chunks", 2, 64, 2, 4, 5, 2, [16, 80, 40, 40], [False] * 4, 16,
                          "chunk_causal", 6, n_chunks=2,
                          description="tiny, two chunks in one forward"),
}

# The five main workloads, smallest (the one the oracle runs in full) first.
WORKLOAD_ORDER = ["tiny", "wan13b", "wan13b_int8", "large_dit", "bsa_sr"]


def make_mask(cfg: Config) -> np.ndarray:
    """uint8 [n_qb, n_kb] keep mask (nonzero = keep). k-blocks restart at each
    segment boundary."""
    nqb, nkb = cfg.n_qb(), cfg.n_kb()
    if cfg.mask_kind == "ones":
        return np.ones((nqb, nkb), dtype=np.uint8)
    if cfg.mask_kind == "frame_causal":
        # Rows are query blocks; a query block sees every cached block and
        # the current-chunk blocks up to and including its own.
        m = np.zeros((nqb, nkb), dtype=np.uint8)
        n_cache_blocks = sum(-(-L // cfg.block) for L in cfg.seg_lens[:cfg.n_cached])
        for qb in range(nqb):
            m[qb, :n_cache_blocks] = 1
            m[qb, n_cache_blocks:n_cache_blocks + qb + 1] = 1
        return m
    if cfg.mask_kind == "local":
        # blocks are windows in window-major order (frame, window row, window
        # column); a key window is kept when it lies within local_range // 2
        # windows of the query window in both directions, in any frame
        assert cfg.block == cfg.window * cfg.window and nqb == nkb
        nwy, nwx = cfg.Hl // cfg.window, cfg.Wl // cfg.window
        b = np.arange(nqb) % (nwy * nwx)
        wy, wx = b // nwx, b % nwx
        r = cfg.local_range // 2
        return ((np.abs(wy[:, None] - wy[None, :]) <= r) & (np.abs(wx[:, None] - wx[None, :]) <= r)).astype(np.uint8)
    if cfg.mask_kind == "chunk_causal":
        # q-blocks of chunk c see every cached block and chunks 0..c
        m = np.zeros((nqb, nkb), dtype=np.uint8)
        col = np.cumsum([0] + [-(-L // cfg.block) for L in cfg.seg_lens])
        per_chunk = cfg.chunk_slot // cfg.block
        for qb in range(nqb):
            c = qb // per_chunk
            m[qb, :col[cfg.n_cached + c + 1]] = 1
        return m
    if cfg.mask_kind == "bsa":
        assert len(cfg.seg_lens) == 1
        n = cfg.seg_lens[0]
        B = cfg.block
        rng = np.random.default_rng([cfg.seed, TID_TILE_MASK])
        m = rng.random((nqb, nkb)) < cfg.bsa_density
        F = cfg.bsa_frame_tokens
        first = np.arange(nqb) * B // F
        last = (np.minimum(np.arange(nqb) * B + B, n) - 1) // F
        # q-range and k-range share a latent frame when their frame intervals overlap
        same = (first[:, None] <= last[None, :]) & (first[None, :] <= last[:, None])
        forced = same | np.eye(nqb, nkb, dtype=bool)
        return (m | forced).astype(np.uint8)
    raise ValueError(cfg.mask_kind)


@dataclass
class Inputs:
    cfg: Config
    q: np.ndarray                  # bf16 bits [n_q, H, d], before norm/rope
    k: np.ndarray                  # bf16 bits [n_q, H, d], before norm/rope (current chunks, see chunk_rows)
    v: np.ndarray                  # bf16 bits [n_q, H, d]
    cache_k: List[np.ndarray] = field(default_factory=list)  # bf16 bits per cached segment
    cache_v: List[np.ndarray] = field(default_factory=list)
    gamma_q: Optional[np.ndarray] = None   # fp32 [d]
    gamma_k: Optional[np.ndarray] = None
    mask: Optional[np.ndarray] = None      # uint8 [n_qb, n_kb]


def make_inputs(cfg: Config, n_heads: Optional[int] = None) -> Inputs:
    """Generate every input of one layer-chunk. ``n_heads`` below the
    configuration's head count draws only the leading heads (same values as
    the full draw is not guaranteed; use it for reduced tests only)."""
    H = cfg.n_heads if n_heads is None else n_heads
    d = cfg.head_dim
    s = cfg.seed
    nq = cfg.n_q
    q = normal_bf16(s, TID_Q, (nq, H, d))
    k = normal_bf16(s, TID_K, (nq, H, d))
    v = normal_bf16(s, TID_V, (nq, H, d))
    cache_k, cache_v = [], []
    tids = [(TID_TEXT_K, TID_TEXT_V), (TID_HIST_K, TID_HIST_V)]
    for i, L in enumerate(cfg.seg_lens[:cfg.n_cached]):
        tk, tv = tids[i]
        p = cfg.outlier_p if cfg.seg_int8[i] else 0.0
        cache_k.append(normal_bf16(s, tk, (L, H, d), p, outlier_tid=TID_K_OUTLIER + 20 * i))
        cache_v.append(normal_bf16(s, tv, (L, H, d), p, outlier_tid=TID_V_OUTLIER + 20 * i))
    gq = uniform_f32(s, TID_GAMMA_Q, (d,), 0.5, 1.5)
    gk = uniform_f32(s, TID_GAMMA_K, (d,), 0.5, 1.5)
    return Inputs(cfg, q, k, v, cache_k, cache_v, gq, gk, make_mask(cfg))


def chunk_rows(cfg: Config, c: int) -> slice:
    """Rows of query chunk c in q / k / v (the rest of its slot is padding)."""
    start = c * cfg.chunk_slot
    return slice(start, start + cfg.chunk_tokens)


def attn_flops(cfg: Config, mask: np.ndarray) -> int:
    """Effective attention FLOPs: 4*d*H * sum over kept (q-block, k-block)
    tiles of rows(qb) * cols(kb), with the real (unpadded) sizes."""
    B = cfg.block
    rows = np.array([min(B, cfg.n_q - i * B) for i in range(cfg.n_qb())], dtype=np.int64)
    cols = []
    for L in cfg.seg_lens:
        cols += [min(B, L - j * B) for j in range(-(-L // B))]
    cols = np.array(cols, dtype=np.int64)
    kept = (mask != 0).astype(np.int64)
    return int(4 * cfg.head_dim * cfg.n_heads * (rows[:, None] * cols[None, :] * kept).sum())


@dataclass
class NormInputs:
    x: np.ndarray        # bf16 bits [n_tok, dim]
    gamma: np.ndarray    # fp32 [dim]   (RMSNorm gain)
    scale: np.ndarray    # fp32 [dim]   (modulation scale)
    shift: np.ndarray    # fp32 [dim]   (modulation shift)


def make_norm_inputs(seed: int, n_tok: int, dim: int, offset: float = 0.0) -> NormInputs:
    """Hidden-state-like rows for the per-token norms: N(0,1) per element
    times a per-channel magnitude (log-uniform over [1/4, 4], and 1 channel
    in 64 at 32x: DiT activations carry a few large channels), plus a
    per-token offset drawn from N(0, offset^2); gamma U(0.5, 1.5), the
    modulation scale U(-0.5, 0.5) and shift U(-1, 1)."""
    rng = np.random.default_rng([seed, TID_HIDDEN])
    x = rng.standard_normal(size=(n_tok, dim))
    crng = np.random.default_rng([seed, TID_CH_SCALE])
    ch = np.exp2(crng.uniform(-2.0, 2.0, size=dim))
    ch = np.where(crng.random(size=dim) < 1.0 / 64, 32.0, ch)
    x = x * ch
    if offset:
        x = x + np.random.default_rng([seed, TID_TOK_OFFSET]).normal(0.0, offset, size=(n_tok, 1))
    return NormInputs(x=_f32_to_bf16_bits(x.astype(np.float32)),
                      gamma=uniform_f32(seed, TID_GAMMA, (dim,), 0.5, 1.5),
                      scale=uniform_f32(seed, TID_MOD_SCALE, (dim,), -0.5, 0.5),
                      shift=uniform_f32(seed, TID_MOD_SHIFT, (dim,), -1.0, 1.0))
