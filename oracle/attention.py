"""Block-masked softmax attention over concatenated K/V segments, fp64
(test infrastructure only).

Sources:
  * The chunk's image queries attend to K/V made of a static text cache, the
    reference-image or history cache, and the current chunk
    (Joy-face_change_optimized README, section 1, item 1, and section 2,
    reference-image K/V reuse).
  * A chunk sees itself and every earlier chunk (block-causal attention;
    Wave Forcing summary, first paragraph).
  * Attention restricted by a (q-block, k-block) keep mask; with a dense mask
    it must equal ordinary scaled-dot-product attention, and a
    lower-triangular block mask gives a different, non-degenerate result
    (FlashVSR deployment notes, Block-Sparse-Attention section).

Readings (where the pages are silent):
  * Keys are indexed segment by segment in cache order. Query block
    qb(i) = i // block_q. Key blocks restart at every segment:
    kb(segment s, local j) = sum_{s' < s} ceil(L_s' / block_k) + j // block_k,
    so a block never straddles two segments; the last block of a segment (and
    of the queries) may be partial. A nonzero mask byte keeps the tile.
  * Softmax scale 1/sqrt(d) unless given (the SDPA default).
  * int8 segments contribute K = code * k_scale and V = code * v_scale,
    exactly, in fp64.
  * A query with no visible key gets O = 0 and LSE = -inf (SDPA would give
    NaN; that convention is not adopted).

The computation is the plain definition: for each head and query i, the
visible set V(i) = {j : mask[qb(i)][kb(j)] != 0},
  s_ij = scale * q_i . K_j,  m = max_j s_ij,  p_ij = exp(s_ij - m),
  l = sum_j p_ij,  o_i = sum_j p_ij V_j / l,  LSE_i = m + ln l,
with fp64 matrix products as the only library primitive.
"""
import numpy as np

from .bf16 import bf16_to_f64
from .kv_quant import kv_dequant


def key_block_index(seg_lens, block_k: int) -> np.ndarray:
    """Global k-block index of every key, segments in order."""
    out = []
    base = 0
    for L in seg_lens:
        out.append(base + np.arange(L) // block_k)
        base += -(-L // block_k)
    return np.concatenate(out) if out else np.zeros(0, dtype=np.int64)


def segment_values(seg: dict):
    """fp64 (K, V) of one segment dict with keys k, v, dtype ('bf16' | 'int8')
    and, for int8, k_scale and v_scale."""
    if seg["dtype"] == "bf16":
        return bf16_to_f64(seg["k"]), bf16_to_f64(seg["v"])
    if seg["dtype"] == "int8":
        return kv_dequant(seg["k"], seg["k_scale"]), kv_dequant(seg["v"], seg["v_scale"])
    raise ValueError(seg["dtype"])


def attention(q_bits: np.ndarray, segments, mask: np.ndarray, block_q: int, block_k: int,
              softmax_scale=None, heads=None, rows=None):
    """Attention of queries q (bf16 bits [n_q, H, d]) over the segments.

    ``heads`` / ``rows`` restrict the computation to a subset of heads and
    query rows (for sampled checks at full size); the result is indexed in
    the order given.
    Returns (O fp64 [len(rows), len(heads), d], LSE fp64 [len(heads), len(rows)]).
    """
    q = bf16_to_f64(q_bits)
    n_q, H, d = q.shape
    heads = list(range(H)) if heads is None else list(heads)
    rows = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    scale = 1.0 / np.sqrt(d) if (softmax_scale is None or softmax_scale <= 0) else float(softmax_scale)

    seg_lens = [int(s["k"].shape[0]) for s in segments]
    kb = key_block_index(seg_lens, block_k)
    n_kb = sum(-(-L // block_k) for L in seg_lens)
    n_qb = -(-n_q // block_q)
    mask = np.asarray(mask)
    if mask.shape != (n_qb, n_kb):
        raise ValueError(f"mask shape {mask.shape} != {(n_qb, n_kb)}")
    vals = [segment_values(s) for s in segments]

    O = np.zeros((len(rows), len(heads), d))
    LSE = np.full((len(heads), len(rows)), -np.inf)
    qb_of_row = rows // block_q
    for hi, h in enumerate(heads):
        K = np.concatenate([kv[0][:, h, :] for kv in vals], axis=0)
        V = np.concatenate([kv[1][:, h, :] for kv in vals], axis=0)
        for qb in np.unique(qb_of_row):
            sel = np.nonzero(qb_of_row == qb)[0]
            visible = mask[qb][kb] != 0
            if not visible.any():
                continue
            if visible.all():
                Kv, Vv = K, V
            else:
                Kv, Vv = K[visible], V[visible]
            s = scale * (q[rows[sel], h, :] @ Kv.T)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True)
            O[sel, hi, :] = (p @ Vv) / l
            LSE[hi, sel] = m[:, 0] + np.log(l[:, 0])
    return O, LSE


def attention_merge(parts):
    """Combine attention results over disjoint key sets (test infrastructure).

    Source: context-parallel attention of the Ulysses / Ring kind, which the
    Wave Forcing summary measures Wave Parallelism against: each step attends
    to one shard of the keys, and the shards' results are combined. Softmax
    over a disjoint union of key sets A, B satisfies, per query,
      LSE = log(e^LSE_A + e^LSE_B),
      o   = e^(LSE_A - LSE) o_A + e^(LSE_B - LSE) o_B,
    because e^LSE_X is the sum of e^s over X and o_X is the e^s-weighted mean
    of V over X. Written here for any number of parts with the usual shift by
    the largest LSE. A part whose query sees no key (LSE = -inf, o = 0) adds
    nothing; a query that sees no key in any part gets o = 0, LSE = -inf.

    parts: list of (O fp64 [n_q, H, d], LSE fp64 [H, n_q]).
    Returns (O [n_q, H, d], LSE [H, n_q]) in fp64.
    """
    if not parts:
        raise ValueError("no parts")
    lses = np.stack([np.asarray(L, dtype=np.float64) for _, L in parts])       # [P, H, n_q]
    outs = np.stack([np.asarray(O, dtype=np.float64) for O, _ in parts])       # [P, n_q, H, d]
    m = lses.max(axis=0)                                                       # [H, n_q]
    seen = np.isfinite(m)
    shift = np.where(seen, m, 0.0)
    w = np.exp(lses - shift[None])                                             # exp(-inf) = 0
    total = w.sum(axis=0)                                                      # [H, n_q]
    O = np.einsum("phq,pqhd->qhd", w, outs)
    safe = np.where(seen, total, 1.0)
    O = np.where(seen.T[:, :, None], O / safe.T[:, :, None], 0.0)
    LSE = np.where(seen, shift + np.log(safe), -np.inf)
    return O, LSE

