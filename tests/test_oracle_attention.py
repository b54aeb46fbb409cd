"""Pins for the oracle's block-masked attention (CPU only).

  * dense mask == torch scaled_dot_product_attention in fp64 (library routine),
    the FlashVSR deployment notes' own acceptance check for block-sparse
    attention;
  * a lower-triangular block mask differs from dense and matches a brute
    force written with plain Python loops and math.fsum (same page);
  * brute force on the tiny workload (both mask readings) and on ragged
    segments with partial blocks;
  * invariants: key permutation, one visible key gives its value, q = 0
    gives the mean of the visible values, LSE merge of two disjoint key sets,
    deleting a masked block's keys changes nothing, NaN in skipped tiles
    never reaches the output, and an empty row gives O = 0, LSE = -inf.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention, bf16_to_f64, key_block_index, kv_quant_int8, qknorm_rope3d, segment_values


def _segs(ks, vs, dtype="bf16"):
    return [{"k": k, "v": v, "dtype": dtype} for k, v in zip(ks, vs)]


def _rand_bits(seed, shape):
    return W.normal_bf16(seed, 0, shape)


def _brute(q_bits, segments, mask, bq, bk, scale=None):
    """Pure-Python loops: softmax over visible keys, math.fsum for every sum."""
    q = bf16_to_f64(q_bits)
    n_q, H, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    Ks, Vs, kbs = [], [], []
    base = 0
    for s in segments:
        K, V = segment_values(s)
        L = K.shape[0]
        for j in range(L):
            Ks.append(K[j]); Vs.append(V[j]); kbs.append(base + j // bk)
        base += -(-L // bk)
    O = np.zeros((n_q, H, d))
    LSE = np.full((H, n_q), -math.inf)
    for h in range(H):
        for i in range(n_q):
            vis = [j for j in range(len(Ks)) if mask[i // bq][kbs[j]]]
            if not vis:
                continue
            sc = [scale * math.fsum(float(a) * float(b) for a, b in zip(q[i, h], Ks[j][h])) for j in vis]
            m = max(sc)
            p = [math.exp(x - m) for x in sc]
            l = math.fsum(p)
            for c in range(d):
                O[i, h, c] = math.fsum(pj * float(Vs[j][h][c]) for pj, j in zip(p, vis)) / l
            LSE[h, i] = m + math.log(l)
    return O, LSE


def test_key_block_index_restarts_per_segment():
    kb = key_block_index([16, 32, 5, 17], 16)
    assert kb.tolist() == [0] * 16 + [1] * 16 + [2] * 16 + [3] * 5 + [4] * 16 + [5]


def test_dense_equals_torch_sdpa_fp64():
    rng = np.random.default_rng(0)
    q = _rand_bits(1, (70, 3, 64))
    ks = [_rand_bits(2, (20, 3, 64)), _rand_bits(3, (45, 3, 64))]
    vs = [_rand_bits(4, (20, 3, 64)), _rand_bits(5, (45, 3, 64))]
    mask = np.ones((-(-70 // 32), 1 + 2), np.uint8)
    O, LSE = attention(q, _segs(ks, vs), mask, 32, 32)
    tq = torch.from_numpy(bf16_to_f64(q)).permute(1, 0, 2)
    tk = torch.from_numpy(np.concatenate([bf16_to_f64(k) for k in ks])).permute(1, 0, 2)
    tv = torch.from_numpy(np.concatenate([bf16_to_f64(v) for v in vs])).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(O, ref, rtol=1e-12, atol=1e-12)
    lse_ref = torch.logsumexp((tq @ tk.transpose(1, 2)) / 8.0, dim=-1).numpy()
    np.testing.assert_allclose(LSE, lse_ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("name", ["tiny", "tiny_dense"])
def test_tiny_workload_against_brute_force(name):
    cfg = W.WORKLOADS[name]
    inp = W.make_inputs(cfg)
    dt, dh, dw = cfg.split
    qr = qknorm_rope3d(inp.q, inp.gamma_q, cfg.T, cfg.Hl, cfg.Wl, cfg.t0, dt, dh, dw)
    kr = qknorm_rope3d(inp.k, inp.gamma_k, cfg.T, cfg.Hl, cfg.Wl, cfg.t0, dt, dh, dw)
    segs = _segs(inp.cache_k + [kr], inp.cache_v + [inp.v])
    O, LSE = attention(qr, segs, inp.mask, cfg.block, cfg.block)
    Ob, LSEb = _brute(qr, segs, inp.mask, cfg.block, cfg.block)
    np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(LSE, LSEb, rtol=1e-12, atol=1e-13)


def test_tiny_mask_readings_differ():
    cfg_c, cfg_d = W.WORKLOADS["tiny"], W.WORKLOADS["tiny_dense"]
    inp = W.make_inputs(cfg_c)
    segs = _segs(inp.cache_k + [inp.k], inp.cache_v + [inp.v])
    Oc, _ = attention(inp.q, segs, W.make_mask(cfg_c), 16, 16)
    Od, _ = attention(inp.q, segs, W.make_mask(cfg_d), 16, 16)
    assert np.array_equal(Oc[16:], Od[16:])          # second q-block keeps every block
    assert np.abs(Oc[:16] - Od[:16]).max() > 1e-3    # first q-block loses the last block


def test_lower_triangular_block_mask_is_different_and_matches_brute_force():
    q = _rand_bits(11, (64, 2, 64))
    k = _rand_bits(12, (64, 2, 64))
    v = _rand_bits(13, (64, 2, 64))
    tri = np.tril(np.ones((4, 4), np.uint8))
    segs = _segs([k], [v])
    O, LSE = attention(q, segs, tri, 16, 16)
    Od, _ = attention(q, segs, np.ones((4, 4), np.uint8), 16, 16)
    assert np.abs(O - Od).max() > 1e-2 and np.all(np.isfinite(O))
    Ob, LSEb = _brute(q, segs, tri, 16, 16)
    np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(LSE, LSEb, rtol=1e-12, atol=1e-13)


def test_ragged_segments_and_int8_against_brute_force():
    q = _rand_bits(21, (37, 2, 64))
    k1, v1 = _rand_bits(22, (23, 2, 64)), _rand_bits(23, (23, 2, 64))
    k2, v2 = _rand_bits(24, (9, 2, 64)), _rand_bits(25, (9, 2, 64))
    ck, sk = kv_quant_int8(k1)
    cv, sv = kv_quant_int8(v1)
    segs = [{"k": ck, "v": cv, "k_scale": sk, "v_scale": sv, "dtype": "int8"},
            {"k": k2, "v": v2, "dtype": "bf16"}]
    rng = np.random.default_rng(9)
    mask = (rng.random((3, 2 + 1)) < 0.6).astype(np.uint8)
    mask[0] = [0, 0, 0]                                   # an empty row block
    O, LSE = attention(q, segs, mask, 16, 16)
    Ob, LSEb = _brute(q, segs, mask, 16, 16)
    np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(LSE, LSEb, rtol=1e-12, atol=1e-13)
    assert np.all(O[:16] == 0) and np.all(np.isneginf(LSE[:, :16]))


def test_invariants():
    q = _rand_bits(31, (32, 1, 64))
    k = _rand_bits(32, (48, 1, 64))
    v = _rand_bits(33, (48, 1, 64))
    ones = np.ones((1, 3), np.uint8)
    O, LSE = attention(q, _segs([k], [v]), ones, 32, 16)
    perm = np.random.default_rng(1).permutation(48)
    Op, LSEp = attention(q, _segs([k[perm]], [v[perm]]), ones, 32, 16)
    np.testing.assert_allclose(Op, O, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(LSEp, LSE, rtol=1e-12)
    # one visible key (block size 1) -> its value
    m1 = np.zeros((1, 48), np.uint8); m1[0, 17] = 1
    O1, _ = attention(q, _segs([k], [v]), m1, 32, 1)
    np.testing.assert_array_equal(O1[:, 0], np.broadcast_to(bf16_to_f64(v)[17, 0], (32, 64)))
    # q = 0 -> mean of the visible values
    O0, LSE0 = attention(np.zeros_like(q), _segs([k], [v]), ones, 32, 16)
    np.testing.assert_allclose(O0[:, 0], np.broadcast_to(bf16_to_f64(v)[:, 0].mean(0), (32, 64)), rtol=1e-12)
    np.testing.assert_allclose(LSE0, math.log(48), rtol=1e-14)
    # LSE merge of two disjoint key sets equals the whole
    ma = np.array([[1, 0, 1]], np.uint8); mb = 1 - ma
    Oa, La = attention(q, _segs([k], [v]), ma, 32, 16)
    Ob, Lb = attention(q, _segs([k], [v]), mb, 32, 16)
    L = np.logaddexp(La, Lb)
    wa, wb = np.exp(La - L).T[:, :, None], np.exp(Lb - L).T[:, :, None]
    np.testing.assert_allclose(wa * Oa + wb * Ob, O, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(L, LSE, rtol=1e-13)


def test_masked_block_equals_deleted_keys_and_nan_never_leaks():
    q = _rand_bits(41, (48, 2, 64))
    k = _rand_bits(42, (64, 2, 64))
    v = _rand_bits(43, (64, 2, 64))
    mask = np.ones((3, 4), np.uint8)
    mask[1, 2] = 0
    O, _ = attention(q, _segs([k], [v]), mask, 16, 16)
    full, _ = attention(q, _segs([k], [v]), np.ones((3, 4), np.uint8), 16, 16)
    keep = np.r_[0:32, 48:64]
    Od, _ = attention(q, _segs([k[keep]], [v[keep]]), np.ones((3, 3), np.uint8), 16, 16)
    np.testing.assert_allclose(O[16:32], Od[16:32], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(O[:16], full[:16])
    np.testing.assert_array_equal(O[32:], full[32:])
    # NaN in the keys/values of a tile that no q-block keeps
    mask2 = np.ones((3, 4), np.uint8); mask2[:, 1] = 0
    kn, vn = k.copy(), v.copy()
    kn[16:32] = 0x7FC0; vn[16:32] = 0x7FC0
    On, _ = attention(q, _segs([kn], [vn]), mask2, 16, 16)
    Oc, _ = attention(q, _segs([k], [v]), mask2, 16, 16)
    assert np.all(np.isfinite(On))
    np.testing.assert_array_equal(On, Oc)


def test_sampled_rows_equal_full_computation():
    q = _rand_bits(51, (100, 3, 64))
    k = _rand_bits(52, (80, 3, 64))
    v = _rand_bits(53, (80, 3, 64))
    mask = (np.random.default_rng(3).random((4, 3)) < 0.7).astype(np.uint8)
    mask[:, 0] = 1
    O, LSE = attention(q, _segs([k], [v]), mask, 32, 32)
    rows = [99, 3, 64, 31, 32]
    Os, LSEs = attention(q, _segs([k], [v]), mask, 32, 32, heads=[2, 0], rows=rows)
    # same arithmetic, only the BLAS blocking may differ
    np.testing.assert_allclose(Os, O[rows][:, [2, 0]], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(LSEs, LSE[[2, 0]][:, rows], rtol=1e-14)
