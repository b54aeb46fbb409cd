"""Pins for the oracle's QK-RMSNorm + 3D RoPE (CPU only).

The pages name the fused operator ("QK-norm+3D RoPE") without formulas, so
the oracle is pinned by independent routines and by invariants:
  * RMSNorm against torch.nn.functional.rms_norm (fp64, a library routine)
    and a closed form for constant vectors;
  * each axis block of the 3D rotary against the interleaved ("rotate every
    two") rotary of the GPT-J model code in transformers, with that axis's
    position, base 1e4;
  * position 0 is the identity, norms are preserved, and q.k depends only
    on the offset between the two tokens on every axis.
"""
import numpy as np
import pytest
import torch

from oracle import apply_rope, f64_to_bf16, bf16_to_f64, qknorm_rope3d, rms_norm, rope3d_angles


def test_rms_norm_matches_torch_library():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 3, 64)) * 3.0
    g = rng.uniform(0.5, 1.5, 64)
    for eps in (1e-6, 0.5):
        want = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps).numpy()
        np.testing.assert_allclose(rms_norm(x, g, eps), want, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("c", [1.0, -0.003, 7.5])
def test_rms_norm_constant_vector_closed_form(c):
    # x = c * ones(d): mean square is c^2, so y = gamma * c / sqrt(c^2 + eps)
    d, eps = 128, 1e-6
    g = np.linspace(0.5, 1.5, d)
    y = rms_norm(np.full((1, d), c), g, eps)[0]
    np.testing.assert_allclose(y, g * np.sign(c) / np.sqrt(1.0 + eps / c**2), rtol=1e-14)


def test_rms_norm_unit_rms_and_scale_invariance_without_eps():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((20, 128))
    y = rms_norm(x, np.ones(128), 0.0)
    np.testing.assert_allclose(np.sqrt((y * y).mean(-1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(rms_norm(1e3 * x, np.ones(128), 0.0), y, rtol=1e-13)


def _gptj_rope(x, positions):
    """Rotary of the GPT-J model in transformers: x [n, d] at integer positions."""
    from transformers.models.gptj.modeling_gptj import apply_rotary_pos_emb, create_sinusoidal_positions
    n, d = x.shape
    table = create_sinusoidal_positions(int(max(positions)) + 1, d).to(torch.float64)
    sincos = table[torch.as_tensor(positions)]
    sin, cos = torch.split(sincos, d // 2, dim=-1)
    t = torch.from_numpy(x)[None, :, None, :]            # [batch, seq, heads, dim]
    out = apply_rotary_pos_emb(t, sin[None], cos[None])
    return out[0, :, 0, :].numpy()


@pytest.mark.parametrize("split", [(44, 42, 42), (24, 20, 20), (64, 0, 0), (0, 0, 64), (0, 32, 0)])
def test_each_axis_block_is_gptj_rotary(split):
    d_t, d_h, d_w = split
    d = d_t + d_h + d_w
    T, Hl, Wl, t0 = 3, 5, 7, 4
    n = T * Hl * Wl
    rng = np.random.default_rng(3)
    y = rng.standard_normal((n, 1, d))
    got = apply_rope(y, rope3d_angles(T, Hl, Wl, t0, d_t, d_h, d_w, 1.0e4))[:, 0, :]
    tok = np.arange(n)
    pos = {"t": t0 + tok // (Hl * Wl), "h": (tok // Wl) % Hl, "w": tok % Wl}
    off = 0
    for axis, width in zip("thw", split):
        if width:
            want = _gptj_rope(y[:, 0, off:off + width], pos[axis])
            # the library builds its table in fp32
            np.testing.assert_allclose(got[:, off:off + width], want, rtol=0, atol=2e-5)
        off += width


def test_position_zero_is_identity_and_norm_is_preserved():
    rng = np.random.default_rng(4)
    y = rng.standard_normal((1, 2, 128))
    np.testing.assert_array_equal(apply_rope(y, rope3d_angles(1, 1, 1, 0, 44, 42, 42, 1e4)), y)
    y = rng.standard_normal((3 * 30 * 52, 2, 128))
    r = apply_rope(y, rope3d_angles(3, 30, 52, 9, 44, 42, 42, 1e4))
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(y, axis=-1), rtol=1e-12)
    # pair by pair as well
    np.testing.assert_allclose(r[..., 0::2] ** 2 + r[..., 1::2] ** 2,
                               y[..., 0::2] ** 2 + y[..., 1::2] ** 2, rtol=1e-12, atol=1e-14)


def test_dot_product_depends_only_on_offset():
    # Same q and k vectors placed at every token of a grid: q(a).k(b) must
    # equal q(a').k(b') whenever a - b == a' - b' on all three axes.
    T, Hl, Wl, t0 = 4, 6, 7, 3
    rng = np.random.default_rng(5)
    qv, kv = rng.standard_normal(128), rng.standard_normal(128)
    n = T * Hl * Wl
    ang = rope3d_angles(T, Hl, Wl, t0, 44, 42, 42, 1e4)
    rq = apply_rope(np.broadcast_to(qv, (n, 1, 128)), ang)[:, 0]
    rk = apply_rope(np.broadcast_to(kv, (n, 1, 128)), ang)[:, 0]
    tok = lambda t, h, w: (t * Hl + h) * Wl + w
    checks = 0
    for (a, b, s) in [((1, 2, 3), (0, 1, 1), (2, 3, 2)), ((3, 5, 6), (1, 1, 1), (-1, -1, -1)),
                      ((0, 0, 6), (2, 5, 0), (1, 0, 0)), ((2, 2, 2), (2, 2, 2), (1, 3, 4))]:
        a2 = tuple(x + y for x, y in zip(a, s))
        b2 = tuple(x + y for x, y in zip(b, s))
        lhs = rq[tok(*a)] @ rk[tok(*b)]
        rhs = rq[tok(*a2)] @ rk[tok(*b2)]
        assert abs(lhs - rhs) < 1e-10 * (1 + abs(lhs))
        checks += 1
    # a different offset gives a different product (the test is not vacuous)
    assert abs(rq[tok(1, 2, 3)] @ rk[tok(0, 1, 1)] - rq[tok(1, 2, 3)] @ rk[tok(0, 1, 2)]) > 1e-3
    assert checks == 4


def test_shift_of_t0_keeps_q_dot_k():
    rng = np.random.default_rng(6)
    xq = rng.integers(0, 1 << 16, (2 * 3 * 4, 2, 64), dtype=np.uint16) & 0x3FFF  # finite, moderate
    xk = rng.integers(0, 1 << 16, (2 * 3 * 4, 2, 64), dtype=np.uint16) & 0x3FFF
    g = np.ones(64)
    a = [qknorm_rope3d(x, g, 2, 3, 4, 5, 24, 20, 20, rounded=False) for x in (xq, xk)]
    b = [qknorm_rope3d(x, g, 2, 3, 4, 11, 24, 20, 20, rounded=False) for x in (xq, xk)]
    np.testing.assert_allclose(np.einsum("nhd,mhd->hnm", *a), np.einsum("nhd,mhd->hnm", *b),
                               rtol=1e-10, atol=1e-10)


def test_rounded_output_is_one_rounding_of_the_fp64_result():
    rng = np.random.default_rng(7)
    from workloads import _f32_to_bf16_bits
    x = _f32_to_bf16_bits(rng.standard_normal((2 * 4 * 4, 1, 64)).astype(np.float32))
    g = rng.uniform(0.5, 1.5, 64)
    exact = qknorm_rope3d(x, g, 2, 4, 4, 2, 24, 20, 20, rounded=False)
    bits = qknorm_rope3d(x, g, 2, 4, 4, 2, 24, 20, 20)
    err = np.abs(bf16_to_f64(bits) - exact)
    ulp = np.ldexp(1.0, np.frexp(np.abs(exact))[1] - 8)
    assert np.all(err <= ulp / 2)
    np.testing.assert_array_equal(bits, f64_to_bf16(exact))
