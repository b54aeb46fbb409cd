"""Pins for the oracle's RMSNorm and LayerNorm + modulate (CPU only): torch's
fp64 rms_norm and layer_norm library routines, and invariants (a constant
added to a row leaves LayerNorm unchanged; scale = shift = 0 gives rows of
mean 0 and variance var / (var + eps); eps = 0 RMSNorm is unchanged by a
power-of-two rescaling of the row)."""
import numpy as np
import torch

import workloads as W
from oracle import bf16_to_f64, f64_to_bf16
from oracle.norms import layernorm_modulate, rmsnorm


def _x(seed, n, C):
    return W.normal_bf16(seed, 0, (n, C), outlier_p=0.01, outlier_tid=1)


def test_rmsnorm_equals_torch_fp64():
    x = _x(1, 64, 1536)
    g = W.uniform_f32(1, 2, (1536,), 0.5, 1.5)
    y = rmsnorm(x, g, 1e-6, rounded=False)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(bf16_to_f64(x)), (1536,),
                                       weight=torch.from_numpy(g.astype(np.float64)), eps=1e-6).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-15)


def test_layernorm_modulate_equals_torch_fp64():
    x = _x(2, 64, 1536)
    sc = W.uniform_f32(2, 2, (1536,), -0.5, 0.5)
    sh = W.uniform_f32(2, 3, (1536,), -1.0, 1.0)
    y = layernorm_modulate(x, sc, sh, 1e-6, rounded=False)
    ln = torch.nn.functional.layer_norm(torch.from_numpy(bf16_to_f64(x)), (1536,), eps=1e-6).numpy()
    np.testing.assert_allclose(y, ln * (1.0 + sc.astype(np.float64)) + sh.astype(np.float64), rtol=1e-12,
                               atol=1e-13)


def test_invariants():
    x = _x(3, 16, 512)
    xf = bf16_to_f64(x)
    zero = np.zeros(512, np.float32)
    # scale = shift = 0: rows of mean 0 and mean square var / (var + eps)
    y = layernorm_modulate(x, zero, zero, 1e-6, rounded=False)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-13)
    var = ((xf - xf.mean(axis=1, keepdims=True)) ** 2).mean(axis=1)
    np.testing.assert_allclose((y ** 2).mean(axis=1), var / (var + 1e-6), rtol=1e-12)
    # a constant added to a row leaves the LayerNorm unchanged: rows of multiples of 1/32 in [-2, 2],
    # so that the values and the values + 4 are all exact in bf16
    k = np.random.default_rng(5).integers(-64, 65, size=(8, 512))
    r = f64_to_bf16(k / 32.0)
    moved = f64_to_bf16(k / 32.0 + 4.0)
    assert np.array_equal(bf16_to_f64(r), k / 32.0) and np.array_equal(bf16_to_f64(moved), k / 32.0 + 4.0)
    np.testing.assert_allclose(layernorm_modulate(moved, zero, zero, 1e-6, rounded=False),
                               layernorm_modulate(r, zero, zero, 1e-6, rounded=False), rtol=1e-11, atol=1e-11)
    # eps = 0 RMSNorm: rescaling the row by 2^3 changes nothing
    g = np.ones(512, np.float32)
    np.testing.assert_array_equal(rmsnorm(x, g, 0.0, rounded=False), rmsnorm(f64_to_bf16(xf * 8.0), g, 0.0,
                                                                          rounded=False))
