"""RMSNorm and LayerNorm + modulate over the hidden dimension, fp64 (test
infrastructure only).

The Joy-face_change_optimized README (table of changed files) lists these
two next to the QK-norm + 3D RoPE operator as the fused kernels of the DiT
block, and states that its PyTorch re-implementation agrees with the CUDA
kernels to one bf16 ulp. The pages give no formulas; the plain readings:

  * RMSNorm per token over the hidden dimension C:
        y_c = x_c / sqrt(mean_c(x_c^2) + eps) * gamma_c;
  * LayerNorm + modulate (adaptive LayerNorm of a DiT block): a LayerNorm
    without parameters of its own, population variance, eps inside the
    square root, then the conditioning's scale and shift:
        y_c = (x_c - mean) / sqrt(var + eps) * (1 + scale_c) + shift_c,
    with scale and shift vectors over C shared by all tokens of the call;
  * inputs bf16, gamma / scale / shift fp32, one rounding to bf16 at the end.
"""
import numpy as np

from .bf16 import bf16_to_f64, f64_to_bf16
from .qknorm_rope3d import rms_norm


def rmsnorm(x_bits: np.ndarray, gamma: np.ndarray, eps: float = 1e-6, rounded: bool = True):
    """x_bits bf16 [n_tok, C] -> bf16 bits (or fp64 when rounded is False)."""
    y = rms_norm(bf16_to_f64(x_bits), gamma, eps)
    return f64_to_bf16(y) if rounded else y


def layernorm_modulate(x_bits: np.ndarray, scale: np.ndarray, shift: np.ndarray, eps: float = 1e-6,
                       rounded: bool = True):
    """x_bits bf16 [n_tok, C] -> bf16 bits (or fp64 when rounded is False)."""
    x = bf16_to_f64(x_bits)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    y = (x - mean) / np.sqrt(var + eps)
    y = y * (1.0 + np.asarray(scale, dtype=np.float64)) + np.asarray(shift, dtype=np.float64)
    return f64_to_bf16(y) if rounded else y
