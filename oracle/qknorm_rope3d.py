"""QK-RMSNorm + 3D (t, h, w) rotary embedding, fp64 (test infrastructure only).

Follows the "QK-norm+3D RoPE" fused operator of the Joy-face_change_optimized
README (table of changed files), whose cached text keys are stored after the
qk-norm (section 1, item 1). The pages name the operator but not its
formulas; the readings below are the plain ones and are listed again in the
design notes:

  * RMSNorm runs per (token, head) over the head dimension d:
        y_c = x_c / sqrt(mean_c(x_c^2) + eps) * gamma_c,
    with eps inside the square root and one gamma[d] per tensor (q or k),
    shared by all heads.
  * Norm first, then RoPE (the operator's name and the "after qk-norm" cache).
  * The head dimension is cut into three contiguous blocks for the t, h and
    w axes (widths d_t, d_h, d_w, all even, in that order). Inside an axis
    block of width d_a, pair j = (2j, 2j+1) is rotated by the angle
    p_a * theta**(-2j / d_a), p_a being the token's position on that axis:
        (y0, y1) -> (y0 cos phi - y1 sin phi, y0 sin phi + y1 cos phi).
  * Tokens of the chunk are in (t, h, w) row-major order, w fastest; token n
    has t = t0 + n // (Hl*Wl), h = (n // Wl) % Hl, w = n % Wl.
  * The result is rounded to bf16 once, at the end.
"""
import numpy as np

from .bf16 import bf16_to_f64, f64_to_bf16


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMS normalisation over the last axis, then an elementwise gain."""
    x = np.asarray(x, dtype=np.float64)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x / r * np.asarray(gamma, dtype=np.float64)


def rope3d_angles(T: int, Hl: int, Wl: int, t0: int, d_t: int, d_h: int, d_w: int,
                  theta: float) -> np.ndarray:
    """Rotation angle of every (token, pair): fp64 array [T*Hl*Wl, (d_t+d_h+d_w)/2]."""
    for w in (d_t, d_h, d_w):
        if w % 2:
            raise ValueError("axis widths must be even")
    n = np.arange(T * Hl * Wl)
    pos = [t0 + n // (Hl * Wl), (n // Wl) % Hl, n % Wl]
    cols = []
    for p, d_a in zip(pos, (d_t, d_h, d_w)):
        j = np.arange(d_a // 2, dtype=np.float64)
        omega = float(theta) ** (-2.0 * j / d_a)
        cols.append(p[:, None].astype(np.float64) * omega[None, :])
    return np.concatenate(cols, axis=1)


def apply_rope(y: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate interleaved pairs of y [n, H, d] by angles [n, d/2] (shared by heads)."""
    y = np.asarray(y, dtype=np.float64)
    c = np.cos(angles)[:, None, :]
    s = np.sin(angles)[:, None, :]
    y0 = y[..., 0::2]
    y1 = y[..., 1::2]
    out = np.empty_like(y)
    out[..., 0::2] = y0 * c - y1 * s
    out[..., 1::2] = y0 * s + y1 * c
    return out


def qknorm_rope3d(x_bits: np.ndarray, gamma: np.ndarray, T: int, Hl: int, Wl: int, t0: int,
                  d_t: int, d_h: int, d_w: int, theta: float = 1.0e4, eps: float = 1.0e-6,
                  rounded: bool = True) -> np.ndarray:
    """Norm then rotate one tensor (q or k) of shape [T*Hl*Wl, H, d].

    Returns bf16 bits (``rounded``) or the unrounded fp64 result.
    """
    x = bf16_to_f64(x_bits)
    n, H, d = x.shape
    if n != T * Hl * Wl or d != d_t + d_h + d_w:
        raise ValueError("shape does not match the token grid or the axis split")
    y = rms_norm(x, gamma, eps)
    y = apply_rope(y, rope3d_angles(T, Hl, Wl, t0, d_t, d_h, d_w, theta))
    return f64_to_bf16(y) if rounded else y
