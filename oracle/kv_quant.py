"""Symmetric int8 K/V cache quantisation, one fp32 scale per (token, head)
(test infrastructure only).

The Joy-face_change_optimized README (section 1, int8 K/V bullet) stores the
cached K/V as int8 scaled per token and head; the cache shrinks from 1.44 to
0.74 GiB, which is what fp32 scales give at head_dim 128 ((128 + 4) / 256 =
0.516). The pages give no formula; the reading used here is the plain
symmetric one, with every rounding fixed so the result is unique:

  amax    = max_c |x_c|                     (exact)
  scale   = fl32(amax / 127)                (IEEE binary32 quotient)
  code_c  = clamp(rne(fl32(x_c / scale)), -127, 127)
  amax == 0  ->  scale = 0 and every code 0.

The binary32 quotient of two binary32 numbers equals the fp64 quotient
rounded to binary32 (fp64 carries more than 2*24+2 bits, so the double
rounding is harmless); the oracle computes it that way. rne is round half
to even (numpy.rint).
"""
import numpy as np

from .bf16 import bf16_to_f64


def kv_quant_int8(x_bits: np.ndarray):
    """bf16 bits [N, H, d] -> (int8 codes [N, H, d], fp32 scales [N, H])."""
    x = bf16_to_f64(x_bits)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / 127.0).astype(np.float32)
    s64 = scale.astype(np.float64)[..., None]
    safe = np.where(s64 > 0, s64, 1.0)
    quot = (x / safe).astype(np.float32).astype(np.float64)
    code = np.clip(np.rint(quot), -127, 127)
    code = np.where(s64 > 0, code, 0.0)
    return code.astype(np.int8), scale


def kv_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact fp64 value of code * scale (7 + 24 significant bits fit in fp64)."""
    return codes.astype(np.float64) * scales.astype(np.float64)[..., None]
