"""Python binding of the sdit C ABI (include/sdit.h).

Argument marshalling only: every step of the hot path runs in the HIP
kernels of libsdit.so. Tensors are passed as device pointers (torch tensors
or raw integer addresses); the stream defaults to torch's current stream.
The library is loaded on first use; every call fails loudly (ImportError)
when the built library is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsdit.so")
# test-only build of the same library with a one-tile-at-a-time attention schedule
SINGLE_STAGE_LIB_PATH = os.path.join(HERE, "libsdit_single_stage.so")

SDIT_OK, SDIT_ERR_INVALID, SDIT_ERR_UNSUPPORTED, SDIT_ERR_DEVICE = 0, 1, 2, 3
SDIT_BF16, SDIT_INT8 = 0, 1
SDIT_MAX_SEGMENTS = 8
ABI_VERSION = 1

_lib = None


class KVSegment(ctypes.Structure):
    """struct sdit_kv_segment."""
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("len", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_i32, _f32, _vp = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p


def lib() -> ctypes.CDLL:
    """The loaded libsdit.so (loaded on first use; raises if it was not built)."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


def load_library(path: str) -> ctypes.CDLL:
    """Load a build of the sdit library (libsdit.so, or the test-only
    libsdit_single_stage.so) and declare the C signatures."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m streaming_video_dit_amd.build`")
    L = ctypes.CDLL(path)
    L.sdit_abi_version.restype = ctypes.c_int
    L.sdit_status_string.restype = ctypes.c_char_p
    L.sdit_status_string.argtypes = [ctypes.c_int]
    L.sdit_last_error.restype = ctypes.c_char_p
    L.sdit_qknorm_rope3d.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp] + [_i32] * 9 + [_f32, _f32, _vp]
    L.sdit_validate_qknorm_rope3d_args.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp] + [_i32] * 9 + [_f32, _f32]
    L.sdit_qknorm_rope3d_kv_quant_int8.argtypes = [_vp] * 11 + [_i32] * 9 + [_f32, _f32, _vp]
    L.sdit_validate_qknorm_rope3d_kv_quant_int8_args.argtypes = [_vp] * 11 + [_i32] * 9 + [_f32, _f32]
    L.sdit_kv_quant_int8.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _vp]
    L.sdit_validate_kv_quant_args.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32]
    L.sdit_attn_fwd.argtypes = [_vp, _i32, ctypes.POINTER(KVSegment), _i32, _vp, _i32, _i32, _i32, _i32, _f32,
                                _vp, _vp, _vp]
    L.sdit_validate_attn_args.argtypes = [_vp, _i32, ctypes.POINTER(KVSegment), _i32, _vp, _i32, _i32, _i32,
                                          _i32, _f32, _vp, _vp]
    L.sdit_attn_fwd_partial.argtypes = L.sdit_attn_fwd.argtypes
    L.sdit_validate_attn_partial_args.argtypes = L.sdit_validate_attn_args.argtypes
    _i64 = ctypes.c_int64
    L.sdit_attn_fwd_balanced.argtypes = L.sdit_attn_fwd.argtypes[:-1] + [_vp, _i64, _i32, _vp]
    L.sdit_validate_attn_balanced_args.argtypes = L.sdit_validate_attn_args.argtypes + [_vp, _i64, _i32]
    L.sdit_attn_fwd_balanced_static.argtypes = L.sdit_attn_fwd.argtypes[:-1] + [_i32, _vp]
    _pi32 = ctypes.POINTER(ctypes.c_int32)
    L.sdit_attn_balanced_plan.argtypes = [_i32, _i32, _i32, _i32, _i32, _pi32, _pi32]
    _pp = ctypes.POINTER(ctypes.c_void_p)
    L.sdit_attn_merge.argtypes = [_pp, _pp, _i32, _i32, _i32, _i32, _vp, _vp, _vp]
    L.sdit_validate_attn_merge_args.argtypes = [_pp, _pp, _i32, _i32, _i32, _i32, _vp, _vp]
    L.sdit_window_permute.argtypes = [_vp, _vp] + [_i32] * 7 + [_vp]
    L.sdit_validate_window_permute_args.argtypes = [_vp, _vp] + [_i32] * 7
    L.sdit_rmsnorm.argtypes = [_vp, _vp, _vp, _i64, _i32, _f32, _vp]
    L.sdit_validate_rmsnorm_args.argtypes = [_vp, _vp, _vp, _i64, _i32, _f32]
    L.sdit_layernorm_modulate.argtypes = [_vp, _vp, _vp, _vp, _i64, _i32, _f32, _vp]
    L.sdit_validate_layernorm_modulate_args.argtypes = [_vp, _vp, _vp, _vp, _i64, _i32, _f32]
    for n in ("sdit_window_permute", "sdit_validate_window_permute_args", "sdit_rmsnorm",
              "sdit_validate_rmsnorm_args", "sdit_layernorm_modulate", "sdit_validate_layernorm_modulate_args",
              "sdit_qknorm_rope3d", "sdit_validate_qknorm_rope3d_args", "sdit_kv_quant_int8",
              "sdit_validate_kv_quant_args", "sdit_attn_fwd", "sdit_validate_attn_args",
              "sdit_attn_fwd_partial", "sdit_validate_attn_partial_args", "sdit_attn_merge",
              "sdit_validate_attn_merge_args", "sdit_attn_fwd_balanced", "sdit_validate_attn_balanced_args",
              "sdit_attn_balanced_plan", "sdit_attn_fwd_balanced_static", "sdit_qknorm_rope3d_kv_quant_int8",
              "sdit_validate_qknorm_rope3d_kv_quant_int8_args"):
        getattr(L, n).restype = ctypes.c_int
    if L.sdit_abi_version() != ABI_VERSION:
        raise ImportError(f"{path} ABI {L.sdit_abi_version()} != binding ABI {ABI_VERSION}")
    return L


class SditError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{lib().sdit_status_string(status).decode()}: {message}")
        self.status = status


def last_error() -> str:
    return lib().sdit_last_error().decode()


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != SDIT_OK:
        raise SditError(status, last_error())


def qknorm_rope3d(q_in, k_in, q_out, k_out, gamma_q, gamma_k, T: int, Hl: int, Wl: int, t0: int,
                  n_heads: int, head_dim: int, d_t: int, d_h: int, d_w: int,
                  theta: float = 1.0e4, eps: float = 1.0e-6, stream=None) -> None:
    """sdit_qknorm_rope3d."""
    _check(lib().sdit_qknorm_rope3d(_ptr(q_in), _ptr(k_in), _ptr(q_out), _ptr(k_out), _ptr(gamma_q), _ptr(gamma_k),
                                   T, Hl, Wl, t0, n_heads, head_dim, d_t, d_h, d_w, theta, eps, _stream(stream)))


def qknorm_rope3d_kv_quant_int8(q_in, k_in, v_in, q_out, k_out, k_codes, k_scales, v_codes, v_scales, gamma_q,
                                gamma_k, T: int, Hl: int, Wl: int, t0: int, n_heads: int, head_dim: int, d_t: int,
                                d_h: int, d_w: int, theta: float = 1.0e4, eps: float = 1.0e-6, stream=None) -> None:
    """sdit_qknorm_rope3d_kv_quant_int8."""
    _check(lib().sdit_qknorm_rope3d_kv_quant_int8(
        _ptr(q_in), _ptr(k_in), _ptr(v_in), _ptr(q_out), _ptr(k_out), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes),
        _ptr(v_scales), _ptr(gamma_q), _ptr(gamma_k), T, Hl, Wl, t0, n_heads, head_dim, d_t, d_h, d_w, theta, eps,
        _stream(stream)))


def validate_qknorm_rope3d_kv_quant_int8_args(q_in, k_in, v_in, q_out, k_out, k_codes, k_scales, v_codes, v_scales,
                                              gamma_q, gamma_k, T, Hl, Wl, t0, n_heads, head_dim, d_t, d_h, d_w,
                                              theta=1.0e4, eps=1.0e-6) -> int:
    return lib().sdit_validate_qknorm_rope3d_kv_quant_int8_args(
        _ptr(q_in), _ptr(k_in), _ptr(v_in), _ptr(q_out), _ptr(k_out), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes),
        _ptr(v_scales), _ptr(gamma_q), _ptr(gamma_k), T, Hl, Wl, t0, n_heads, head_dim, d_t, d_h, d_w, theta, eps)


def kv_quant_int8(x, codes, scales, n_tok: int, n_heads: int, head_dim: int, stream=None) -> None:
    """sdit_kv_quant_int8."""
    _check(lib().sdit_kv_quant_int8(_ptr(x), _ptr(codes), _ptr(scales), n_tok, n_heads, head_dim, _stream(stream)))


def window_permute(x, y, T: int, Hl: int, Wl: int, n_heads: int, head_dim: int, window: int = 8,
                   inverse: bool = False, stream=None) -> None:
    """sdit_window_permute."""
    _check(lib().sdit_window_permute(_ptr(x), _ptr(y), T, Hl, Wl, n_heads, head_dim, window, int(inverse),
                                    _stream(stream)))


def validate_window_permute_args(x, y, T, Hl, Wl, n_heads, head_dim, window=8, inverse=False) -> int:
    return lib().sdit_validate_window_permute_args(_ptr(x), _ptr(y), T, Hl, Wl, n_heads, head_dim, window,
                                                  int(inverse))


def rmsnorm(x, y, gamma, n_tok: int, dim: int, eps: float = 1e-6, stream=None) -> None:
    """sdit_rmsnorm."""
    _check(lib().sdit_rmsnorm(_ptr(x), _ptr(y), _ptr(gamma), n_tok, dim, eps, _stream(stream)))


def validate_rmsnorm_args(x, y, gamma, n_tok, dim, eps=1e-6) -> int:
    return lib().sdit_validate_rmsnorm_args(_ptr(x), _ptr(y), _ptr(gamma), n_tok, dim, eps)


def layernorm_modulate(x, y, scale, shift, n_tok: int, dim: int, eps: float = 1e-6, stream=None) -> None:
    """sdit_layernorm_modulate."""
    _check(lib().sdit_layernorm_modulate(_ptr(x), _ptr(y), _ptr(scale), _ptr(shift), n_tok, dim, eps,
                                         _stream(stream)))


def validate_layernorm_modulate_args(x, y, scale, shift, n_tok, dim, eps=1e-6) -> int:
    return lib().sdit_validate_layernorm_modulate_args(_ptr(x), _ptr(y), _ptr(scale), _ptr(shift), n_tok, dim,
                                                       eps)


def make_segments(segs: Sequence[dict]):
    """Host array of sdit_kv_segment from dicts with k, v, len, dtype and
    (int8) k_scale, v_scale."""
    arr = (KVSegment * max(1, len(segs)))()
    for i, s in enumerate(segs):
        arr[i].k = _ptr(s.get("k"))
        arr[i].v = _ptr(s.get("v"))
        arr[i].k_scale = _ptr(s.get("k_scale"))
        arr[i].v_scale = _ptr(s.get("v_scale"))
        arr[i].len = int(s["len"])
        arr[i].dtype = int(s.get("dtype", SDIT_BF16))
    return arr


def attn_fwd(q, n_q: int, segs, block_mask, block_q: int, block_k: int, n_heads: int, head_dim: int,
             out, lse=None, softmax_scale: float = 0.0, stream=None, library=None) -> None:
    """sdit_attn_fwd. ``segs`` is a list of dicts (see make_segments) or a
    ctypes array made by make_segments. ``library``: another build loaded
    with load_library (default libsdit.so)."""
    arr = segs if isinstance(segs, ctypes.Array) else make_segments(segs)
    n = len(segs)
    L = library if library is not None else lib()
    _check(L.sdit_attn_fwd(_ptr(q), n_q, arr, n, _ptr(block_mask), block_q, block_k, n_heads, head_dim,
                           softmax_scale, _ptr(out), _ptr(lse), _stream(stream)))


def attn_workspace_bytes(head_dim: int) -> int:
    """SDIT_ATTN_WORKSPACE_BYTES(head_dim): workspace size of attn_fwd_balanced."""
    return 8 * 31 * 2 * 256 * (head_dim + 1) * 4


def attn_fwd_balanced(q, n_q: int, segs, block_mask, block_q: int, block_k: int, n_heads: int, head_dim: int,
                      out, workspace, lse=None, softmax_scale: float = 0.0, split_tile: int = -1,
                      workspace_bytes=None, stream=None, library=None) -> None:
    """sdit_attn_fwd_balanced: ``workspace`` is device memory of at least
    attn_workspace_bytes(head_dim) bytes (its size is taken from the tensor
    unless ``workspace_bytes`` is given)."""
    arr = segs if isinstance(segs, ctypes.Array) else make_segments(segs)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    L = library if library is not None else lib()
    _check(L.sdit_attn_fwd_balanced(_ptr(q), n_q, arr, len(segs), _ptr(block_mask), block_q, block_k, n_heads,
                                    head_dim, softmax_scale, _ptr(out), _ptr(lse), _ptr(workspace),
                                    workspace_bytes, split_tile, _stream(stream)))


def attn_fwd_balanced_static(q, n_q: int, segs, block_mask, block_q: int, block_k: int, n_heads: int,
                             head_dim: int, out, lse=None, softmax_scale: float = 0.0, split_tile: int = -1,
                             stream=None) -> None:
    """sdit_attn_fwd_balanced_static: the balanced launch with the library's
    own device scratch (no workspace argument, nothing allocated)."""
    arr = segs if isinstance(segs, ctypes.Array) else make_segments(segs)
    _check(lib().sdit_attn_fwd_balanced_static(_ptr(q), n_q, arr, len(segs), _ptr(block_mask), block_q, block_k,
                                               n_heads, head_dim, softmax_scale, _ptr(out), _ptr(lse), split_tile,
                                               _stream(stream)))


def attn_balanced_plan(n_q: int, n_heads: int, n_tiles: int, n_cus: int, split_tile: int = -1):
    """sdit_attn_balanced_plan: (key tile of the cut or 0, workgroups of the launch)."""
    t, g = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().sdit_attn_balanced_plan(n_q, n_heads, n_tiles, n_cus, split_tile, ctypes.byref(t), ctypes.byref(g)))
    return t.value, g.value


def validate_attn_balanced_args(q, n_q, segs, block_mask, block_q, block_k, n_heads, head_dim, out, lse,
                                workspace, workspace_bytes, split_tile=-1, softmax_scale: float = 0.0) -> int:
    arr = segs if isinstance(segs, ctypes.Array) else make_segments(segs)
    return lib().sdit_validate_attn_balanced_args(_ptr(q), n_q, arr, len(segs), _ptr(block_mask), block_q, block_k,
                                                 n_heads, head_dim, softmax_scale, _ptr(out), _ptr(lse),
                                                 _ptr(workspace), workspace_bytes, split_tile)


def attn_fwd_partial(q, n_q: int, segs, block_mask, block_q: int, block_k: int, n_heads: int, head_dim: int,
                     out, lse, softmax_scale: float = 0.0, stream=None) -> None:
    """sdit_attn_fwd_partial: ``out`` fp32 [n_q, H, d], ``lse`` fp32 [H, n_q]."""
    arr = segs if isinstance(segs, ctypes.Array) else make_segments(segs)
    _check(lib().sdit_attn_fwd_partial(_ptr(q), n_q, arr, len(segs), _ptr(block_mask), block_q, block_k, n_heads,
                                      head_dim, softmax_scale, _ptr(out), _ptr(lse), _stream(stream)))


def _pointer_array(xs):
    arr = (ctypes.c_void_p * max(1, len(xs)))()
    for i, x in enumerate(xs):
        arr[i] = _ptr(x)
    return arr


def attn_merge(o_parts, lse_parts, n_q: int, n_heads: int, head_dim: int, out, lse_out=None,
               stream=None) -> None:
    """sdit_attn_merge: lists of fp32 partial outputs and their LSEs."""
    _check(lib().sdit_attn_merge(_pointer_array(o_parts), _pointer_array(lse_parts), len(o_parts), n_q, n_heads,
                                head_dim, _ptr(out), _ptr(lse_out), _stream(stream)))


def validate_attn_partial_args(q, n_q, segs, block_mask, block_q, block_k, n_heads, head_dim, out, lse,
                               softmax_scale: float = 0.0) -> int:
    arr = segs if isinstance(segs, ctypes.Array) else make_segments(segs)
    return lib().sdit_validate_attn_partial_args(_ptr(q), n_q, arr, len(segs), _ptr(block_mask), block_q, block_k,
                                                n_heads, head_dim, softmax_scale, _ptr(out), _ptr(lse))


def validate_attn_merge_args(o_parts, lse_parts, n_q, n_heads, head_dim, out, lse_out=None) -> int:
    return lib().sdit_validate_attn_merge_args(_pointer_array(o_parts), _pointer_array(lse_parts), len(o_parts),
                                              n_q, n_heads, head_dim, _ptr(out), _ptr(lse_out))


def validate_attn_args(q, n_q, segs, block_mask, block_q, block_k, n_heads, head_dim, out, lse=None,
                       softmax_scale: float = 0.0) -> int:
    arr = segs if isinstance(segs, ctypes.Array) else make_segments(segs)
    return lib().sdit_validate_attn_args(_ptr(q), n_q, arr, len(segs), _ptr(block_mask), block_q, block_k, n_heads,
                                        head_dim, softmax_scale, _ptr(out), _ptr(lse))


def validate_qknorm_rope3d_args(q_in, k_in, q_out, k_out, gamma_q, gamma_k, T, Hl, Wl, t0, n_heads, head_dim,
                                d_t, d_h, d_w, theta=1.0e4, eps=1.0e-6) -> int:
    return lib().sdit_validate_qknorm_rope3d_args(_ptr(q_in), _ptr(k_in), _ptr(q_out), _ptr(k_out), _ptr(gamma_q),
                                                 _ptr(gamma_k), T, Hl, Wl, t0, n_heads, head_dim, d_t, d_h, d_w,
                                                 theta, eps)


def validate_kv_quant_args(x, codes, scales, n_tok, n_heads, head_dim) -> int:
    return lib().sdit_validate_kv_quant_args(_ptr(x), _ptr(codes), _ptr(scales), n_tok, n_heads, head_dim)
