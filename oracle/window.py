"""Token order of windowed (locality) sparse attention (test infrastructure
only).

Source: FlashVSR deployment notes, spatial tiling section: one token covers
16 x 16 output pixels, one attention block is a window of 8 x 8 tokens
(128 px), and local_range = 11 blocks reaches +-640 px, i.e. +-5 windows.
For a block of the block-sparse attention to be a spatial window, the tokens
(raster order t, h, w within a clip) are reordered window by window.

Readings (the page is silent on them):
  * window-major order: frame t, then window row h // win, then window column
    w // win; inside a window, raster order (h % win, w % win);
  * frame height and width are multiples of the window (the page aligns its
    tiles to 128 px, i.e. whole windows);
  * the locality mask keeps a key window when both its window row and its
    window column are within radius r = (local_range - 1) / 2 of the query
    window's, in every frame of the clip.

window_order(T, Hl, Wl, win)[j] is the raster index of the token at window-
major position j, so x_window = x_raster[order] and
x_raster[order] = x_window.
"""
import numpy as np


def window_order(T: int, Hl: int, Wl: int, win: int) -> np.ndarray:
    if Hl % win or Wl % win:
        raise ValueError("frame sides must be multiples of the window")
    t, wy, wx, iy, ix = np.meshgrid(np.arange(T), np.arange(Hl // win), np.arange(Wl // win),
                                    np.arange(win), np.arange(win), indexing="ij")
    h = wy * win + iy
    w = wx * win + ix
    return (t * Hl * Wl + h * Wl + w).reshape(-1).astype(np.int64)


def window_coords(T: int, Hl: int, Wl: int, win: int):
    """(frame, window row, window column) of every window, in window-major order."""
    t, wy, wx = np.meshgrid(np.arange(T), np.arange(Hl // win), np.arange(Wl // win), indexing="ij")
    return t.reshape(-1), wy.reshape(-1), wx.reshape(-1)


def local_window_mask(T: int, Hl: int, Wl: int, win: int, local_range: int) -> np.ndarray:
    """uint8 [n_windows][n_windows] keep mask of windowed attention: key window
    kept when its window row and column are both within (local_range - 1) / 2
    of the query window's, in any frame."""
    if local_range % 2 != 1:
        raise ValueError("local_range must be odd (a centred range)")
    r = (local_range - 1) // 2
    _, wy, wx = window_coords(T, Hl, Wl, win)
    keep = (np.abs(wy[:, None] - wy[None, :]) <= r) & (np.abs(wx[:, None] - wx[None, :]) <= r)
    return keep.astype(np.uint8)
