"""Pins for the oracle's window order and locality mask (CPU only): brute
force with plain loops over the page's definitions (8 x 8-token windows,
local_range in windows), permutation and inverse, and the mask's symmetry and
row counts in closed form."""
import numpy as np
import pytest

from oracle.window import local_window_mask, window_coords, window_order


@pytest.mark.parametrize("shape", [(1, 8, 8, 8), (2, 16, 24, 8), (3, 8, 16, 4), (2, 4, 6, 2)])
def test_window_order_brute_force(shape):
    T, Hl, Wl, win = shape
    order = window_order(T, Hl, Wl, win)
    # a permutation of all tokens
    assert np.array_equal(np.sort(order), np.arange(T * Hl * Wl))
    # block b (win * win consecutive positions) holds exactly window b's tokens, in raster order
    pos = 0
    for t in range(T):
        for wy in range(Hl // win):
            for wx in range(Wl // win):
                for iy in range(win):
                    for ix in range(win):
                        assert order[pos] == t * Hl * Wl + (wy * win + iy) * Wl + (wx * win + ix)
                        pos += 1
    # inverse: scattering back restores raster order
    x = np.arange(T * Hl * Wl) * 7 + 3
    y = x[order]
    back = np.empty_like(x)
    back[order] = y
    assert np.array_equal(back, x)


def test_window_order_rejects_partial_windows():
    with pytest.raises(ValueError):
        window_order(1, 12, 16, 8)


def test_local_mask_closed_form():
    T, Hl, Wl, win, rng = 2, 96, 168, 8, 11      # the page's 2688 x 1536 clip geometry, two frames
    m = local_window_mask(T, Hl, Wl, win, rng)
    nwy, nwx = Hl // win, Wl // win
    assert m.shape == (T * nwy * nwx,) * 2
    assert np.array_equal(m, m.T)
    assert np.all(np.diag(m) == 1)
    t, wy, wx = window_coords(T, Hl, Wl, win)
    # kept key windows of a query window = T * (rows within 5) * (columns within 5)
    ny = np.minimum(wy + 5, nwy - 1) - np.maximum(wy - 5, 0) + 1
    nx = np.minimum(wx + 5, nwx - 1) - np.maximum(wx - 5, 0) + 1
    assert np.array_equal(m.sum(axis=1), T * ny * nx)
    # a centre window of a wide frame keeps 11 x 11 windows per frame
    assert m.sum(axis=1).max() == T * 11 * 11
    with pytest.raises(ValueError):
        local_window_mask(T, Hl, Wl, win, 10)
