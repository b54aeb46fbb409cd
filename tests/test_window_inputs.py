"""The windowed workloads' locality mask (built by the input generator) equals
the oracle's definition (CPU only)."""
import numpy as np
import pytest

import workloads as W
from oracle import local_window_mask


@pytest.mark.parametrize("name", ["vsr_local", "tiny_local"])
def test_workload_local_mask_equals_oracle(name):
    cfg = W.WORKLOADS[name]
    m = W.make_mask(cfg)
    ref = local_window_mask(cfg.T, cfg.Hl, cfg.Wl, cfg.window, cfg.local_range)
    assert np.array_equal(m, ref)
    assert cfg.block == cfg.window ** 2
