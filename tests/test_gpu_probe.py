"""The measurement probe (include/pisa_probe.h) runs and reports a plausible rate."""
import ctypes
import math

import pytest

from piecewise_block_sparse_amd import _lib

pytestmark = pytest.mark.gpu


def test_probe_rates_are_below_the_published_peak():
    import torch
    torch.cuda.set_device(0)
    probe = _lib.load_probe()
    rates = {}
    for mix, zeros in ((0, 0), (1, 0), (1, 1), (2, 0), (2, 1)):
        r = ctypes.c_double(0.0)
        assert probe.pisa_probe_chunk_rate(mix, zeros, 200, 2, ctypes.byref(r)) == 0
        assert math.isfinite(r.value) and 0.0 < r.value < 2500.0 * 1.05, (mix, zeros, r.value)
        rates[(mix, zeros)] = r.value
    # the softmax work can only slow the same MFMAs down (small launches are noisy)
    assert rates[(1, 0)] < 1.1 * rates[(0, 0)]
    # feeding the MFMAs from LDS can only slow the register-only stream down
    assert rates[(0, 0)] < 1.1 * rates[(2, 0)]


def test_read_probe_is_below_the_published_hbm_peak():
    import torch
    torch.cuda.set_device(0)
    probe = _lib.load_probe()
    r = ctypes.c_double(0.0)
    assert probe.pisa_probe_read_rate(1 << 30, 2, ctypes.byref(r)) == 0
    assert math.isfinite(r.value) and 1000.0 < r.value < 8000.0 * 1.05, r.value
