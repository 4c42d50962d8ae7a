"""pisa_precompute_noalloc (the workspace in the library's static device array)
gives pisa_precompute's results bit for bit, called through the C ABI twice in
a row, the second call on a smaller input."""
import ctypes

import numpy as np
import pytest

import piecewise_block_sparse_amd as pisa
from piecewise_block_sparse_amd import _lib
from piecewise_block_sparse_amd import workloads as wl

pytestmark = pytest.mark.gpu

KEYS = ("centroid", "vsum", "Hbar", "M", "packed")


def _inputs(torch, h, L, d, seed):
    g = np.random.default_rng(seed)
    K, V = (wl.round_bf16(g.standard_normal((1, h, L, d)).astype(np.float32)) for _ in range(2))
    return tuple(torch.from_numpy(x).to("cuda:0", torch.bfloat16) for x in (K, V))


def _noalloc(torch, K, V, block):
    """The outputs pisa.precompute returns, filled by pisa_precompute_noalloc."""
    lib = _lib.load()
    b, h, L, d = K.shape
    nb = L // block
    shp = _lib.PisaShape(b, h, L, d, block, _lib.DTYPE_BF16, None)
    f32 = dict(dtype=torch.float32, device=K.device)
    out = {"centroid": torch.full((b, h, nb, d), float("nan"), **f32),
           "vsum": torch.full((b, h, nb, d), float("nan"), **f32),
           "Hbar": torch.full((b, h, d, d), float("nan"), **f32),
           "M": torch.full((b, h, nb), float("nan"), **f32),
           "packed": torch.full((lib.pisa_packed_size(ctypes.byref(shp)),), 0xFF, dtype=torch.uint8,
                                device=K.device)}
    st = _lib.PisaStats(out["centroid"].data_ptr(), out["vsum"].data_ptr(), None,
                        out["Hbar"].data_ptr(), out["M"].data_ptr(), out["packed"].data_ptr(), None,
                        _lib.NORM_FROBENIUS)
    stream = torch.cuda.current_stream().cuda_stream
    rc = lib.pisa_precompute_noalloc(ctypes.byref(shp), K.data_ptr(), V.data_ptr(),
                                     ctypes.byref(st), stream)
    assert rc == _lib.PISA_OK, lib.pisa_last_error().decode()
    return out


@pytest.mark.parametrize("d", [128, 64])
def test_noalloc_precompute_matches_precompute_twice(d):
    import torch
    torch.cuda.set_device(0)
    # a larger input first, then a smaller one with another block size: the
    # second call reuses the static array the first one filled
    for h, L, block, seed in ((8, 8192, 128, 11), (3, 2048, 64, 12)):
        print(f"noalloc precompute: h={h} L={L} d={d} block={block} seed={seed}", flush=True)
        K, V = _inputs(torch, h, L, d, seed)
        ref = pisa.precompute(K, V, block)
        got = _noalloc(torch, K, V, block)
        torch.cuda.synchronize()
        for key in KEYS:
            assert torch.equal(got[key], ref[key]), (key, h, L, d, block)
