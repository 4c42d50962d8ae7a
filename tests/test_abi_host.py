"""Host-only checks of libpisa's C ABI: the library loads, exports every symbol
include/pisa.h declares, and rejects bad arguments before touching the GPU.

Every call here fails validation, which happens on the host before any HIP
call, so no device is needed.
"""

import ctypes
import os
import re

import pytest

from piecewise_block_sparse_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x1000)       # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libpisa.so is not built (run python -m piecewise_block_sparse_amd.build)")
    return _lib.load()


def shape(b=1, h=2, L=1024, d=128, B=64, dtype=_lib.DTYPE_BF16):
    return _lib.PisaShape(b, h, L, d, B, dtype)


def stats(full=True):
    p = FAKE.value
    return _lib.PisaStats(p, p, None, p, p, None) if full else _lib.PisaStats(None, p, None, p, p, None)


def test_exports_every_declared_symbol(lib):
    header = open(os.path.join(ROOT, "include", "pisa.h")).read()
    declared = set(re.findall(r"\b(pisa_\w+)\s*\(", header))
    assert declared == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.pisa_version() == 103


def test_probe_library_exports_its_declared_symbol():
    if not os.path.exists(_lib.PROBE_PATH):
        pytest.fail("libpisa_probe.so is not built (run python -m piecewise_block_sparse_amd.build)")
    header = open(os.path.join(ROOT, "include", "pisa_probe.h")).read()
    declared = set(re.findall(r"\b(pisa_\w+)\s*\(", header))
    assert declared == set(_lib.PROBE_EXPORTS)
    probe = _lib.load_probe()
    for name in declared:
        assert hasattr(probe, name), name
    # invalid arguments are rejected on the host (hipErrorInvalidValue = 1), nothing launched
    out = ctypes.c_double(0.0)
    assert probe.pisa_probe_chunk_rate(3, 0, 10, 1, ctypes.byref(out)) == 1
    assert probe.pisa_probe_chunk_rate(-1, 0, 10, 1, ctypes.byref(out)) == 1
    assert probe.pisa_probe_chunk_rate(0, 0, 0, 1, ctypes.byref(out)) == 1
    assert probe.pisa_probe_chunk_rate(0, 0, 10, 1, None) == 1
    assert probe.pisa_probe_read_rate(1 << 20, 1, ctypes.byref(out)) == 1      # below 32 MiB
    assert probe.pisa_probe_read_rate((1 << 30) + 8, 1, ctypes.byref(out)) == 1  # not 16-byte
    assert probe.pisa_probe_read_rate(1 << 30, 0, ctypes.byref(out)) == 1


def test_status_strings(lib):
    for code in range(7):
        assert lib.pisa_status_string(code)
    assert lib.pisa_status_string(99) == b"unknown status"


def pre(lib, shp, out=None, ws=FAKE, wsb=1 << 40):
    out = stats() if out is None else out
    return lib.pisa_precompute(ctypes.byref(shp) if shp else None, FAKE, FAKE,
                               ctypes.byref(out), ws, wsb, None)


def rte(lib, shp, k=4, scale=0.1, lam=0.1, Q=FAKE):
    return lib.pisa_route(ctypes.byref(shp), Q, FAKE, FAKE, k, scale, lam, FAKE, None)


def att(lib, shp, kmax=4, mode=0, scale=0.1, st=None, O=FAKE):
    st = stats() if st is None else st
    return lib.pisa_attention(ctypes.byref(shp), FAKE, FAKE, FAKE, FAKE, kmax, ctypes.byref(st),
                              mode, scale, O, None)


def test_shape_rules(lib):
    assert pre(lib, None) == 1
    assert pre(lib, shape(dtype=7)) == 4
    assert pre(lib, shape(L=1000)) == 2              # ragged last block
    assert pre(lib, shape(d=96)) == 2
    assert pre(lib, shape(B=32)) == 2
    assert pre(lib, shape(L=64 * 4096)) == 2         # more than 2048 blocks
    assert pre(lib, shape(b=0)) == 2
    assert pre(lib, shape(h=-1)) == 2
    assert rte(lib, shape(L=1000)) == 2
    assert att(lib, shape(L=1000)) == 2
    assert lib.pisa_workspace_size(ctypes.byref(shape(L=1000))) == 0


def test_precompute_arguments(lib):
    s = shape()
    assert pre(lib, s, out=stats(full=False)) == 1                 # missing centroid
    need = lib.pisa_workspace_size(ctypes.byref(s))
    # fp32 d x d per head: one partial per workgroup range (16 blocks in ranges of 4), then Hbar
    assert need == 2 * (16 // 4 + 1) * 128 * 128 * 4
    assert pre(lib, s, ws=None) == 1
    assert pre(lib, s, wsb=need - 1) == 5
    assert b"needs" in lib.pisa_last_error()
    f = shape(dtype=_lib.DTYPE_FP32, d=64)
    assert lib.pisa_workspace_size(ctypes.byref(f)) == 2 * 16 * 64 * 64 * 4
    assert lib.pisa_packed_size(ctypes.byref(s)) == 2 * (2 * 64 * 128 + 128 * 128) * 2   # nbp = 64
    assert lib.pisa_packed_size(ctypes.byref(shape(L=72 * 64))) == 2 * (2 * 128 * 128 + 128 * 128) * 2
    assert lib.pisa_packed_size(ctypes.byref(f)) == 0


def test_route_arguments(lib):
    s = shape()                                                     # nb = 16
    assert rte(lib, s, k=0) == 3
    assert rte(lib, s, k=17) == 3
    assert rte(lib, s, scale=float("nan")) == 3
    assert rte(lib, s, lam=float("inf")) == 3
    assert rte(lib, s, Q=None) == 1


def test_attention_arguments(lib):
    s = shape()
    assert att(lib, s, kmax=0) == 3
    assert att(lib, s, kmax=17) == 3
    assert att(lib, s, mode=4) == 3
    assert att(lib, s, mode=-1) == 3
    assert att(lib, s, scale=float("nan")) == 3
    assert att(lib, s, scale=-0.5) == 3
    assert att(lib, s, O=None) == 1
    assert att(lib, s, st=stats(full=False)) == 1                  # APPROX needs centroids
    assert b"centroid" in lib.pisa_last_error()
    for m in (_lib.MODE_ZEROTH, _lib.MODE_FIRST):
        assert att(lib, s, mode=m, st=stats(full=False)) == 1
    p = FAKE.value
    no_hbar = _lib.PisaStats(p, p, None, None, p, p, p)
    assert att(lib, s, mode=_lib.MODE_APPROX, st=no_hbar) == 1     # APPROX needs Hbar
    assert b"Hbar" in lib.pisa_last_error()
    no_ht = _lib.PisaStats(p, p, p, p, p, p, None)
    assert att(lib, s, mode=_lib.MODE_FIRST, st=no_ht) == 1        # bf16 FIRST needs Ht
    assert b"Ht" in lib.pisa_last_error()
    no_pack = _lib.PisaStats(p, p, p, p, p, None, p)
    assert att(lib, s, mode=_lib.MODE_FIRST, st=no_pack) == 1      # ... and the bf16 pack
    f = shape(dtype=_lib.DTYPE_FP32)
    no_h = _lib.PisaStats(p, p, None, p, p, None, p)
    assert att(lib, f, mode=_lib.MODE_FIRST, st=no_h) == 1         # fp32 FIRST needs H
    assert b"needs stats H" in lib.pisa_last_error()


def test_precompute_norm_option(lib):
    p = FAKE.value
    bad = _lib.PisaStats(p, p, None, p, p, None, None, 7)
    assert pre(lib, shape(), out=bad) == 3
    assert b"m_norm" in lib.pisa_last_error()
    spec_no_h = _lib.PisaStats(p, p, None, p, p, None, None, _lib.NORM_SPECTRAL)
    assert pre(lib, shape(), out=spec_no_h) == 1                    # bf16 spectral reads H
    assert b"needs the H output" in lib.pisa_last_error()


def test_precompute_Ht_is_bf16_only(lib):
    p = FAKE.value
    out = _lib.PisaStats(p, p, None, p, p, None, p)
    assert pre(lib, shape(dtype=_lib.DTYPE_FP32), out=out) == 3
    assert b"Ht" in lib.pisa_last_error()


def ra(lib, shp, k=4, lam=0.1, mode=0, scale=0.1, st=None, O=FAKE, idx=None,
       form=_lib.ROUTE_IN_KERNEL):
    st = stats() if st is None else st
    return lib.pisa_route_attention(ctypes.byref(shp), FAKE, FAKE, FAKE, ctypes.byref(st), k, lam,
                                    mode, scale, idx, O, form, None)


def test_route_attention_arguments(lib):
    s = shape()                                                     # nb = 16
    assert ra(lib, shape(L=1000)) == 2
    assert ra(lib, s, k=0) == 3
    assert ra(lib, s, k=17) == 3
    assert ra(lib, s, lam=float("nan")) == 3
    assert ra(lib, s, scale=float("inf")) == 3
    assert ra(lib, s, scale=1e-300) == 3                            # zero as a float
    assert ra(lib, s, mode=9) == 3
    assert ra(lib, s, mode=_lib.MODE_FIRST) == 3
    assert b"pisa_route" in lib.pisa_last_error()
    assert ra(lib, s, O=None) == 1
    p = FAKE.value
    assert ra(lib, s, st=_lib.PisaStats(p, p, None, p, None, None)) == 1    # routing reads M
    assert ra(lib, s, st=_lib.PisaStats(p, p, None, None, p, None)) == 1    # APPROX reads Hbar
    assert ra(lib, s, mode=_lib.MODE_ZEROTH, st=_lib.PisaStats(p, None, None, None, p, None)) == 1
    assert ra(lib, shape(dtype=_lib.DTYPE_FP32)) == 4
    # score rows that do not fit the kernel's LDS: 64-token blocks, d = 128, nb = 1921
    assert ra(lib, shape(L=64 * 1921)) == 2
    assert b"pisa_route, then pisa_attention" in lib.pisa_last_error()
    assert ra(lib, shape(L=64 * 961, d=64)) == 2                    # d = 64: nb <= 960
    # the form: known values only; two launches need idx for the selection
    assert ra(lib, s, form=3) == 3
    assert ra(lib, s, form=-1) == 3
    assert ra(lib, s, form=_lib.ROUTE_TWO_LAUNCH) == 1
    assert b"two-launch" in lib.pisa_last_error()
    # without idx the automatic form routes in-kernel, so the LDS limit holds
    assert ra(lib, shape(L=64 * 1921), form=_lib.ROUTE_AUTO) == 2


def test_noalloc_precompute_refuses_shapes_above_its_scratch(lib):
    # validation on the host: nothing is launched and no HIP call is made
    fake = 1 << 40                                                   # never dereferenced
    big = _lib.PisaShape(1, 48, 32768, 128, 64, _lib.DTYPE_BF16, None)
    need = lib.pisa_workspace_size(ctypes.byref(big))
    assert need > 64 << 20
    st = _lib.PisaStats(fake, fake, None, fake, fake, None, None, 0)
    assert lib.pisa_precompute_noalloc(ctypes.byref(big), fake, fake, ctypes.byref(st), None) == 5
    assert b"pisa_precompute with a workspace" in lib.pisa_last_error()
    assert lib.pisa_precompute_noalloc(ctypes.byref(big), None, fake, ctypes.byref(st), None) == 1
    bad = _lib.PisaShape(1, 2, 1000, 128, 64, _lib.DTYPE_BF16, None)
    assert lib.pisa_precompute_noalloc(ctypes.byref(bad), fake, fake, ctypes.byref(st), None) == 2


def test_sizes_of_very_large_shapes_do_not_wrap(lib):
    # 2^26 - 1 heads of two 64-token blocks: every size is far above 2^32 bytes
    # and must come out exact (host arithmetic in 64 bits)
    h = (1 << 26) - 1
    s = shape(h=h, L=128)
    assert lib.pisa_packed_size(ctypes.byref(s)) == h * (2 * 64 * 128 + 128 * 128) * 2     # nbp = 64
    assert lib.pisa_workspace_size(ctypes.byref(s)) == h * (1 + 1) * 128 * 128 * 4      # one range per head
    # 2^27 heads: the Hbar reduction's grid (16 workgroups per head) would not fit an int
    big = shape(h=1 << 27, L=64)
    assert lib.pisa_workspace_size(ctypes.byref(big)) == 0
    assert pre(lib, big) == 2
    assert b"2^27" in lib.pisa_last_error()
    # split attention whose parts would overflow one grid: refused on the host
    fake = 1 << 40                                                  # never dereferenced
    s = shape(h=h, L=32 * 64)                                       # nb = 32: 16 pairs per head
    rc = lib.pisa_attention_split(ctypes.byref(s), fake, fake, fake, fake, 16, None, 1, 0.125, 1, fake,
                                  fake, 1 << 62, None)
    assert rc == 2
    assert b"exceed one grid" in lib.pisa_last_error()


def test_split_attention_arguments(lib):
    s = shape()                                                     # nb = 16, 64-token blocks
    fake = 1 << 40                                                  # never dereferenced
    need = lib.pisa_attention_split_workspace_size(ctypes.byref(s), 8, 3)
    # pairs of query blocks: 8 items per head, 2 heads; an item holds up to
    # min(nb, 2 kmax) = 16 blocks, so up to 6 parts of 3; a part's slot is
    # 128 rows x (128 + 2) fp32; the parts-per-item array takes 256 bytes
    assert need == 256 + 2 * 8 * 6 * 128 * 130 * 4
    assert lib.pisa_attention_split_workspace_size(ctypes.byref(s), 8, 0) == 0
    assert lib.pisa_attention_split_workspace_size(ctypes.byref(s), 17, 3) == 0
    f = shape(dtype=_lib.DTYPE_FP32)
    assert lib.pisa_attention_split_workspace_size(ctypes.byref(f), 8, 3) == 0
    call = lambda shp=s, mode=1, maxb=3, ws=fake, wsb=need: lib.pisa_attention_split(
        ctypes.byref(shp), fake, fake, fake, fake, 8, None, mode, 0.125, maxb, fake, ws, wsb, None)
    assert call(wsb=need - 1) == 5
    assert call(ws=None) == 1
    assert call(maxb=0) == 3
    assert call(mode=3) == 3                                        # the per-block first order
    assert call(mode=0) == 1                                        # APPROX needs the statistics
    assert call(shp=f) == 4
