"""Host checks of the seeded input generators and the fixed multimodal mask."""

import os

import numpy as np
import torch
import torch.nn.functional as F

from piecewise_block_sparse_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_grid(name):
    rows = [ln.strip() for ln in open(os.path.join(GOLDEN, name)) if ln.strip() and ln[0] != "#"]
    return np.array([[int(c) for c in r] for r in rows], dtype=np.int8)


def test_round_bf16_matches_torch():
    g = np.random.default_rng(0)
    x = (g.standard_normal(100000) * 10.0 ** g.integers(-6, 6, 100000)).astype(np.float32)
    # exact halfway cases: low 16 bits 0x8000, with even and odd kept parts
    u = (g.integers(0, 2**14, 1000).astype(np.uint32) << 16) | np.uint32(0x8000)
    x = np.concatenate([x, (u + np.uint32(0x3F800000 & 0xFF000000)).view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(wl.round_bf16(x), ref)


def test_trilinear_matches_torch_interpolate():
    g = np.random.default_rng(1)
    coarse = g.standard_normal((3,) + wl.VIDEO_COARSE)
    ref = F.interpolate(torch.from_numpy(coarse)[None], size=wl.VIDEO_GRID, mode="trilinear",
                        align_corners=False)[0].numpy()
    assert np.allclose(wl._trilinear_x4(coarse, wl.VIDEO_GRID), ref, atol=1e-12)


def test_inputs_are_seeded_and_head_separable():
    w = wl.WORKLOADS[2]
    a = wl.make_inputs(w, heads=[0, 5])
    b = wl.make_inputs(w, heads=[5])
    c = wl.make_inputs(w, heads=[0, 5])
    for x, y, z in zip(a, b, c):
        assert x.shape == (1, 2, 4096, 128) and x.dtype == np.float32
        assert np.array_equal(x, z)
        assert np.array_equal(x[:, 1:], y)
        assert np.array_equal(wl.round_bf16(x), x)          # bf16-exact values


def test_fp32_workload_stays_fp32():
    Q, K, V = wl.make_inputs(wl.WORKLOADS[1])
    assert Q.shape == (1, 1, 1024, 64)
    assert not np.array_equal(wl.round_bf16(K), K)


def test_block_mask_matches_hand_enumeration():
    """The section 4.2 rules on the section's own 1 text + 8 image block example."""
    mask = wl.block_mask_multimodal(1, 8, window=2, global_stride=4)
    assert np.array_equal(mask, _read_grid("multimodal_mask_1text_8image.txt"))
    assert int(mask.sum()) == 59


def test_fixed_mask_idx_counts():
    w = wl.WORKLOADS[5]
    idx = wl.idx_fixed_mask(w)
    assert idx.shape == (1, 24, 72, 72)
    lines = [ln for ln in open(os.path.join(GOLDEN, "multimodal_mask_counts_8text_64image.txt"))
             if ln[0] != "#"]
    counts = [int(x) for x in lines[0].split()]
    got = (idx[0, 0] >= 0).sum(axis=1)
    assert list(got) == counts and sum(counts) == 1522
    for row in idx[0, 0]:
        valid = row[row >= 0]
        assert np.all(np.diff(valid) > 0)                   # ascending, no duplicates
        assert np.all(row[len(valid):] == -1)               # padding only at the end
    assert np.array_equal(idx[0, 0], idx[0, 23])
