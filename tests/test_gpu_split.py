"""GPU parity of pisa_attention_split (long exact lists split over several
workgroups, partial softmax states merged by a second kernel) against the
fp64 oracle, and against pisa_attention on the same inputs.

Tolerances as in the other attention parity tests (bf16: rel-L2 <= 1e-2,
max-abs <= 2e-2 against the oracle).  Against pisa_attention the split call
differs only in the order of the floating-point sums: where nothing splits it
must be the same bits, elsewhere within 2 bf16 ulps of the output scale.
"""

import math

import numpy as np
import pytest

import oracle
from _parity import check_attention, to_dev, to_np
from piecewise_block_sparse_amd import workloads as wl

pytestmark = pytest.mark.gpu

MODES = {"approx": oracle.MODE_APPROX, "drop": oracle.MODE_DROP, "zeroth": oracle.MODE_ZEROTH}


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a visible MI355X"
    import piecewise_block_sparse_amd as pisa
    pisa._lib.load()
    return t


def _rand(shape, seed, bf16=True):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    return wl.round_bf16(x) if bf16 else x


def _close_to_unsplit(got, ref, name):
    # same terms, other summation order: within a few bf16 ulps of the values
    err = float(np.abs(got - ref).max())
    scale = float(np.abs(ref).max()) + 1e-30
    assert err <= 2.0 ** -7 * scale, f"{name}: split vs unsplit max-abs {err:.3e} (scale {scale:.3e})"


@pytest.mark.parametrize("cap", [24, 8])
def test_split_multimodal_fixed_mask(torch, cap):
    """The multimodal workload with its fixed text/image mask (text rows: all
    72 blocks, image rows: 12 to 15): text work items split into 3 or 9 parts;
    sampled heads against the oracle in every mode."""
    import piecewise_block_sparse_amd as pisa
    w = wl.WORKLOADS[5]
    Q, K, V = wl.make_inputs(w)
    Qd, Kd, Vd = (to_dev(x, "bf16") for x in (Q, K, V))
    idx_h = wl.idx_fixed_mask(w)
    idx = torch.from_numpy(idx_h).to("cuda")
    st = pisa.precompute(Kd, Vd, w.block)
    heads = [0, 13, 23]
    ref_st = oracle.precompute(K[:, heads], V[:, heads], w.block)
    for m, code in MODES.items():
        print(f"split multimodal cap={cap} mode={m}", flush=True)
        got = pisa.attention(Qd, Kd, Vd, idx, st, w.block, mode=m, split_blocks=cap)
        plain = pisa.attention(Qd, Kd, Vd, idx, st, w.block, mode=m)
        torch.cuda.synchronize()
        g = to_np(got)
        _close_to_unsplit(g, to_np(plain), f"multimodal/{m}/cap{cap}")
        ref = oracle.attention(Q[:, heads], K[:, heads], V[:, heads], idx_h[:, heads],
                               ref_st["centroid"], ref_st["vsum"], ref_st["Hbar"], code, w.scale,
                               w.block)
        check_attention(g[:, heads], ref, "bf16", name=f"multimodal/{m}/cap{cap}")


@pytest.mark.parametrize("d,B,L,k", [(128, 64, 64 * 21, 6), (128, 128, 128 * 12, 5), (64, 64, 64 * 16, 7)])
def test_split_without_any_split_is_pisa_attention(torch, d, B, L, k):
    """max_blocks at or above every list: one part per item, the same bits."""
    import piecewise_block_sparse_amd as pisa
    Q, K, V = (_rand((1, 2, L, d), s) for s in (41, 42, 43))
    Qd, Kd, Vd = (to_dev(x, "bf16") for x in (Q, K, V))
    st = pisa.precompute(Kd, Vd, B)
    idx = pisa.route(Qd, st, k, 0.05, B)
    for m in MODES:
        a = pisa.attention(Qd, Kd, Vd, idx, st, B, mode=m, split_blocks=2 * k)
        b = pisa.attention(Qd, Kd, Vd, idx, st, B, mode=m)
        torch.cuda.synchronize()
        assert torch.equal(a, b), (m, d, B, L, k)


@pytest.mark.parametrize("seed", range(8))
def test_split_random_small(torch, seed):
    """Seeded random small problems: head dim, block size, odd block counts
    (pairs with a missing second block), variable lengths with NaN padding,
    rows with -1 padding and empty rows, every mode, and max_blocks from 1
    (every block its own part) up; against the oracle and the unsplit call."""
    import piecewise_block_sparse_amd as pisa
    g = np.random.default_rng(1000 + seed)
    d = int(g.choice([64, 128]))
    B = int(g.choice([64, 128]))
    nb = int(g.integers(1, 19))
    L = nb * B
    b, h = int(g.integers(1, 3)), int(g.integers(1, 3))
    kmax = int(g.integers(1, nb + 1))
    cap = int(g.integers(1, max(2, kmax)))
    varlen = bool(seed % 2)
    lens = [int(g.integers(1, L + 1)) for _ in range(b)] if varlen else None
    print(f"split random seed={seed}: d={d} B={B} nb={nb} b={b} h={h} kmax={kmax} cap={cap} lens={lens}",
          flush=True)
    Q, K, V = (_rand((b, h, L, d), 50 + 3 * seed + s) for s in range(3))
    idx_h = np.full((b, h, nb, kmax), -1, dtype=np.int32)
    for bi in range(b):
        for hi in range(h):
            for i in range(nb):
                n = int(g.integers(0, kmax + 1))             # 0: an empty row
                idx_h[bi, hi, i, :n] = np.sort(g.choice(nb, n, replace=False))
    Qn, Kn, Vn = Q.copy(), K.copy(), V.copy()
    if lens is not None:
        for bi, n in enumerate(lens):
            for X in (Qn, Kn, Vn):
                X[bi, :, n:] = np.nan
        # ids of empty blocks are skipped by both sides: keep the rows as drawn
    Qd, Kd, Vd = (to_dev(x, "bf16") for x in (Qn, Kn, Vn))
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda") if lens is not None else None
    st = pisa.precompute(Kd, Vd, B, seq_lens=sl)
    idx = torch.from_numpy(idx_h).to("cuda")
    ref_st = oracle.precompute(K, V, B, seq_lens=lens)
    scale = 1 / math.sqrt(d)
    for m, code in MODES.items():
        got = pisa.attention(Qd, Kd, Vd, idx, st, B, mode=m, seq_lens=sl, split_blocks=cap)
        plain = pisa.attention(Qd, Kd, Vd, idx, st, B, mode=m, seq_lens=sl)
        torch.cuda.synchronize()
        gn = to_np(got)
        _close_to_unsplit(gn, to_np(plain), f"random{seed}/{m}")
        ref = oracle.attention(Q, K, V, idx_h, ref_st["centroid"], ref_st["vsum"], ref_st["Hbar"],
                               code, scale, B, seq_lens=lens)
        check_attention(gn, ref, "bf16", name=f"random{seed}/{m}")
        if lens is not None:
            for bi, n in enumerate(lens):
                assert np.all(gn[bi, :, n:] == 0.0), f"random{seed}/{m}: padding rows"
