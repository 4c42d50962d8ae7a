"""GPU parity of the in-kernel routing (pisa_route_attention) through the C ABI.

The fused call must select exactly what pisa_route selects (bit for bit) and
then produce exactly what pisa_attention produces on that selection (bit for
bit: the same kernel body runs on the same list).  Both halves are also
checked against the fp64 oracle, with the tolerances of the other GPU parity
tests: routing indices bit-exact except swaps among oracle near-ties (1e-6),
attention rel-L2 <= 1e-2 and max-abs <= 2e-2 for bf16 inputs.
"""

import math

import numpy as np
import pytest

import oracle
from _parity import check_attention, check_route, to_dev, to_np
from piecewise_block_sparse_amd import workloads as wl

pytestmark = pytest.mark.gpu

MODES = {"approx": oracle.MODE_APPROX, "drop": oracle.MODE_DROP, "zeroth": oracle.MODE_ZEROTH}


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a visible MI355X"
    import piecewise_block_sparse_amd as pisa
    pisa._lib.load()        # fails loudly if libpisa.so is missing
    return t


def pisa_mod():
    import piecewise_block_sparse_amd as pisa
    return pisa


def _rand(shape, dtype, seed):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    return wl.round_bf16(x) if dtype == "bf16" else x


FORMS = ("in_kernel", "auto", "two_launch")


def _fused_vs_split(torch, pisa, Qd, Kd, Vd, st, k, lam, B, sl=None, modes=MODES, name=""):
    """Fused and split paths on the same tensors: identical idx and outputs,
    in every form of the fused call (in-kernel routing forced, the automatic
    choice, and the two-launch form)."""
    idx = pisa.route(Qd, st, k, lam, B, seq_lens=sl)
    outs = {}
    for m in modes:
        ref = pisa.attention(Qd, Kd, Vd, idx, st, B, mode=m, seq_lens=sl)
        for form in FORMS:
            got, gidx = pisa.route_attention(Qd, Kd, Vd, st, k, lam, B, mode=m, seq_lens=sl,
                                             return_idx=True, form=form)
            torch.cuda.synchronize()
            assert torch.equal(gidx, idx), f"{name}/{m}/{form}: selection differs from pisa_route"
            assert torch.equal(got, ref), f"{name}/{m}/{form}: output differs from route + attention"
        # without idx the in-kernel form writes no selection
        got = pisa.route_attention(Qd, Kd, Vd, st, k, lam, B, mode=m, seq_lens=sl, form="in_kernel")
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"{name}/{m}: output without idx differs from route + attention"
        outs[m] = got
    return idx, outs


@pytest.mark.parametrize("wid", [2, 3, 4])
def test_workloads_fused_equals_route_then_attention(torch, wid):
    """The image and both video workloads at full size, in the launch
    configuration the benchmark times; PISA, keep-or-drop and zeroth order."""
    pisa = pisa_mod()
    w = wl.WORKLOADS[wid]
    Q, K, V = wl.make_inputs(w)
    Qd, Kd, Vd = (to_dev(x, w.dtype) for x in (Q, K, V))
    st = pisa.precompute(Kd, Vd, w.block)
    idx, outs = _fused_vs_split(torch, pisa, Qd, Kd, Vd, st, w.k, w.lam, w.block, name=w.name)
    if wid == 2:
        # the whole image workload against the oracle as well
        d = w.head_dim
        scores = oracle.route_scores(Q, to_np(st["centroid"]), to_np(st["M"]), w.lam, w.block,
                                     1 / math.sqrt(d))
        check_route(idx.cpu().numpy(), scores, w.k, name=w.name)
        ref_st = oracle.precompute(K, V, w.block)
        for m, code in MODES.items():
            ref = oracle.attention(Q, K, V, idx.cpu().numpy(), ref_st["centroid"], ref_st["vsum"],
                                   ref_st["Hbar"], code, 1 / math.sqrt(d), w.block)
            check_attention(to_np(outs[m]), ref, "bf16", name=f"{w.name}/{m}")


@pytest.mark.parametrize("seed", range(10))
def test_random_small_configurations(torch, seed):
    """Seeded random bf16 problems over the supported space (head dim, block
    size, 1 to 24 blocks including odd counts for query-block pairs, batch,
    heads, k, variable lengths with empty and one-token sequences), against
    the split path bit for bit and against the oracle."""
    pisa = pisa_mod()
    g = np.random.default_rng(9100 + seed)
    d, B = int(g.choice([64, 128])), int(g.choice([64, 128]))
    nb, b, h = int(g.integers(1, 25)), int(g.integers(1, 3)), int(g.integers(1, 4))
    k = int(g.integers(1, nb + 1))
    L = nb * B
    lens = None
    if seed % 2 == 1:
        lens = [int(x) for x in g.choice([0, 1, L, int(g.integers(1, L + 1))], size=b)]
    Q, K, V = (_rand((b, h, L, d), "bf16", 100 * seed + s) for s in (1, 2, 3))
    K = wl.round_bf16(K + np.repeat(_rand((b, h, nb, d), "fp32", 100 * seed + 4) * 0.5, B, axis=2))
    Qn, Kn, Vn = Q.copy(), K.copy(), V.copy()
    if lens is not None:
        for bi, n in enumerate(lens):
            for X in (Qn, Kn, Vn):
                X[bi, :, n:] = np.nan
    Qd, Kd, Vd = (to_dev(x, "bf16") for x in (Qn, Kn, Vn))
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    st = pisa.precompute(Kd, Vd, B, seq_lens=sl)
    name = f"fused{seed}(d={d}, B={B}, nb={nb}, b={b}, h={h}, k={k}, lens={lens})"
    idx, outs = _fused_vs_split(torch, pisa, Qd, Kd, Vd, st, k, 0.05, B, sl=sl, name=name)
    scale = 1 / math.sqrt(d)
    scores = oracle.route_scores(Q, to_np(st["centroid"]), to_np(st["M"]), 0.05, B, scale,
                                 seq_lens=lens)
    check_route(idx.cpu().numpy(), scores, k, name=name)
    ref_st = oracle.precompute(K, V, B, seq_lens=lens)
    for m, code in MODES.items():
        ref = oracle.attention(Q, K, V, idx.cpu().numpy(), ref_st["centroid"], ref_st["vsum"],
                               ref_st["Hbar"], code, scale, B, seq_lens=lens)
        check_attention(to_np(outs[m]), ref, "bf16", name=f"{name}/{m}")


@pytest.mark.parametrize("d,B,nb,k", [(128, 64, 1920, 200), (64, 64, 960, 100),
                                      (128, 128, 2048, 300), (64, 128, 2048, 64)])
def test_largest_block_counts(torch, d, B, nb, k):
    """The largest nb each configuration's LDS holds (score rows of 1920 and
    960 blocks for query-block pairs, 2048 otherwise): same selection and
    outputs as the split path.  One block more is refused on the host for
    in-kernel routing, and the automatic form runs it as two launches."""
    pisa = pisa_mod()
    L = nb * B
    Q, K, V = (_rand((1, 1, L, d), "bf16", s) for s in (21, 22, 23))
    Qd, Kd, Vd = (to_dev(x, "bf16") for x in (Q, K, V))
    st = pisa.precompute(Kd, Vd, B)
    _fused_vs_split(torch, pisa, Qd, Kd, Vd, st, k, 0.02, B, modes=("approx",),
                    name=f"d{d}/B{B}/nb{nb}")
    if nb < 2048:
        Qx = torch.zeros((1, 1, L + B, d), dtype=torch.bfloat16, device="cuda")
        stx = pisa.precompute(Qx, Qx, B)
        with pytest.raises(pisa._lib.PisaError):
            pisa.route_attention(Qx, Qx, Qx, stx, k, 0.02, B, form="in_kernel")
        got, gidx = pisa.route_attention(Qx, Qx, Qx, stx, k, 0.02, B, return_idx=True)
        idx = pisa.route(Qx, stx, k, 0.02, B)
        ref = pisa.attention(Qx, Qx, Qx, idx, stx, B)
        torch.cuda.synchronize()
        assert torch.equal(gidx, idx) and torch.equal(got, ref)


@pytest.mark.parametrize("form", ["in_kernel", "two_launch"])
@pytest.mark.parametrize("nb,k", [(16, 5), (72, 30), (512, 64)])
def test_exact_ties_go_to_lower_ids(torch, nb, k, form):
    """Zero queries make every score lambda * M_j; repeated M values (and
    +-0) force exact ties at the k-th score: the in-kernel selection breaks
    them towards the lower block id, as the oracle does."""
    pisa = pisa_mod()
    B, d = 64, 128
    g = np.random.default_rng(nb)
    Q = np.zeros((1, 2, nb * B, d), dtype=np.float32)
    M = g.integers(-2, 3, (1, 2, nb)).astype(np.float32)
    M[0, 1, ::3] = -0.0
    cen = np.zeros((1, 2, nb, d), dtype=np.float32)
    Qd = to_dev(Q, "bf16")
    st = {"centroid": torch.from_numpy(cen).cuda(), "M": torch.from_numpy(M).cuda()}
    _, idx = pisa.route_attention(Qd, Qd, Qd, st, k, 1.0, B, mode="drop", return_idx=True,
                                  form=form)
    torch.cuda.synchronize()
    ref = oracle.route(Q, cen, M, k, 1.0, B, 1 / math.sqrt(d))
    assert np.array_equal(idx.cpu().numpy(), ref)


def test_fp32_and_first_order_are_refused(torch):
    pisa = pisa_mod()
    X = torch.zeros((1, 1, 256, 64), dtype=torch.float32, device="cuda")
    st = pisa.precompute(X, X, 64)
    with pytest.raises(pisa._lib.PisaError):
        pisa.route_attention(X, X, X, st, 2, 0.1, 64)
    Xb = X.to(torch.bfloat16)
    stb = pisa.precompute(Xb, Xb, 64)
    with pytest.raises(pisa._lib.PisaError):
        pisa.route_attention(Xb, Xb, Xb, stb, 2, 0.1, 64, mode="first")


@pytest.mark.parametrize("wid", [2, 5])
def test_without_the_statistics_pack(torch, wid):
    """Without the bf16 pack the kernel converts the fp32 statistics itself,
    staging them in the ring that the routing prologue used first: same
    selection and outputs as the split path without the pack."""
    pisa = pisa_mod()
    w = wl.WORKLOADS[wid]
    Q, K, V = wl.make_inputs(w)
    Qd, Kd, Vd = (to_dev(x, w.dtype) for x in (Q, K, V))
    st = dict(pisa.precompute(Kd, Vd, w.block), packed=None)
    k = w.k if w.k > 0 else 8
    _fused_vs_split(torch, pisa, Qd, Kd, Vd, st, k, 0.1, w.block, name=f"{w.name}/no-pack")
