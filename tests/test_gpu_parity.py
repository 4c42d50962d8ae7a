"""GPU parity: libpisa's HIP kernels (through the C ABI) against the fp64 oracle.

Tolerances (GPU vs oracle):
* statistics: rel-L2 <= 1e-5 per tensor, max relative error of M <= 1e-5
  (spectral M_j: max relative error <= 1e-4, for blocks whose two largest
  singular values nearly coincide, where 24 Lanczos steps stop short);
* routing: same inputs on both sides (the GPU's fp32 centroids and M, upcast
  exactly); indices bit-exact except swaps among blocks whose oracle scores
  are within 1e-6;
* attention: same idx on both sides, each side with its own statistics;
  bf16 inputs rel-L2 <= 1e-2 and max-abs <= 2e-2, fp32 inputs both <= 1e-5.

The full-size video workloads are compared on sampled heads / query blocks
that the oracle computes one by one, with the kernel launched exactly as the
benchmark launches it.
"""

import math

import numpy as np
import pytest

import oracle
from _parity import (STATS_REL, check_attention, check_route, check_stats, oracle_stats, rel_l2,
                     to_dev, to_np)
from piecewise_block_sparse_amd import workloads as wl

pytestmark = pytest.mark.gpu

_CACHE = {}


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


def inputs(wid):
    if wid not in _CACHE:
        _CACHE.clear()                       # keep one workload resident at a time
        w = wl.WORKLOADS[wid]
        Q, K, V = wl.make_inputs(w)
        _CACHE[wid] = (w, Q, K, V, to_dev(Q, w.dtype), to_dev(K, w.dtype), to_dev(V, w.dtype))
    return _CACHE[wid]


SAMPLE_HEADS = {1: None, 2: None, 5: None, 3: [0, 7, 11], 4: [0, 21, 39]}


def sample_qblocks(w, heads, per_head=6, seed=0):
    g = np.random.default_rng(seed)
    nb = w.nb
    out = []
    for hi in range(len(heads)):
        picks = {0, nb - 1, nb // 2} | set(int(x) for x in g.choice(nb, per_head - 3, replace=False))
        out += [(0, hi, i) for i in sorted(picks)]
    return out


@pytest.mark.parametrize("wid", [1, 2, 5, 3, 4])
def test_precompute_parity(torch, wid):
    pisa = pisa_mod()
    w, Q, K, V, Qd, Kd, Vd = inputs(wid)
    heads = SAMPLE_HEADS[wid]
    st = pisa.precompute(Kd, Vd, w.block, store_H=wid in (1, 2))
    torch.cuda.synchronize()
    ref = oracle_stats(K, V, w.block, heads)
    check_stats(st, ref, heads, name=w.name)


@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_route_parity_shared_inputs(torch, wid):
    pisa = pisa_mod()
    w, Q, K, V, Qd, Kd, Vd = inputs(wid)
    heads = SAMPLE_HEADS[wid] or list(range(w.heads))
    st = pisa.precompute(Kd, Vd, w.block)
    idx = pisa.route(Qd, st, w.k, w.lam, w.block)
    torch.cuda.synchronize()
    scores = oracle.route_scores(Q[:, heads], to_np(st["centroid"])[:, heads],
                                 to_np(st["M"])[:, heads], w.lam, w.block, w.scale)
    ndiff = check_route(idx.cpu().numpy()[:, heads], scores, w.k, name=w.name)
    print(f"{w.name}: {ndiff} near-tie rows")


def _idx_for(pisa, w, Qd, st):
    if w.wid == 5:
        import torch
        return torch.from_numpy(wl.idx_fixed_mask(w)).cuda()
    return pisa.route(Qd, st, w.k, w.lam, w.block)


@pytest.mark.parametrize("mode", ["approx", "drop"])
@pytest.mark.parametrize("wid", [1, 2, 5, 3, 4])
def test_attention_parity(torch, wid, mode):
    pisa = pisa_mod()
    w, Q, K, V, Qd, Kd, Vd = inputs(wid)
    st = pisa.precompute(Kd, Vd, w.block)
    idx = _idx_for(pisa, w, Qd, st)
    out = pisa.attention(Qd, Kd, Vd, idx, st, w.block, mode=mode)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    heads = SAMPLE_HEADS[wid]
    m = oracle.MODE_APPROX if mode == "approx" else oracle.MODE_DROP
    if heads is None:
        ref_st = oracle.precompute(K, V, w.block)
        ref = oracle.attention(Q, K, V, idx_np, ref_st["centroid"], ref_st["vsum"], ref_st["Hbar"],
                               m, w.scale, w.block)
        got = to_np(out)
    else:
        Qs, Ks, Vs = Q[:, heads], K[:, heads], V[:, heads]
        ref_st = oracle.precompute(Ks, Vs, w.block)
        ref = oracle.attention(Qs, Ks, Vs, idx_np[:, heads], ref_st["centroid"], ref_st["vsum"],
                               ref_st["Hbar"], m, w.scale, w.block,
                               qblocks=sample_qblocks(w, heads))
        got = to_np(out)[:, heads]
    err, mab = check_attention(got, ref, w.dtype, name=f"{w.name}/{mode}")
    print(f"{w.name}/{mode}: rel-L2 {err:.3e} max-abs {mab:.3e}")


ORDER_MODES = {"zeroth": oracle.MODE_ZEROTH, "first": oracle.MODE_FIRST}


@pytest.mark.parametrize("mode", ["zeroth", "first"])
@pytest.mark.parametrize("wid", [1, 2, 5, 3, 4])
def test_attention_orders_parity(torch, wid, mode):
    """The zeroth-order and the per-block first-order treatments of the
    unselected blocks, against the oracle's expansions of the same order."""
    pisa = pisa_mod()
    w, Q, K, V, Qd, Kd, Vd = inputs(wid)
    bf = w.dtype == "bf16"
    st = pisa.precompute(Kd, Vd, w.block, store_H=(mode == "first" and not bf),
                         store_Ht=(mode == "first" and bf))
    idx = _idx_for(pisa, w, Qd, st)
    out = pisa.attention(Qd, Kd, Vd, idx, st, w.block, mode=mode)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    heads = SAMPLE_HEADS[wid] or list(range(w.heads))
    Qs, Ks, Vs = Q[:, heads], K[:, heads], V[:, heads]
    ref_st = oracle.precompute(Ks, Vs, w.block)
    qb = None if SAMPLE_HEADS[wid] is None else sample_qblocks(w, heads, per_head=4)
    ref = oracle.attention(Qs, Ks, Vs, idx_np[:, heads], ref_st["centroid"], ref_st["vsum"],
                           ref_st["Hbar"], ORDER_MODES[mode], w.scale, w.block, qblocks=qb,
                           H=ref_st["H"])
    err, mab = check_attention(to_np(out)[:, heads], ref, w.dtype, name=f"{w.name}/{mode}")
    print(f"{w.name}/{mode}: rel-L2 {err:.3e} max-abs {mab:.3e}")


def test_first_order_Ht_pack_is_H_transposed(torch):
    """The bf16 H_j^T pack equals the fp32 H_j transposed, rounded to bf16."""
    pisa = pisa_mod()
    w, Q, K, V, Qd, Kd, Vd = inputs(2)
    st = pisa.precompute(Kd, Vd, w.block, store_H=True, store_Ht=True)
    torch.cuda.synchronize()
    assert torch.equal(st["Ht"], st["H"].transpose(-1, -2).to(torch.bfloat16))


# ---------------------------------------------------------------- spectral M_j

SPECTRAL_MAX_REL = 1e-4    # Lanczos (24 steps) on blocks with a tiny top singular-value gap


@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_spectral_M_parity(torch, wid):
    """M_j = largest singular value of H_j - Hbar against the oracle's LAPACK SVD;
    every other statistic is the same as with the Frobenius reading."""
    pisa = pisa_mod()
    w, Q, K, V, Qd, Kd, Vd = inputs(wid)
    heads = SAMPLE_HEADS[wid] or list(range(w.heads))
    st = pisa.precompute(Kd, Vd, w.block, norm="spectral")
    fro = pisa.precompute(Kd, Vd, w.block)
    torch.cuda.synchronize()
    for key in ("centroid", "vsum", "Hbar"):
        assert torch.equal(st[key], fro[key])
    Ks, Vs = K[:, heads], V[:, heads]
    ref = oracle.precompute(Ks, Vs, w.block, norm="spectral")
    g = to_np(st["M"])[:, heads]
    err = rel_l2(g, ref["M"])
    mrel = float(np.max(np.abs(g - ref["M"]) / np.maximum(ref["M"], 1e-30)))
    print(f"{w.name}: spectral M rel-L2 {err:.3e}, max rel {mrel:.3e}")
    assert err <= STATS_REL and mrel <= SPECTRAL_MAX_REL
    assert np.all(g <= to_np(fro["M"])[:, heads] * (1 + 1e-5))


@pytest.mark.parametrize("dtype,d,B,nb", [("bf16", 64, 128, 9), ("bf16", 128, 64, 13),
                                          ("fp32", 128, 128, 5), ("fp32", 64, 64, 11)])
def test_spectral_M_small_shapes(torch, dtype, d, B, nb):
    """Spectral M_j on both head dims and block sizes, batch 2 with a second
    sequence that ends inside a block and leaves empty blocks (M = 0 there),
    against the oracle's SVD; one head whose H_j are rank one (within a block
    every value row is one vector times a power of two, exact in bf16), and one
    head with V = 0 (every H_j = Hbar = 0, so M = 0 exactly)."""
    pisa = pisa_mod()
    L = nb * B
    lens = [L, L - 3 * B - 5]
    K = _rand(torch, (2, 3, L, d), dtype, 81)
    V = _rand(torch, (2, 3, L, d), dtype, 82)
    c = np.random.default_rng(83).choice([-2.0, -1.0, -0.5, 0.5, 1.0, 2.0], size=(2, L, 1))
    V[:, 1] = (c * np.repeat(V[:, 1, ::B], B, axis=1)).astype(np.float32)   # rank-one H_j
    V[:, 2] = 0.0
    Kd, Vd = (to_dev(x, dtype) for x in (K, V))
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    st = pisa.precompute(Kd, Vd, B, norm="spectral", seq_lens=sl)
    torch.cuda.synchronize()
    ref = oracle.precompute(K, V, B, norm="spectral", seq_lens=lens)["M"]
    g = to_np(st["M"])
    assert np.all(g[:, 2] == 0.0)
    nne = (lens[1] + B - 1) // B
    assert np.all(g[1, :, nne:] == 0.0)
    live = ref > 1e-6 * ref.max()
    mrel = float(np.max(np.abs(g - ref)[live] / ref[live]))
    print(f"spectral {dtype}/d{d}/B{B}: max rel {mrel:.3e}")
    assert mrel <= SPECTRAL_MAX_REL
    assert np.all(np.abs(g - ref)[~live] <= 1e-6 * ref.max())


@pytest.mark.parametrize("wid", [2, 3])
def test_route_with_spectral_M(torch, wid):
    """Routing on the spectral M_j: bit-exact with the oracle's top-k of the same
    scores; prints how far the two readings of the norm change the routing."""
    pisa = pisa_mod()
    w, Q, K, V, Qd, Kd, Vd = inputs(wid)
    heads = SAMPLE_HEADS[wid] or list(range(w.heads))
    st = pisa.precompute(Kd, Vd, w.block, norm="spectral")
    idx = pisa.route(Qd, st, w.k, w.lam, w.block)
    idx_f = pisa.route(Qd, pisa.precompute(Kd, Vd, w.block), w.k, w.lam, w.block)
    torch.cuda.synchronize()
    scores = oracle.route_scores(Q[:, heads], to_np(st["centroid"])[:, heads],
                                 to_np(st["M"])[:, heads], w.lam, w.block, w.scale)
    check_route(idx.cpu().numpy()[:, heads], scores, w.k, name=f"{w.name}/spectral")
    a, b = idx.cpu().numpy(), idx_f.cpu().numpy()
    overlap = np.mean([len(np.intersect1d(x, y)) / w.k for x, y in
                       zip(a.reshape(-1, w.k), b.reshape(-1, w.k))])
    print(f"{w.name}: routing overlap spectral vs Frobenius M {overlap:.4f}")


def test_norm_reading_diagnostic(torch):
    """The two readings of ||.||_2 in the routing score, compared by PISA-vs-dense
    error on the image workload (both routed with their own M_j); reported."""
    pisa = pisa_mod()
    w, Q, K, V, Qd, Kd, Vd = inputs(2)
    nb = w.nb
    full = torch.arange(nb, dtype=torch.int32, device="cuda").expand(1, w.heads, nb, nb).contiguous()
    fro = pisa.precompute(Kd, Vd, w.block)
    dense = to_np(pisa.attention(Qd, Kd, Vd, full, fro, w.block, mode="drop"))
    res = {}
    for norm in ("fro", "spectral"):
        st = pisa.precompute(Kd, Vd, w.block, norm=norm)
        for lam in (0.0, w.lam, 1.0):
            idx = pisa.route(Qd, st, w.k, lam, w.block)
            out = to_np(pisa.attention(Qd, Kd, Vd, idx, st, w.block, mode="approx"))
            res[(norm, lam)] = rel_l2(out, dense)
    torch.cuda.synchronize()
    print("PISA vs dense rel-L2 (image workload): " +
          ", ".join(f"{n} lambda={l}: {e:.4f}" for (n, l), e in res.items()))
    assert res[("fro", 0.0)] == res[("spectral", 0.0)]


# ---------------------------------------------------------------- variable lengths

VL_MODES = {"approx": oracle.MODE_APPROX, "drop": oracle.MODE_DROP, **ORDER_MODES}


@pytest.mark.parametrize("dtype,d,B,L,k,lens", [
    ("bf16", 128, 64, 1024, 5, [1024, 1000, 321]),      # full, ragged last block, empty blocks
    ("bf16", 128, 128, 1024, 3, [1024, 700, 130]),
    ("bf16", 64, 64, 1024, 4, [999, 64, 1]),
    ("bf16", 64, 128, 1024, 2, [1024, 129, 0]),          # an empty sequence
    ("bf16", 128, 64, 1024, 4, [320, 1024, 577]),        # a live and an empty block share a pair
    ("bf16", 64, 64, 1344, 3, [1344, 700, 64]),          # odd block count
    ("fp32", 128, 64, 512, 3, [512, 300, 65]),
    ("fp32", 64, 128, 512, 2, [257, 128, 5]),
])
def test_varlen_pipeline_parity(torch, dtype, d, B, L, k, lens):
    """Each batch entry is a sequence of its own length inside a padded buffer:
    statistics, routing and every attention mode against the oracle's
    count-aware definitions; the padding holds NaN, which must not reach any
    result, and padding query rows must come out 0."""
    pisa = pisa_mod()
    b, h = len(lens), 2
    Q, K, V = (_rand(torch, (b, h, L, d), dtype, s) for s in (31, 32, 33))
    K = K + np.repeat(_rand(torch, (b, h, L // B, d), "fp32", 34) * 0.5, B, axis=2)
    if dtype == "bf16":
        K = wl.round_bf16(K)
    Qn, Kn, Vn = Q.copy(), K.copy(), V.copy()
    for bi, n in enumerate(lens):
        for X in (Qn, Kn, Vn):
            X[bi, :, n:] = np.nan
    Qd, Kd, Vd = (to_dev(x, dtype) for x in (Qn, Kn, Vn))
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    st = pisa.precompute(Kd, Vd, B, store_H=True, store_Ht=dtype == "bf16", seq_lens=sl)
    idx = pisa.route(Qd, st, k, 0.05, B, seq_lens=sl)
    outs = {m: pisa.attention(Qd, Kd, Vd, idx, st, B, mode=m, seq_lens=sl) for m in VL_MODES}
    torch.cuda.synchronize()
    ref_st = oracle.precompute(K, V, B, seq_lens=lens)
    check_stats(st, ref_st, name="varlen")
    scale = 1 / math.sqrt(d)
    scores = oracle.route_scores(Q, to_np(st["centroid"]), to_np(st["M"]), 0.05, B, scale,
                                 seq_lens=lens)
    check_route(idx.cpu().numpy(), scores, k, name="varlen")
    for m, code in VL_MODES.items():
        ref = oracle.attention(Q, K, V, idx.cpu().numpy(), ref_st["centroid"], ref_st["vsum"],
                               ref_st["Hbar"], code, scale, B, H=ref_st["H"], seq_lens=lens)
        got = to_np(outs[m])
        check_attention(got, ref, dtype, name=f"varlen/{m}")
        for bi, n in enumerate(lens):
            assert np.all(got[bi, :, n:] == 0.0), f"varlen/{m}: padding rows of entry {bi}"


@pytest.mark.parametrize("seed", range(12))
def test_random_small_configurations(torch, seed):
    """Seeded random small problems across the supported space: element type,
    head dim, block size, 1 to 24 blocks (one block, odd counts: query-block
    pairs with a missing second block), batch and heads, k, and with half the
    seeds variable lengths including empty and one-token sequences; the whole
    pipeline and every attention mode against the oracle."""
    pisa = pisa_mod()
    g = np.random.default_rng(7000 + seed)
    dtype = "fp32" if seed % 4 == 3 else "bf16"
    d, B = int(g.choice([64, 128])), int(g.choice([64, 128]))
    nb, b, h = int(g.integers(1, 25)), int(g.integers(1, 3)), int(g.integers(1, 4))
    k = int(g.integers(1, nb + 1))
    L = nb * B
    lens = None
    if seed % 2 == 1:
        lens = [int(x) for x in g.choice([0, 1, L, int(g.integers(1, L + 1))], size=b)]
    Q, K, V = (_rand(torch, (b, h, L, d), dtype, 100 * seed + s) for s in (1, 2, 3))
    K = K + np.repeat(_rand(torch, (b, h, nb, d), "fp32", 100 * seed + 4) * 0.5, B, axis=2)
    if dtype == "bf16":
        K = wl.round_bf16(K)
    Qn, Kn, Vn = Q.copy(), K.copy(), V.copy()
    if lens is not None:
        for bi, n in enumerate(lens):
            for X in (Qn, Kn, Vn):
                X[bi, :, n:] = np.nan
    Qd, Kd, Vd = (to_dev(x, dtype) for x in (Qn, Kn, Vn))
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    st = pisa.precompute(Kd, Vd, B, store_H=True, store_Ht=dtype == "bf16", seq_lens=sl)
    idx = pisa.route(Qd, st, k, 0.05, B, seq_lens=sl)
    outs = {m: pisa.attention(Qd, Kd, Vd, idx, st, B, mode=m, seq_lens=sl) for m in VL_MODES}
    torch.cuda.synchronize()
    name = f"random{seed}({dtype}, d={d}, B={B}, nb={nb}, b={b}, h={h}, k={k}, lens={lens})"
    ref_st = oracle.precompute(K, V, B, seq_lens=lens)
    check_stats(st, ref_st, name=name)
    scale = 1 / math.sqrt(d)
    scores = oracle.route_scores(Q, to_np(st["centroid"]), to_np(st["M"]), 0.05, B, scale,
                                 seq_lens=lens)
    check_route(idx.cpu().numpy(), scores, k, name=name)
    for m, code in VL_MODES.items():
        ref = oracle.attention(Q, K, V, idx.cpu().numpy(), ref_st["centroid"], ref_st["vsum"],
                               ref_st["Hbar"], code, scale, B, H=ref_st["H"], seq_lens=lens)
        got = to_np(outs[m])
        check_attention(got, ref, dtype, name=f"{name}/{m}")
        if lens is not None:
            for bi, n in enumerate(lens):
                assert np.all(got[bi, :, n:] == 0.0), f"{name}/{m}: padding rows of entry {bi}"


def test_varlen_full_lengths_match_the_plain_call(torch):
    """Lengths equal to the buffer length reproduce the call without lengths."""
    pisa = pisa_mod()
    w, Q, K, V, Qd, Kd, Vd = inputs(2)
    sl = torch.full((w.batch,), w.seq_len, dtype=torch.int32, device="cuda")
    st0 = pisa.precompute(Kd, Vd, w.block, store_Ht=True)
    st1 = pisa.precompute(Kd, Vd, w.block, store_Ht=True, seq_lens=sl)
    idx0 = pisa.route(Qd, st0, w.k, w.lam, w.block)
    idx1 = pisa.route(Qd, st1, w.k, w.lam, w.block, seq_lens=sl)
    torch.cuda.synchronize()
    for key in ("centroid", "vsum", "Hbar", "M", "packed", "Ht"):
        assert torch.equal(st0[key], st1[key]), key
    assert torch.equal(idx0, idx1)
    for m in VL_MODES:
        a = pisa.attention(Qd, Kd, Vd, idx0, st0, w.block, mode=m)
        b_ = pisa.attention(Qd, Kd, Vd, idx0, st0, w.block, mode=m, seq_lens=sl)
        torch.cuda.synchronize()
        assert torch.equal(a, b_), m


def test_varlen_image_workload_sampled(torch):
    """The image workload as a ragged sequence (4096 - 37 tokens), every mode,
    on sampled query blocks including the ragged one."""
    pisa = pisa_mod()
    w, Q, K, V, Qd, Kd, Vd = inputs(2)
    n = w.seq_len - 37
    sl = torch.tensor([n], dtype=torch.int32, device="cuda")
    st = pisa.precompute(Kd, Vd, w.block, store_Ht=True, seq_lens=sl)
    idx = pisa.route(Qd, st, w.k, w.lam, w.block, seq_lens=sl)
    outs = {m: to_np(pisa.attention(Qd, Kd, Vd, idx, st, w.block, mode=m, seq_lens=sl))
            for m in VL_MODES}
    torch.cuda.synchronize()
    heads = [0, 13]
    Qs, Ks, Vs = Q[:, heads], K[:, heads], V[:, heads]
    ref_st = oracle.precompute(Ks, Vs, w.block, seq_lens=[n])
    qb = [(0, hi, i) for hi in range(2) for i in (0, 17, w.nb - 2, w.nb - 1)]
    for m, code in VL_MODES.items():
        ref = oracle.attention(Qs, Ks, Vs, idx.cpu().numpy()[:, heads], ref_st["centroid"],
                               ref_st["vsum"], ref_st["Hbar"], code, w.scale, w.block, qblocks=qb,
                               H=ref_st["H"], seq_lens=[n])
        err, mab = check_attention(outs[m][:, heads], ref, w.dtype, name=f"varlen-image/{m}")
        print(f"varlen image {m}: rel-L2 {err:.3e} max-abs {mab:.3e}")


# ---------------------------------------------------------------- edge cases

def _rand(torch, shape, dtype, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal(shape).astype(np.float32)
    if dtype == "bf16":
        x = wl.round_bf16(x)
    return x


@pytest.mark.parametrize("dtype,d,B,L,k", [
    ("bf16", 64, 64, 1024, 3),
    ("bf16", 64, 128, 1024, 2),
    ("bf16", 128, 128, 384, 1),      # nb = 3: partial centroid tile
    ("bf16", 128, 64, 4608, 7),      # nb = 72: partial centroid tile
    ("fp32", 128, 128, 512, 2),
    ("fp32", 64, 64, 1024, 5),
])
def test_small_shapes_full_pipeline(torch, dtype, d, B, L, k):
    pisa = pisa_mod()
    h = 3
    Q, K, V = (_rand(torch, (1, h, L, d), dtype, s) for s in (1, 2, 3))
    K = K + np.repeat(_rand(torch, (1, h, L // B, d), "fp32", 4) * 0.5, B, axis=2)
    if dtype == "bf16":
        K = wl.round_bf16(K)
    Qd, Kd, Vd = (to_dev(x, dtype) for x in (Q, K, V))
    st = pisa.precompute(Kd, Vd, B, store_H=True, store_Ht=dtype == "bf16")
    idx = pisa.route(Qd, st, k, 0.05, B)
    modes = {"approx": oracle.MODE_APPROX, "drop": oracle.MODE_DROP, **ORDER_MODES}
    outs = {m: pisa.attention(Qd, Kd, Vd, idx, st, B, mode=m) for m in modes}
    torch.cuda.synchronize()
    ref_st = oracle.precompute(K, V, B)
    check_stats(st, ref_st, name="small")
    scale = 1 / math.sqrt(d)
    scores = oracle.route_scores(Q, to_np(st["centroid"]), to_np(st["M"]), 0.05, B, scale)
    check_route(idx.cpu().numpy(), scores, k, name="small")
    for m, code in modes.items():
        ref = oracle.attention(Q, K, V, idx.cpu().numpy(), ref_st["centroid"], ref_st["vsum"],
                               ref_st["Hbar"], code, scale, B, H=ref_st["H"])
        check_attention(to_np(outs[m]), ref, dtype, name=f"small/{m}")


def test_density_one_equals_dense(torch):
    """k = nb: both modes are dense softmax attention (checked against the oracle)."""
    pisa = pisa_mod()
    B, L, d = 64, 1024, 128
    Q, K, V = (_rand(torch, (1, 2, L, d), "bf16", s) for s in (5, 6, 7))
    Qd, Kd, Vd = (to_dev(x, "bf16") for x in (Q, K, V))
    st = pisa.precompute(Kd, Vd, B, store_Ht=True)
    nb = L // B
    idx = torch.arange(nb, dtype=torch.int32, device="cuda").expand(1, 2, nb, nb).contiguous()
    a = pisa.attention(Qd, Kd, Vd, idx, st, B, mode="approx")
    dr = pisa.attention(Qd, Kd, Vd, idx, st, B, mode="drop")
    others = [pisa.attention(Qd, Kd, Vd, idx, st, B, mode=m) for m in ("zeroth", "first")]
    torch.cuda.synchronize()
    ref_st = oracle.precompute(K, V, B)
    ref = oracle.attention(Q, K, V, idx.cpu().numpy(), ref_st["centroid"], ref_st["vsum"],
                           ref_st["Hbar"], oracle.MODE_DROP, 1 / math.sqrt(d), B)
    check_attention(to_np(a), ref, "bf16", "dense/approx")
    check_attention(to_np(dr), ref, "bf16", "dense/drop")
    assert torch.equal(a, dr)
    for o in others:
        assert torch.equal(o, dr)


def test_padding_empty_rows_and_out_of_range_ids(torch):
    """-1 anywhere in a row is skipped, ids >= nb are skipped, an empty row gives
    0 in keep-or-drop and the pure zeroth-order sum in PISA mode."""
    pisa = pisa_mod()
    B, L, d = 64, 512, 128
    nb = L // B
    Q, K, V = (_rand(torch, (1, 1, L, d), "bf16", s) for s in (8, 9, 10))
    Qd, Kd, Vd = (to_dev(x, "bf16") for x in (Q, K, V))
    rows = [[3, -1, 5, -1], [-1, -1, -1, -1], [-1, 0, -1, 7], [1, 2, 3, 4],
            [6, 99, -1, -1], [0, -1, -1, -1], [-1, -1, -1, 2], [5, 6, 7, -1]]
    idx = torch.tensor(rows, dtype=torch.int32).reshape(1, 1, nb, 4).cuda()
    st = pisa.precompute(Kd, Vd, B, store_Ht=True)
    modes = {"approx": oracle.MODE_APPROX, "drop": oracle.MODE_DROP, **ORDER_MODES}
    outs = {m: to_np(pisa.attention(Qd, Kd, Vd, idx, st, B, mode=m)) for m in modes}
    torch.cuda.synchronize()
    clean = np.array([([j for j in r if 0 <= j < nb] + [-1] * 4)[:4] for r in rows],
                     dtype=np.int32).reshape(1, 1, nb, 4)
    ref_st = oracle.precompute(K, V, B)
    for m, code in modes.items():
        ref = oracle.attention(Q, K, V, clean, ref_st["centroid"], ref_st["vsum"], ref_st["Hbar"],
                               code, 1 / math.sqrt(d), B, H=ref_st["H"])
        check_attention(outs[m], ref, "bf16", f"padding/{m}")
    assert np.all(outs["drop"][0, 0, B:2 * B] == 0.0)


@pytest.mark.parametrize("d,L,k", [(128, 64 * 21, 6), (64, 64 * 21, 5), (128, 64 * 40, 9)])
def test_query_block_pairs_with_unrelated_rows(torch, d, L, k):
    """With 64-token blocks two neighbouring query blocks share a workgroup and
    stream the union of their routed blocks; here every row routes its own
    random set (with -1 padding in some rows and one empty row), so most
    blocks of the union belong to one query block only.  Odd block counts leave
    the last pair with a single query block."""
    pisa = pisa_mod()
    B, h = 64, 2
    nb = L // B
    Q, K, V = (_rand(torch, (1, h, L, d), "bf16", s) for s in (41, 42, 43))
    g = np.random.default_rng(nb * 1000 + k)
    rows = np.full((1, h, nb, k), -1, dtype=np.int32)
    for hh in range(h):
        for i in range(nb):
            n = 0 if (hh, i) == (1, 3) else (k if i % 5 else k - 2)
            rows[0, hh, i, :n] = np.sort(g.choice(nb, size=n, replace=False))
    idx = torch.from_numpy(rows).cuda()
    st = pisa.precompute(Kd := to_dev(K, "bf16"), Vd := to_dev(V, "bf16"), B, store_Ht=True)
    Qd = to_dev(Q, "bf16")
    modes = {"approx": oracle.MODE_APPROX, "drop": oracle.MODE_DROP, **ORDER_MODES}
    outs = {m: to_np(pisa.attention(Qd, Kd, Vd, idx, st, B, mode=m)) for m in modes}
    torch.cuda.synchronize()
    ref_st = oracle.precompute(K, V, B)
    for m, code in modes.items():
        ref = oracle.attention(Q, K, V, rows, ref_st["centroid"], ref_st["vsum"], ref_st["Hbar"],
                               code, 1 / math.sqrt(d), B, H=ref_st["H"])
        check_attention(outs[m], ref, "bf16", f"pairs/{m}")
    assert np.all(outs["drop"][0, 1, 3 * B:4 * B] == 0.0)


def test_runs_are_bitwise_reproducible(torch):
    pisa = pisa_mod()
    w, Q, K, V, Qd, Kd, Vd = inputs(2)
    res = []
    for _ in range(2):
        st = pisa.precompute(Kd, Vd, w.block, store_H=True)
        idx = pisa.route(Qd, st, w.k, w.lam, w.block)
        out = pisa.attention(Qd, Kd, Vd, idx, st, w.block, mode="approx")
        torch.cuda.synchronize()
        res.append([st[n].clone() for n in ("centroid", "vsum", "H", "Hbar", "M")] + [idx, out])
    for a, b in zip(*res):
        assert torch.equal(a, b)


@pytest.mark.parametrize("wid", [2, 4])
def test_step_replays_in_a_captured_graph(torch, wid):
    """The library's calls only enqueue kernels on the caller's stream (no host
    synchronisation, allocation or memset inside it; the binding's output
    tensors come from torch's graph pool), so a whole step can be captured in a
    HIP graph.  Every replay, with eager steps in between, equals the eager step
    bit for bit."""
    pisa = pisa_mod()
    w, Q, K, V, Qd, Kd, Vd = inputs(wid)
    ws = torch.empty(pisa.workspace_size(Kd, w.block), dtype=torch.uint8, device="cuda")

    def step():
        st = pisa.precompute(Kd, Vd, w.block, workspace=ws)
        idx = pisa.route(Qd, st, w.k, w.lam, w.block)
        return idx, pisa.attention(Qd, Kd, Vd, idx, st, w.block, mode="approx")

    ref_idx, ref = step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        g_idx, g_out = step()
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(g_idx, ref_idx)
        assert torch.equal(g_out, ref)
        step()                                # eager work between replays
        torch.cuda.synchronize()


def test_end_to_end_routing_diagnostic(torch):
    """Each side routes with its own statistics; reported, not gated (fp32 vs
    fp64 M differs by ~1e-7 relative, which can flip near-ties)."""
    pisa = pisa_mod()
    w, Q, K, V, Qd, Kd, Vd = inputs(2)
    st = pisa.precompute(Kd, Vd, w.block)
    idx = pisa.route(Qd, st, w.k, w.lam, w.block).cpu().numpy()
    ref_st = oracle.precompute(K, V, w.block)
    ref = oracle.route(Q, ref_st["centroid"], ref_st["M"], w.k, w.lam, w.block, w.scale)
    agree = float(np.mean(np.all(idx == ref, axis=-1)))
    print(f"{w.name}: {agree:.4f} of rows identical with independent statistics")
    assert agree > 0.9


def test_route_max_blocks(torch):
    """nb = 2048 (the largest supported block count): routing still matches."""
    pisa = pisa_mod()
    B, L, d, k = 64, 2048 * 64, 128, 200
    Q, K, V = (_rand(torch, (1, 1, L, d), "bf16", s) for s in (11, 12, 13))
    Qd, Kd, Vd = (to_dev(x, "bf16") for x in (Q, K, V))
    st = pisa.precompute(Kd, Vd, B)
    idx = pisa.route(Qd, st, k, 0.02, B)
    torch.cuda.synchronize()
    scores = oracle.route_scores(Q, to_np(st["centroid"]), to_np(st["M"]), 0.02, B, 1 / math.sqrt(d))
    check_route(idx.cpu().numpy(), scores, k, name="nb2048")


@pytest.mark.parametrize("dtype,d,nb", [("bf16", 128, 255), ("bf16", 128, 256), ("bf16", 64, 257),
                                        ("bf16", 128, 300), ("fp32", 128, 300), ("fp32", 64, 255)])
def test_route_block_counts_around_the_row_split(torch, dtype, d, nb):
    """Block counts on both sides of the route kernel's switch from four to
    eight query blocks per workgroup (256), counts that are not a multiple of
    the 16-block score tiles, both input types and head dims, batch 2 with
    one shorter sequence: routing against the oracle's scores."""
    pisa = pisa_mod()
    B, k = 64, 23
    L = nb * B
    lens = [L, L - 5 * B - 17]
    Q, K, V = (_rand(torch, (2, 2, L, d), dtype, s) for s in (71, 72, 73))
    K = K + np.repeat(_rand(torch, (2, 2, nb, d), "fp32", 74) * 0.5, B, axis=2)
    if dtype == "bf16":
        K = wl.round_bf16(K)
    Qd, Kd, Vd = (to_dev(x, dtype) for x in (Q, K, V))
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    st = pisa.precompute(Kd, Vd, B, seq_lens=sl)
    idx = pisa.route(Qd, st, k, 0.05, B, seq_lens=sl)
    torch.cuda.synchronize()
    scores = oracle.route_scores(Q, to_np(st["centroid"]), to_np(st["M"]), 0.05, B, 1 / math.sqrt(d),
                                 seq_lens=lens)
    check_route(idx.cpu().numpy(), scores, k, name=f"route/{dtype}/d{d}/nb{nb}")


@pytest.mark.parametrize("B", [64, 128])
def test_attention_max_blocks_all_modes(torch, B):
    """nb = 2048 (the largest supported block count) with a large k: the
    statistics, and every mode against the oracle on sampled query blocks
    (first, middle, last), for both block sizes' kernels."""
    pisa = pisa_mod()
    L, d, k = 2048 * B, 128, 300
    Q, K, V = (_rand(torch, (1, 1, L, d), "bf16", s) for s in (14, 15, 16))
    K = wl.round_bf16(K + np.repeat(_rand(torch, (1, 1, L // B, d), "fp32", 17) * 0.5, B, axis=2))
    Qd, Kd, Vd = (to_dev(x, "bf16") for x in (Q, K, V))
    st = pisa.precompute(Kd, Vd, B, store_Ht=True)
    idx = pisa.route(Qd, st, k, 0.02, B)
    outs = {m: to_np(pisa.attention(Qd, Kd, Vd, idx, st, B, mode=m)) for m in VL_MODES}
    torch.cuda.synchronize()
    ref_st = oracle.precompute(K, V, B)
    check_stats(st, ref_st, name=f"nb2048/B{B}")
    qb = [(0, 0, i) for i in (0, 1024, 2047)]
    for m, code in VL_MODES.items():
        ref = oracle.attention(Q, K, V, idx.cpu().numpy(), ref_st["centroid"], ref_st["vsum"],
                               ref_st["Hbar"], code, 1 / math.sqrt(d), B, qblocks=qb, H=ref_st["H"])
        err, mab = check_attention(outs[m], ref, "bf16", name=f"nb2048/B{B}/{m}")
        print(f"nb2048 B{B} {m}: rel-L2 {err:.3e} max-abs {mab:.3e}")


@pytest.mark.parametrize("wid", [2, 5])
def test_packed_and_fp32_statistics_paths_agree(torch, wid):
    """PISA mode reads the bf16 statistics pack when present and converts the
    fp32 statistics itself otherwise; both feed identical bf16 operands."""
    pisa = pisa_mod()
    w, Q, K, V, Qd, Kd, Vd = inputs(wid)
    st = pisa.precompute(Kd, Vd, w.block)
    assert st["packed"] is not None
    idx = _idx_for(pisa, w, Qd, st)
    a = pisa.attention(Qd, Kd, Vd, idx, st, w.block, mode="approx")
    b = pisa.attention(Qd, Kd, Vd, idx, dict(st, packed=None), w.block, mode="approx")
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("nb,k", [(16, 5), (72, 30), (512, 64), (2048, 700)])
def test_route_exact_ties_go_to_lower_ids(torch, nb, k):
    """Zero queries make every score lambda * M_j; M with many repeated values
    (and +-0) forces exact ties at the k-th score, which the oracle breaks
    towards the lower block id."""
    pisa = pisa_mod()
    B, d = 64, 128
    g = np.random.default_rng(nb)
    Q = np.zeros((1, 2, nb * B, d), dtype=np.float32)
    M = g.integers(-2, 3, (1, 2, nb)).astype(np.float32)
    M[0, 1, ::3] = -0.0
    cen = np.zeros((1, 2, nb, d), dtype=np.float32)
    st = {"centroid": torch.from_numpy(cen).cuda(), "M": torch.from_numpy(M).cuda()}
    idx = pisa.route(to_dev(Q, "bf16"), st, k, 1.0, B)
    ref = oracle.route(Q, cen, M, k, 1.0, B, 1 / math.sqrt(d))
    assert np.array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("dtype,d,B", [("bf16", 128, 64), ("bf16", 128, 128), ("bf16", 64, 128),
                                       ("fp32", 128, 64)])
def test_duplicate_ids_count_once(torch, dtype, d, B):
    """S_i is a set: an id repeated in an idx row (in any order) gives the
    result of the row without the repeat, bit for bit, on every path (64-token
    pairs, 128-token blocks, fp32), and matches the oracle on the clean rows."""
    pisa = pisa_mod()
    nb = 10
    L = nb * B
    Q, K, V = (_rand(torch, (1, 2, L, d), dtype, s) for s in (61, 62, 63))
    Qd, Kd, Vd = (to_dev(x, dtype) for x in (Q, K, V))
    g = np.random.default_rng(64)
    clean = np.full((1, 2, nb, 6), -1, dtype=np.int32)
    dup = np.full((1, 2, nb, 6), -1, dtype=np.int32)
    for hi in range(2):
        for i in range(nb):
            n = int(g.integers(1, 5))
            ids = np.sort(g.choice(nb, n, replace=False))
            clean[0, hi, i, :n] = ids
            row = np.concatenate([ids, ids[:1], ids[-1:]])[::-1]       # repeats, descending
            dup[0, hi, i, :len(row)] = row
    st = pisa.precompute(Kd, Vd, B, store_H=True)
    ref_st = oracle.precompute(K, V, B)
    scale = 1 / math.sqrt(d)
    for m, code in (("approx", oracle.MODE_APPROX), ("drop", oracle.MODE_DROP)):
        a = pisa.attention(Qd, Kd, Vd, torch.from_numpy(dup).cuda(), st, B, mode=m)
        b = pisa.attention(Qd, Kd, Vd, torch.from_numpy(clean).cuda(), st, B, mode=m)
        torch.cuda.synchronize()
        assert torch.equal(a, b), (dtype, d, B, m)
        ref = oracle.attention(Q, K, V, clean, ref_st["centroid"], ref_st["vsum"], ref_st["Hbar"],
                               code, scale, B)
        check_attention(to_np(a), ref, dtype, name=f"duplicates/{dtype}/{B}/{m}")
