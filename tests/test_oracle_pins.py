"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

Nothing here compares the oracle with itself: each check uses a library routine
(torch SDPA in fp64, numpy norms, a plain sort), a closed form worked out by
hand, an invariant, or a brute-force token-level loop written from the
definitions (PISA page, section 2 "Core algorithm" and "Covariance-aware
routing"; block-sparse notes, section 3.3).
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import MODE_APPROX, MODE_DROP, MODE_FIRST, MODE_ZEROTH, attention, precompute, route

RTOL = 1e-12


def sdpa(Q, K, V, scale, mask=None):
    """Library dense softmax attention in fp64 (torch on the CPU)."""
    q, k, v = (torch.from_numpy(np.asarray(x, dtype=np.float64)) for x in (Q, K, V))
    m = None if mask is None else torch.from_numpy(mask)
    return F.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale).numpy()


def rand_qkv(seed, b=1, h=2, L=256, d=16, kscale=1.0):
    g = np.random.default_rng(seed)
    Q = g.standard_normal((b, h, L, d))
    K = kscale * g.standard_normal((b, h, L, d))
    V = g.standard_normal((b, h, L, d))
    return Q, K, V


def rand_idx(seed, b, h, nqb, nb, k):
    g = np.random.default_rng(seed)
    idx = np.empty((b, h, nqb, k), dtype=np.int32)
    for bi in range(b):
        for hi in range(h):
            for i in range(nqb):
                idx[bi, hi, i] = np.sort(g.choice(nb, size=k, replace=False))
    return idx


def run(Q, K, V, idx, B, mode, scale, st=None):
    st = precompute(K, V, B) if st is None else st
    return attention(Q, K, V, idx, st["centroid"], st["vsum"], st["Hbar"], mode, scale, B, H=st["H"])


def block_mask(idx, B, L):
    """Token-level boolean mask [b,h,L,L] (True = attend) from block lists."""
    b, h, nqb, _ = idx.shape
    m = np.zeros((b, h, L, L), dtype=bool)
    for bi in range(b):
        for hi in range(h):
            for i in range(nqb):
                for j in idx[bi, hi, i]:
                    if j >= 0:
                        m[bi, hi, i * B:(i + 1) * B, j * B:(j + 1) * B] = True
    return m


# ---------------------------------------------------------------- precompute

def test_precompute_matches_plain_loops():
    """Centroid, value sum and H_j by explicit Python sums on a tiny case."""
    Q, K, V = rand_qkv(1, h=1, L=12, d=3)
    B = 4
    st = precompute(K, V, B)
    for j in range(3):
        kb = [K[0, 0, j * B + n] for n in range(B)]
        vb = [V[0, 0, j * B + n] for n in range(B)]
        cen = [sum(kb[n][a] for n in range(B)) / B for a in range(3)]
        vs = [sum(vb[n][c] for n in range(B)) for c in range(3)]
        H = [[sum((kb[n][a] - cen[a]) * vb[n][c] for n in range(B)) for c in range(3)]
             for a in range(3)]
        assert np.allclose(st["centroid"][0, 0, j], cen, rtol=RTOL, atol=1e-14)
        assert np.allclose(st["vsum"][0, 0, j], vs, rtol=RTOL, atol=1e-14)
        assert np.allclose(st["H"][0, 0, j], H, rtol=RTOL, atol=1e-14)


def test_hbar_closed_form_and_frobenius():
    """Hbar = (K^T V - sum_j kbar_j^T sigma_j) / nb; M_j = numpy Frobenius norm."""
    Q, K, V = rand_qkv(2, h=3, L=512, d=32)
    B = 64
    nb = 512 // B
    st = precompute(K, V, B)
    for hi in range(3):
        KtV = K[0, hi].T @ V[0, hi]
        corr = sum(np.outer(st["centroid"][0, hi, j], st["vsum"][0, hi, j]) for j in range(nb))
        assert np.allclose(st["Hbar"][0, hi], (KtV - corr) / nb, rtol=1e-10, atol=1e-12)
        for j in range(nb):
            ref = np.linalg.norm(st["H"][0, hi, j] - st["Hbar"][0, hi], "fro")
            assert abs(st["M"][0, hi, j] - ref) <= 1e-12 * ref


def test_deviations_sum_to_zero():
    """The first-order weights alpha (1 + q (k - kbar)) of a block sum to B alpha."""
    Q, K, V = rand_qkv(3, h=1, L=128, d=8)
    B = 32
    st = precompute(K, V, B)
    dev = K[0, 0].reshape(4, B, 8) - st["centroid"][0, 0][:, None, :]
    assert np.abs(dev.sum(axis=1)).max() < 1e-13


# ---------------------------------------------------------------- attention vs library

@pytest.mark.parametrize("B,d", [(16, 16), (32, 8)])
def test_density_one_equals_dense(B, d):
    """With every block exact (k = nb) both modes equal dense softmax attention."""
    Q, K, V = rand_qkv(4, h=2, L=128, d=d)
    nb = 128 // B
    idx = np.broadcast_to(np.arange(nb, dtype=np.int32), (1, 2, nb, nb)).copy()
    s = 1 / math.sqrt(d)
    ref = sdpa(Q, K, V, s)
    for mode in (MODE_APPROX, MODE_DROP):
        out = run(Q, K, V, idx, B, mode, s)
        assert np.allclose(out, ref, rtol=1e-11, atol=1e-12)


def test_density_one_pure_python_loop():
    """Density 1 against a pure-Python softmax loop (no numpy/torch algebra)."""
    Q, K, V = rand_qkv(5, h=1, L=8, d=3)
    B, s = 4, 0.7
    idx = np.array([[[[0, 1], [0, 1]]]], dtype=np.int32)
    out = run(Q, K, V, idx, B, MODE_APPROX, s)
    for t in range(8):
        logits = [s * sum(Q[0, 0, t, a] * K[0, 0, n, a] for a in range(3)) for n in range(8)]
        w = [math.exp(x) for x in logits]
        o = [sum(w[n] * V[0, 0, n, c] for n in range(8)) / sum(w) for c in range(3)]
        assert np.allclose(out[0, 0, t], o, rtol=1e-12)


def test_drop_equals_masked_sdpa():
    """Keep-or-drop = softmax over the selected blocks only (block-sparse notes 3.3)."""
    Q, K, V = rand_qkv(6, h=2, L=256, d=16)
    B, nb, k = 32, 8, 3
    idx = rand_idx(7, 1, 2, nb, nb, k)
    s = 0.25
    ref = sdpa(Q, K, V, s, mask=block_mask(idx, B, 256))
    out = run(Q, K, V, idx, B, MODE_DROP, s)
    assert np.allclose(out, ref, rtol=1e-11, atol=1e-12)


def test_drop_padding_and_empty_row():
    """-1 padding is ignored; an empty keep-set gives a zero row."""
    Q, K, V = rand_qkv(8, h=1, L=128, d=8)
    B = 32
    idx = np.array([[[[1, 3, -1, -1], [-1, -1, -1, -1], [0, -1, -1, -1], [0, 1, 2, 3]]]],
                   dtype=np.int32)
    s = 0.3
    out = run(Q, K, V, idx, B, MODE_DROP, s)
    assert np.all(out[0, 0, 32:64] == 0.0)
    keep = idx.copy()
    keep[0, 0, 1] = [0, -1, -1, -1]   # any non-empty row; rows 0, 2, 3 are compared
    ref = sdpa(Q, K, V, s, mask=block_mask(keep, B, 128))
    for i in (0, 2, 3):
        assert np.allclose(out[0, 0, i * B:(i + 1) * B], ref[0, 0, i * B:(i + 1) * B], rtol=1e-11)


def test_constant_keys_make_zeroth_order_exact():
    """If every block's keys are constant, H_j = 0 and PISA equals dense attention
    for any exact set (the zeroth-order block term is then exact)."""
    g = np.random.default_rng(9)
    B, nb, d = 16, 8, 8
    cen = g.standard_normal((1, 2, nb, d))
    K = np.repeat(cen, B, axis=2)
    Q = g.standard_normal((1, 2, nb * B, d))
    V = g.standard_normal((1, 2, nb * B, d))
    s = 1 / math.sqrt(d)
    ref = sdpa(Q, K, V, s)
    for k in (1, 3, 8):
        idx = rand_idx(10 + k, 1, 2, nb, nb, k)
        out = run(Q, K, V, idx, B, MODE_APPROX, s)
        assert np.allclose(out, ref, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("mode", [MODE_APPROX, MODE_DROP])
def test_value_shift(mode):
    """O(Q, K, V + 1 v0^T) = O(Q, K, V) + v0 (pins the B alpha denominator and the
    value *sum*)."""
    Q, K, V = rand_qkv(11, h=2, L=256, d=16)
    B, nb = 32, 8
    idx = rand_idx(12, 1, 2, nb, nb, 3)
    v0 = np.random.default_rng(13).standard_normal(16) * 3
    s = 0.25
    a = run(Q, K, V, idx, B, mode, s)
    b = run(Q, K, V + v0, idx, B, mode, s)
    assert np.allclose(b, a + v0, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("mode", [MODE_APPROX, MODE_DROP])
def test_key_shift(mode):
    """A common shift of every key leaves O unchanged for a fixed exact set."""
    Q, K, V = rand_qkv(14, h=2, L=256, d=16)
    B, nb = 32, 8
    idx = rand_idx(15, 1, 2, nb, nb, 2)
    c0 = np.random.default_rng(16).standard_normal(16)
    s = 0.25
    a = run(Q, K, V, idx, B, mode, s)
    b = run(Q, K + c0, V, idx, B, mode, s)
    assert np.allclose(a, b, rtol=1e-9, atol=1e-10)


def test_zero_query_gives_means():
    """Q = 0: PISA averages V over all tokens; keep-or-drop over the kept ones."""
    _, K, V = rand_qkv(17, h=1, L=128, d=8)
    Q = np.zeros_like(K)
    B, nb = 32, 4
    idx = np.array([[[[0, 2], [1, 3], [3, -1], [0, 1]]]], dtype=np.int32)
    a = run(Q, K, V, idx, B, MODE_APPROX, 0.5)
    assert np.allclose(a[0, 0], V[0, 0].mean(axis=0), rtol=1e-12)
    d = run(Q, K, V, idx, B, MODE_DROP, 0.5)
    for i in range(nb):
        toks = np.concatenate([np.arange(j * B, (j + 1) * B) for j in idx[0, 0, i] if j >= 0])
        assert np.allclose(d[0, 0, i * B:(i + 1) * B], V[0, 0, toks].mean(axis=0), rtol=1e-12)


def test_block_permutation():
    """Reordering KV blocks (with idx remapped) leaves O unchanged; reordering
    query blocks reorders O's rows."""
    Q, K, V = rand_qkv(18, h=1, L=256, d=16)
    B, nb = 32, 8
    idx = rand_idx(19, 1, 1, nb, nb, 3)
    s = 0.25
    base = run(Q, K, V, idx, B, MODE_APPROX, s)
    perm = np.random.default_rng(20).permutation(nb)          # new block p holds old block perm[p]
    inv = np.argsort(perm)
    Kp = K.reshape(1, 1, nb, B, 16)[:, :, perm].reshape(K.shape)
    Vp = V.reshape(1, 1, nb, B, 16)[:, :, perm].reshape(V.shape)
    idxp = np.sort(inv[idx], axis=-1).astype(np.int32)
    assert np.allclose(run(Q, Kp, Vp, idxp, B, MODE_APPROX, s), base, rtol=1e-11, atol=1e-12)
    qp = np.random.default_rng(21).permutation(nb)
    Qp = Q.reshape(1, 1, nb, B, 16)[:, :, qp].reshape(Q.shape)
    outq = run(Qp, K, V, idx[:, :, qp], B, MODE_APPROX, s)
    assert np.allclose(outq.reshape(1, 1, nb, B, 16), base.reshape(1, 1, nb, B, 16)[:, :, qp],
                       rtol=1e-12)


# ---------------------------------------------------------------- first-order term

def equal_H_inputs(seed, eps, nb=6, B=8, d=4, L_q=None):
    """Blocks K_j = c_j + eps * delta, V_j = W + 1 v_j^T with a shared zero-mean
    delta and a shared W, so H_j = eps delta^T W for every j and Hbar = H_j."""
    g = np.random.default_rng(seed)
    delta = g.standard_normal((B, d))
    delta -= delta.mean(axis=0)
    W = g.standard_normal((B, d))
    cen = g.standard_normal((nb, d))
    vshift = g.standard_normal((nb, d))
    K = (cen[:, None, :] + eps * delta[None]).reshape(1, 1, nb * B, d)
    V = (W[None] + vshift[:, None, :]).reshape(1, 1, nb * B, d)
    Q = g.standard_normal((1, 1, nb * B, d))
    return Q, K, V


def taylor_bruteforce(Q, K, V, idx, B, s, Lvalid=None):
    """Token-level first-order block Taylor expansion written from its
    definition: exact weights e^{q k} on S_i, weights
    e^{q kbar_j} (1 + q (k - kbar_j)) on every token of U_i; o = sum w v / sum w.
    With Lvalid only tokens t < Lvalid exist (kbar_j is the mean of the block's
    existing keys, empty blocks drop out) and later rows are 0.
    Pure Python loops; only for tiny inputs."""
    _, _, L, d = Q.shape
    Lv = L if Lvalid is None else Lvalid
    nb = L // B
    out = np.zeros((L, d))
    for t in range(Lv):
        i = t // B
        S = {int(j) for j in idx[0, 0, i] if j >= 0}
        q = [s * Q[0, 0, t, a] for a in range(d)]
        num = [0.0] * d
        den = 0.0
        for j in range(nb):
            toks = range(j * B, min((j + 1) * B, Lv))
            if len(toks) == 0:
                continue
            kbar = [sum(K[0, 0, n, a] for n in toks) / len(toks) for a in range(d)]
            alpha = math.exp(sum(q[a] * kbar[a] for a in range(d)))
            for n in toks:
                if j in S:
                    w = math.exp(sum(q[a] * K[0, 0, n, a] for a in range(d)))
                else:
                    w = alpha * (1 + sum(q[a] * (K[0, 0, n, a] - kbar[a]) for a in range(d)))
                den += w
                for c in range(d):
                    num[c] += w * V[0, 0, n, c]
        out[t] = [x / den for x in num]
    return out


@pytest.mark.parametrize("eps", [0.3, 1.0])
def test_pisa_equals_token_taylor_when_H_equal(eps):
    """With all H_j equal, the mixed-order form (global Hbar) is exactly the
    token-level first-order expansion of every unselected block."""
    Q, K, V = equal_H_inputs(22, eps)
    B, nb = 8, 6
    idx = rand_idx(23, 1, 1, nb, nb, 2)
    s = 0.5
    st = precompute(K, V, B)
    assert np.allclose(st["H"][0, 0], st["Hbar"][0, 0][None], atol=1e-12)
    out = run(Q, K, V, idx, B, MODE_APPROX, s, st)
    ref = taylor_bruteforce(Q, K, V, idx, B, s)
    assert np.allclose(out[0, 0], ref, rtol=1e-11, atol=1e-12)


def test_error_is_second_order_in_block_spread():
    """PISA vs dense error falls as eps^2 when H_j = Hbar; without the
    correction (Hbar := 0) it falls only as eps."""
    B, nb, s = 8, 6, 0.5
    idx = rand_idx(24, 1, 1, nb, nb, 2)
    errs, errs0 = [], []
    for eps in (0.2, 0.1, 0.05):
        Q, K, V = equal_H_inputs(25, eps)
        st = precompute(K, V, B)
        ref = sdpa(Q, K, V, s)
        out = run(Q, K, V, idx, B, MODE_APPROX, s, st)
        out0 = attention(Q, K, V, idx, st["centroid"], st["vsum"], 0 * st["Hbar"],
                         MODE_APPROX, s, B)
        errs.append(np.abs(out - ref).max())
        errs0.append(np.abs(out0 - ref).max())
    r = [errs[i] / errs[i + 1] for i in range(2)]
    r0 = [errs0[i] / errs0[i + 1] for i in range(2)]
    assert all(3.4 < x < 4.6 for x in r), r
    assert all(1.7 < x < 2.3 for x in r0), r0


# ---------------------------------------------------------------- approximation orders

def het_inputs(seed, eps, nb=6, B=8, d=4):
    """Blocks with their own centroid and their own zero-mean key deviations of
    size eps, independent N(0,1) values: every H_j differs (and is not
    symmetric), so Hbar != H_j."""
    g = np.random.default_rng(seed)
    cen = g.standard_normal((nb, d))
    dev = g.standard_normal((nb, B, d))
    dev -= dev.mean(axis=1, keepdims=True)
    K = (cen[:, None, :] + eps * dev).reshape(1, 1, nb * B, d)
    V = g.standard_normal((1, 1, nb * B, d))
    Q = g.standard_normal((1, 1, nb * B, d))
    return Q, K, V


def zeroth_bruteforce(Q, K, V, idx, B, s, Lvalid=None):
    """Token-level zeroth-order expansion from its definition: exact weights
    e^{q k} on S_i, the weight e^{q kbar_j} on every token of a block of U_i
    (with Lvalid: existing tokens only, as in taylor_bruteforce).
    Pure Python loops; only for tiny inputs."""
    _, _, L, d = Q.shape
    Lv = L if Lvalid is None else Lvalid
    nb = L // B
    out = np.zeros((L, d))
    for t in range(Lv):
        i = t // B
        S = {int(j) for j in idx[0, 0, i] if j >= 0}
        q = [s * Q[0, 0, t, a] for a in range(d)]
        num, den = [0.0] * d, 0.0
        for j in range(nb):
            toks = range(j * B, min((j + 1) * B, Lv))
            if len(toks) == 0:
                continue
            kbar = [sum(K[0, 0, n, a] for n in toks) / len(toks) for a in range(d)]
            alpha = math.exp(sum(q[a] * kbar[a] for a in range(d)))
            for n in toks:
                w = math.exp(sum(q[a] * K[0, 0, n, a] for a in range(d))) if j in S else alpha
                den += w
                for c in range(d):
                    num[c] += w * V[0, 0, n, c]
        out[t] = [x / den for x in num]
    return out


@pytest.mark.parametrize("seed", [40, 41])
def test_first_order_per_block_equals_token_taylor(seed):
    """MODE_FIRST is the token-level first-order expansion of every unselected
    block, for heterogeneous (non-symmetric) H_j and any S_i, including a row
    with an empty S_i."""
    Q, K, V = het_inputs(seed, 0.7)
    B, nb, s = 8, 6, 0.5
    idx = rand_idx(seed + 1, 1, 1, nb, nb, 2)
    idx[0, 0, 3] = -1
    st = precompute(K, V, B)
    assert not np.allclose(st["H"][0, 0, 0], st["H"][0, 0, 0].T)
    out = run(Q, K, V, idx, B, MODE_FIRST, s, st)
    assert np.allclose(out[0, 0], taylor_bruteforce(Q, K, V, idx, B, s), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("seed", [42, 43])
def test_zeroth_order_equals_token_zeroth(seed):
    Q, K, V = het_inputs(seed, 0.7)
    B, nb, s = 8, 6, 0.5
    idx = rand_idx(seed + 1, 1, 1, nb, nb, 3)
    out = run(Q, K, V, idx, B, MODE_ZEROTH, s)
    assert np.allclose(out[0, 0], zeroth_bruteforce(Q, K, V, idx, B, s), rtol=1e-11, atol=1e-12)


def test_error_order_of_each_approximation():
    """Against dense attention, with heterogeneous H_j: the per-block first
    order errs as eps^2; the zeroth order and the mixed order (whose global
    Hbar leaves H_j - Hbar uncorrected) err as eps."""
    B, nb, s = 8, 6, 0.5
    idx = rand_idx(24, 1, 1, nb, nb, 2)
    ratios = {}
    for mode in (MODE_APPROX, MODE_ZEROTH, MODE_FIRST):
        errs = []
        for eps in (0.1, 0.05, 0.025):
            Q, K, V = het_inputs(31, eps)
            errs.append(np.abs(run(Q, K, V, idx, B, mode, s) - sdpa(Q, K, V, s)).max())
        ratios[mode] = [errs[i] / errs[i + 1] for i in range(2)]
    assert all(3.4 < x < 4.6 for x in ratios[MODE_FIRST]), ratios
    assert all(1.7 < x < 2.3 for x in ratios[MODE_APPROX]), ratios
    assert all(1.7 < x < 2.3 for x in ratios[MODE_ZEROTH]), ratios


def test_orders_coincide_in_their_special_cases():
    """All H_j equal (so Hbar = H_j): the per-block and the mixed order agree.
    Values constant inside every block (so every H_j = 0): all three agree.
    Density one (U empty): all four modes are dense attention."""
    B, nb, s = 8, 6, 0.5
    idx = rand_idx(50, 1, 1, nb, nb, 2)
    Q, K, V = equal_H_inputs(51, 0.8)
    assert np.allclose(run(Q, K, V, idx, B, MODE_FIRST, s), run(Q, K, V, idx, B, MODE_APPROX, s),
                       rtol=1e-11, atol=1e-12)
    Q, K, _ = het_inputs(52, 0.8)
    Vc = np.repeat(np.random.default_rng(53).standard_normal((1, 1, nb, 1, 4)), B, axis=3).reshape(K.shape)
    outs = [run(Q, K, Vc, idx, B, m, s) for m in (MODE_APPROX, MODE_ZEROTH, MODE_FIRST)]
    assert np.allclose(outs[0], outs[1], rtol=1e-11, atol=1e-12)
    assert np.allclose(outs[0], outs[2], rtol=1e-11, atol=1e-12)
    full = np.broadcast_to(np.arange(nb, dtype=np.int32), (1, 1, nb, nb)).copy()
    ref = sdpa(Q, K, Vc, s)
    for m in (MODE_APPROX, MODE_ZEROTH, MODE_FIRST, MODE_DROP):
        assert np.allclose(run(Q, K, Vc, full, B, m, s), ref, rtol=1e-10, atol=1e-12)


def test_first_order_needs_H():
    Q, K, V = het_inputs(54, 0.5)
    st = precompute(K, V, 8)
    idx = rand_idx(55, 1, 1, 6, 6, 2)
    with pytest.raises(ValueError):
        attention(Q, K, V, idx, st["centroid"], st["vsum"], st["Hbar"], MODE_FIRST, 0.5, 8)


# ---------------------------------------------------------------- worked examples

LN3 = math.log(3.0)
SQ3 = math.sqrt(3.0)
V00, V01 = np.array([1., 2., 0., 0.]), np.array([3., 0., 1., 0.])
V10, V11 = np.array([0., 1., 2., 3.]), np.array([2., 0., 0., 1.])


def worked_inputs(a):
    """2 blocks of B=2 tokens, d=4, scale 1/2.  Block 0 keys are 0; block 1 keys
    are (1+a, 0,0,0) and (1-a, 0,0,0).  Queries: q0 = q2 = (2 ln 3, 0, 0, 0),
    q1 = q3 = 0."""
    K = np.zeros((1, 1, 4, 4))
    K[0, 0, 2, 0] = 1 + a
    K[0, 0, 3, 0] = 1 - a
    V = np.stack([V00, V01, V10, V11])[None, None]
    Q = np.zeros((1, 1, 4, 4))
    Q[0, 0, 0, 0] = Q[0, 0, 2, 0] = 2 * LN3
    return Q, K, V


def test_worked_example_constant_keys():
    """a = 0, S_0 = {0}: logits 0, 0 exact; alpha_1 = e^{ln 3} = 3, H = 0.
    o_0 = (v00 + v01 + 3 (v10 + v11)) / (2 + 2*3) = (10, 5, 7, 12) / 8;
    keep-or-drop o_0 = (v00 + v01) / 2; q1 = 0 gives (6, 3, 3, 4) / 4."""
    Q, K, V = worked_inputs(0.0)
    idx = np.array([[[[0], [1]]]], dtype=np.int32)
    out = run(Q, K, V, idx, 2, MODE_APPROX, 0.5)
    assert np.allclose(out[0, 0, 0], np.array([10, 5, 7, 12]) / 8, rtol=1e-14)
    assert np.allclose(out[0, 0, 1], np.array([6, 3, 3, 4]) / 4, rtol=1e-14)
    drop = run(Q, K, V, idx, 2, MODE_DROP, 0.5)
    assert np.allclose(drop[0, 0, 0], (V00 + V01) / 2, rtol=1e-14)


def test_worked_example_first_order():
    """a = 1/2: H_0 = 0, H_1 has row 0 = a (v10 - v11) = (-1, .5, 1, 1), so Hbar
    row 0 = (-.5, .25, .5, .5) and M_0 = M_1 = sqrt(.8125).
    Query 0 (S = {0}, alpha = 3): N = (10,5,7,12) + 3 ln3 (-.5,.25,.5,.5), D = 8.
    Query 2 (S = {1}, U = {0}, alpha = 1): exact weights 3^{1.5}, 3^{0.5};
    N = 3 sqrt3 v10 + sqrt3 v11 + (v00 + v01) + ln3 (-.5,.25,.5,.5),
    D = 3 sqrt3 + sqrt3 + 2."""
    Q, K, V = worked_inputs(0.5)
    st = precompute(K, V, 2)
    hbar = np.zeros((4, 4))
    hbar[0] = [-0.5, 0.25, 0.5, 0.5]
    assert np.allclose(st["Hbar"][0, 0], hbar, rtol=1e-14, atol=1e-15)
    assert np.allclose(st["M"][0, 0], [math.sqrt(0.8125)] * 2, rtol=1e-14)
    assert np.allclose(st["centroid"][0, 0, 1], [1, 0, 0, 0], rtol=1e-14)
    assert np.allclose(st["vsum"][0, 0, 1], V10 + V11, rtol=1e-14)
    idx = np.array([[[[0], [1]]]], dtype=np.int32)
    out = run(Q, K, V, idx, 2, MODE_APPROX, 0.5, st)
    e0 = (np.array([10, 5, 7, 12]) + 3 * LN3 * hbar[0]) / 8
    assert np.allclose(out[0, 0, 0], e0, rtol=1e-14)
    n2 = 3 * SQ3 * V10 + SQ3 * V11 + V00 + V01 + LN3 * hbar[0]
    assert np.allclose(out[0, 0, 2], n2 / (4 * SQ3 + 2), rtol=1e-14)
    assert np.allclose(out[0, 0, 3], (V00 + V01 + V10 + V11) / 4, rtol=1e-14)


# ---------------------------------------------------------------- routing

def test_route_lambda_zero_is_topk_of_block_mean_logits():
    """With lambda = 0 the score is the mean of the B x B tile of dense logits
    (bilinearity), so S_i is the top-k of those tile means."""
    Q, K, V = rand_qkv(26, h=2, L=256, d=16)
    B, nb, k, s = 32, 8, 3, 0.25
    st = precompute(K, V, B)
    idx = route(Q, st["centroid"], st["M"], k, 0.0, B, s)
    for hi in range(2):
        logits = s * Q[0, hi] @ K[0, hi].T
        tile = logits.reshape(nb, B, nb, B).mean(axis=(1, 3))
        for i in range(nb):
            ranked = sorted(range(nb), key=lambda j: (-tile[i, j], j))
            assert list(idx[0, hi, i]) == sorted(ranked[:k])


def test_route_large_lambda_follows_M():
    Q, K, V = rand_qkv(27, h=1, L=256, d=16)
    B, nb, k = 32, 8, 3
    st = precompute(K, V, B)
    idx = route(Q, st["centroid"], st["M"], k, 1e9, B, 0.25)
    top = sorted(sorted(range(nb), key=lambda j: (-st["M"][0, 0, j], j))[:k])
    assert all(list(r) == top for r in idx[0, 0])


def test_route_bruteforce_and_ties():
    """Plain full sort on tiny inputs, plus a hand-made tie: centroids 0 and
    M = (3, 1, 3, 3) with lambda 1 give scores M, and k = 2 keeps {0, 2}."""
    g = np.random.default_rng(28)
    Q = g.standard_normal((1, 1, 16, 4))
    cen = g.standard_normal((1, 1, 4, 4))
    M = np.abs(g.standard_normal((1, 1, 4)))
    for k in (1, 2, 4):
        idx = route(Q, cen, M, k, 0.7, 4, 0.5)
        for i in range(4):
            qbar = [sum(Q[0, 0, 4 * i + n, a] for n in range(4)) / 4 for a in range(4)]
            sc = [0.5 * sum(qbar[a] * cen[0, 0, j, a] for a in range(4)) + 0.7 * M[0, 0, j]
                  for j in range(4)]
            want = sorted(sorted(range(4), key=lambda j: (-sc[j], j))[:k])
            assert list(idx[0, 0, i]) == want
    idx = route(Q, np.zeros((1, 1, 4, 4)), np.array([[[3., 1., 3., 3.]]]), 2, 1.0, 4, 0.5)
    assert all(list(r) == [0, 2] for r in idx[0, 0])


# ---------------------------------------------------------------- sensitivity

def test_pins_catch_planted_statistic_mistakes():
    """Plausible mistakes in the statistics (value mean instead of sum, Hbar as a
    sum, transposed Hbar, centroid off by a factor) each fail a pin above."""
    Q, K, V = equal_H_inputs(29, 0.5)
    B, nb, s = 8, 6, 0.5
    idx = rand_idx(30, 1, 1, nb, nb, 2)
    st = precompute(K, V, B)
    ref = taylor_bruteforce(Q, K, V, idx, B, s)
    good = attention(Q, K, V, idx, st["centroid"], st["vsum"], st["Hbar"], MODE_APPROX, s, B)
    assert np.allclose(good[0, 0], ref, rtol=1e-11)
    mutants = {
        "vsum as mean": (st["centroid"], st["vsum"] / B, st["Hbar"]),
        "Hbar as sum": (st["centroid"], st["vsum"], st["Hbar"] * nb),
        "Hbar transposed": (st["centroid"], st["vsum"], np.swapaxes(st["Hbar"], -1, -2)),
        "centroid scaled": (st["centroid"] * 1.01, st["vsum"], st["Hbar"]),
    }
    for name, (c, vs, hb) in mutants.items():
        bad = attention(Q, K, V, idx, c, vs, hb, MODE_APPROX, s, B)
        assert not np.allclose(bad[0, 0], ref, rtol=1e-6), name


def test_pins_catch_planted_first_order_mistakes():
    """Plausible mistakes in the per-block first-order term (H_j transposed,
    Hbar used in place of H_j, the first-order term scaled by B, a block's H
    taken from its neighbour) each fail the token-level Taylor pin."""
    Q, K, V = het_inputs(56, 0.6)
    B, nb, s = 8, 6, 0.5
    idx = rand_idx(57, 1, 1, nb, nb, 2)
    st = precompute(K, V, B)
    ref = taylor_bruteforce(Q, K, V, idx, B, s)
    args = (Q, K, V, idx, st["centroid"], st["vsum"], st["Hbar"], MODE_FIRST, s, B)
    assert np.allclose(attention(*args, H=st["H"])[0, 0], ref, rtol=1e-11, atol=1e-12)
    mutants = {
        "H_j transposed": np.swapaxes(st["H"], -1, -2),
        "Hbar for every block": np.broadcast_to(st["Hbar"][:, :, None], st["H"].shape),
        "first order times B": st["H"] * B,
        "H of the next block": np.roll(st["H"], 1, axis=2),
    }
    for name, Hm in mutants.items():
        bad = attention(*args, H=Hm)
        assert not np.allclose(bad[0, 0], ref, rtol=1e-6), name


# ---------------------------------------------------------------- spectral M_j

def diag34_blocks():
    """Two blocks of B = 4 tokens, d = 2.  Block 0: key deviations e1, -e1, e2,
    -e2 around a centroid, values 3 e1, 0, 4 e2, 0, so H_0 = diag(3, 4); block 1
    has the values negated, so H_1 = -H_0, Hbar = 0 and H_j - Hbar = +-diag(3, 4):
    spectral norm 4, Frobenius norm 5."""
    e1, e2 = np.array([1.0, 0.0]), np.array([0.0, 1.0])
    c0, c1 = np.array([0.3, -0.2]), np.array([-1.0, 0.5])
    dev = np.stack([e1, -e1, e2, -e2])
    K = np.concatenate([c0 + dev, c1 + dev])[None, None]
    v0 = np.stack([3 * e1, 0 * e1, 4 * e2, 0 * e2])
    V = np.concatenate([v0, -v0])[None, None]
    return K, V


def test_spectral_norm_closed_form():
    K, V = diag34_blocks()
    sp = precompute(K, V, 4, norm="spectral")
    fr = precompute(K, V, 4)
    assert np.allclose(sp["H"][0, 0, 0], np.diag([3.0, 4.0]), atol=1e-15)
    assert np.allclose(sp["Hbar"], 0.0, atol=1e-15)
    assert np.allclose(sp["M"], 4.0, rtol=1e-14)
    assert np.allclose(fr["M"], 5.0, rtol=1e-14)


def power_iteration_sigma(A, iters=3000):
    """Largest singular value by plain power iteration on A^T A, pure Python."""
    n = len(A)
    x = [1.0 + 0.1 * i for i in range(n)]
    lam = 0.0
    for _ in range(iters):
        y = [sum(A[r][c] * x[c] for c in range(n)) for r in range(n)]
        z = [sum(A[r][c] * y[r] for r in range(n)) for c in range(n)]
        nz = math.sqrt(sum(t * t for t in z))
        lam = nz / math.sqrt(sum(t * t for t in x))
        x = [t / nz for t in z]
    return math.sqrt(lam)


def test_spectral_norm_bruteforce_invariance_and_bounds():
    """Tiny random blocks: spectral M equals a power-iteration brute force, is
    unchanged by orthogonal rotations of the key and value spaces
    (K -> K R, V -> V S turns H_j into R^T H_j S), and sits between
    ||.||_F / sqrt(d) and ||.||_F."""
    Q, K, V = rand_qkv(60, h=1, L=24, d=3)
    B = 6
    sp = precompute(K, V, B, norm="spectral")
    fr = precompute(K, V, B)
    diff = sp["H"] - sp["Hbar"][:, :, None]
    for j in range(4):
        assert math.isclose(sp["M"][0, 0, j], power_iteration_sigma(diff[0, 0, j].tolist()),
                            rel_tol=1e-9)
    g = np.random.default_rng(61)
    R, _ = np.linalg.qr(g.standard_normal((3, 3)))
    S, _ = np.linalg.qr(g.standard_normal((3, 3)))
    rot = precompute(K @ R, V @ S, B, norm="spectral")
    assert np.allclose(rot["M"], sp["M"], rtol=1e-12)
    assert np.all(sp["M"] <= fr["M"] * (1 + 1e-12))
    assert np.all(sp["M"] >= fr["M"] / math.sqrt(3) * (1 - 1e-12))
    assert not np.allclose(sp["M"], fr["M"], rtol=1e-3)


def test_spectral_is_an_option_not_a_change():
    """The default (Frobenius) statistics and everything but M are unchanged by the option."""
    Q, K, V = rand_qkv(62, h=1, L=64, d=8)
    a, b = precompute(K, V, 8), precompute(K, V, 8, norm="spectral")
    for key in ("centroid", "vsum", "H", "Hbar"):
        assert np.array_equal(a[key], b[key])
    with pytest.raises(ValueError):
        precompute(K, V, 8, norm="nuclear")


# ---------------------------------------------------------------- variable lengths

def varlen_inputs(seed, b=2, h=2, L=48, d=4, B=8):
    Q, K, V = rand_qkv(seed, b=b, h=h, L=L, d=d)
    K = K + np.repeat(np.random.default_rng(seed + 1).standard_normal((b, h, L // B, 1, d)),
                      B, axis=3).reshape(K.shape)
    return Q, K, V


def runv(Q, K, V, idx, B, mode, scale, lens, st=None):
    st = precompute(K, V, B, seq_lens=lens) if st is None else st
    return attention(Q, K, V, idx, st["centroid"], st["vsum"], st["Hbar"], mode, scale, B,
                     H=st["H"], seq_lens=lens)


ALL_MODES = (MODE_APPROX, MODE_ZEROTH, MODE_FIRST, MODE_DROP)


def test_varlen_full_lengths_are_the_plain_call():
    Q, K, V = varlen_inputs(70)
    B, nb, s = 8, 6, 0.5
    idx = rand_idx(71, 2, 2, nb, nb, 2)
    lens = [48, 48]
    a, b_ = precompute(K, V, B), precompute(K, V, B, seq_lens=lens)
    for key in a:
        assert np.allclose(a[key], b_[key], rtol=1e-13, atol=1e-13)
    for m in ALL_MODES:
        assert np.allclose(run(Q, K, V, idx, B, m, s), runv(Q, K, V, idx, B, m, s, lens),
                           rtol=1e-12, atol=1e-13)


def test_varlen_density_one_is_sdpa_on_the_valid_prefix():
    """Every non-empty block exact: each batch entry is dense attention over its
    own valid tokens (torch SDPA on the truncated tensors); padding rows are 0."""
    Q, K, V = varlen_inputs(72)
    B, nb, s = 8, 6, 0.5
    lens = [37, 16]                       # a partial block; an exact multiple of B
    full = np.broadcast_to(np.arange(nb, dtype=np.int32), (2, 2, nb, nb)).copy()
    for m in ALL_MODES:
        out = runv(Q, K, V, full, B, m, s, lens)
        for bi, n in enumerate(lens):
            ref = sdpa(Q[bi:bi + 1, :, :n], K[bi:bi + 1, :, :n], V[bi:bi + 1, :, :n], s)
            assert np.allclose(out[bi:bi + 1, :, :n], ref, rtol=1e-10, atol=1e-12), m
            assert np.all(out[bi, :, n:] == 0.0)


def test_varlen_drop_is_masked_sdpa():
    Q, K, V = varlen_inputs(73)
    B, nb, s = 8, 6, 0.5
    lens = [37, 21]
    idx = rand_idx(74, 2, 2, nb, nb, 3)
    out = runv(Q, K, V, idx, B, MODE_DROP, s, lens)
    mask = block_mask(idx, B, 48)
    for bi, n in enumerate(lens):
        mk = mask[bi:bi + 1, :, :n, :n]
        ref = sdpa(Q[bi:bi + 1, :, :n], K[bi:bi + 1, :, :n], V[bi:bi + 1, :, :n], s, mask=mk)
        rows = mk.any(axis=-1)                      # query rows with at least one valid key
        got = out[bi:bi + 1, :, :n]
        assert np.allclose(got[rows], ref[rows], rtol=1e-10, atol=1e-12)
        assert np.all(got[~rows] == 0.0)


@pytest.mark.parametrize("Lv", [37, 40, 33])
def test_varlen_first_and_zeroth_equal_token_expansions(Lv):
    """Ragged last block (and an empty one): the per-block first order and the
    zeroth order equal their token-level expansions over the existing tokens."""
    Q, K, V = het_inputs(75, 0.7)
    B, nb, s = 8, 6, 0.5
    idx = rand_idx(76, 1, 1, nb, nb, 2)
    idx[0, 0, 0] = [4, 5]                          # the partial / empty block as exact
    idx[0, 0, 1] = [0, 5]
    out1 = runv(Q, K, V, idx, B, MODE_FIRST, s, [Lv])
    out0 = runv(Q, K, V, idx, B, MODE_ZEROTH, s, [Lv])
    assert np.allclose(out1[0, 0], taylor_bruteforce(Q, K, V, idx, B, s, Lv), rtol=1e-11, atol=1e-12)
    assert np.allclose(out0[0, 0], zeroth_bruteforce(Q, K, V, idx, B, s, Lv), rtol=1e-11, atol=1e-12)


def test_varlen_padding_contents_never_matter():
    """NaN in every padding position: statistics and outputs are unchanged."""
    Q, K, V = varlen_inputs(77)
    B, nb, s = 8, 6, 0.5
    lens = [37, 16]
    idx = rand_idx(78, 2, 2, nb, nb, 2)
    Qn, Kn, Vn = Q.copy(), K.copy(), V.copy()
    for bi, n in enumerate(lens):
        for X in (Qn, Kn, Vn):
            X[bi, :, n:] = np.nan
    a, b_ = precompute(K, V, B, seq_lens=lens), precompute(Kn, Vn, B, seq_lens=lens)
    for key in a:
        assert np.array_equal(a[key], b_[key]), key
    for m in ALL_MODES:
        assert np.array_equal(runv(Q, K, V, idx, B, m, s, lens), runv(Qn, Kn, Vn, idx, B, m, s, lens))


def test_varlen_statistics_closed_forms():
    """Partial block: centroid = mean of its valid keys; empty block: zero
    statistics and M = 0; Hbar = mean of H_j over the non-empty blocks only."""
    Q, K, V = varlen_inputs(79, b=1, h=1)
    B = 8
    st = precompute(K, V, B, seq_lens=[37])
    assert np.allclose(st["centroid"][0, 0, 4], K[0, 0, 32:37].mean(axis=0), rtol=1e-14)
    assert np.allclose(st["vsum"][0, 0, 4], V[0, 0, 32:37].sum(axis=0), rtol=1e-14)
    dev = K[0, 0, 32:37] - K[0, 0, 32:37].mean(axis=0)
    assert np.allclose(st["H"][0, 0, 4], dev.T @ V[0, 0, 32:37], rtol=1e-12, atol=1e-14)
    assert np.all(st["centroid"][0, 0, 5] == 0) and np.all(st["H"][0, 0, 5] == 0)
    assert st["M"][0, 0, 5] == 0.0
    assert np.allclose(st["Hbar"][0, 0], st["H"][0, 0, :5].sum(axis=0) / 5, rtol=1e-13)


def test_varlen_route_skips_empty_blocks():
    """Empty key blocks are never chosen; a query block with no valid token gets
    an all -1 row; with fewer than k non-empty blocks the row is padded with -1.
    The rest is a plain sort of the prefix-pooled scores."""
    Q, K, V = varlen_inputs(80)
    B, nb, s = 8, 6, 0.5
    lens = [37, 14]                                # entry 1: blocks 0 (8) and 1 (6) only
    st = precompute(K, V, B, seq_lens=lens)
    idx = route(Q, st["centroid"], st["M"], 3, 0.1, B, s, seq_lens=lens)
    assert np.all(idx[0, :, :5] <= 4) and np.all(idx[0, :, 5] == -1)
    assert np.all(idx[1, :, :2, :2] >= 0) and np.all(idx[1, :, :2, 2] == -1)
    assert np.all(idx[1, :, 2:] == -1)
    for hi in range(2):
        for i in range(5):
            toks = range(i * B, min((i + 1) * B, 37))
            qbar = Q[0, hi, list(toks)].mean(axis=0)
            sc = [s * qbar @ st["centroid"][0, hi, j] + 0.1 * st["M"][0, hi, j] for j in range(5)]
            best = sorted(range(5), key=lambda j: (-sc[j], j))[:3]
            assert list(idx[0, hi, i]) == sorted(best)
