"""Plain fp64 CPU oracle for piecewise block-sparse attention (PISA).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check in
``__graft_entry__.smoke`` and the ``cpu_baseline`` leg of ``bench.py`` may import
or call anything in this package.  The product path (the HIP library and its
Python binding) never imports it, and this module imports nothing from the
product: the two share no code, constants or helpers.

What it computes, and where each step comes from
-------------------------------------------------
Sources (cited by page title and section; no line numbers):

* PISA page -- "PISA: Piecewise Sparse Attention Is Wiser for Efficient
  Diffusion Transformers", technical summary on gist.science (arXiv 2602.01077):
  section 2 "Methodology", sub-parts "Core algorithm" (the output ratio
  o_t = N_t / D_t and the numerator N_t), "Covariance-aware routing" (the block
  score uses the attention score and M_j = ||H_j - Hbar||_2) and "Hardware
  implementation" (the precompute of centroids, value sums and Hbar).
* Block-sparse notes -- the block-sparse attention on multimodal DiT notes on
  dpshk.com: section 3.3 (keep-or-drop block-sparse softmax,
  O_i = softmax(Q_i K_{S_i}^T / sqrt(d)) V_{S_i}) and section 4.1 (blocks are
  padded so no block is ragged).

Functions, one per call of the C ABI:

* ``precompute(K, V, B, norm="fro")`` -> block centroids, value sums, per-block
  H_j, Hbar, M_j (``norm="spectral"``: the other reading of ||.||_2, below)
* ``route(Q, centroid, M, k, lam, B, scale)`` -> per-query-block exact set S_i
  (``route_scores`` exposes the float64 scores it ranks)
* ``attention(Q, K, V, idx, centroid, vsum, Hbar, mode, scale, B, H=None)`` -> O

Approximation orders of the unselected blocks (``mode``):

* ``MODE_APPROX`` -- the PISA mixed order: zeroth-order block terms plus the
  global first-order correction with Hbar.
* ``MODE_ZEROTH`` -- the zeroth-order block terms alone (no correction).
* ``MODE_FIRST`` -- a separate first-order term for every unselected block,
  alpha_{t,j} * (q H_j), i.e. the full block Taylor expansion that the mixed
  order approximates by replacing each H_j with Hbar (PISA page, section 2,
  "Core algorithm", the global first-order correction, which the page
  introduces to avoid exactly these per-block terms; section 3, the mixed-order
  scheme).
* ``MODE_DROP`` -- keep-or-drop block-sparse attention over S_i only.

Readings where the pages are silent or ambiguous:

* Softmax scale: the PISA numerator is printed without a scale, the keep-or-drop
  formula divides by sqrt(d).  Reading: every q_t is pre-multiplied by
  ``scale`` (1/sqrt(d) by default), in the exact logits, in alpha and in the
  first-order correction q_t Hbar.
* Denominator D_t: the page only says it is made of the same three parts.
  Reading, from the first-order block Taylor expansion
  exp(q k) ~ exp(q kbar_j) (1 + q (k - kbar_j)): summing the weights over a
  block gives B * alpha_{t,j} because the deviations k_{j,n} - kbar_j sum to
  zero, so D_t = sum_{S_i} sum_n exp(q k) + B * sum_{U_i} alpha_{t,j} and the
  first-order term contributes nothing to D_t.
* Centroid = arithmetic mean of the block's B keys; value sum = plain sum.
* H_j = sum_n (k_{j,n} - kbar_j)^T v_{j,n} is d_k x d_v; q Hbar is a row vector.
* Hbar = mean of H_j over all blocks of the same (batch, head).
* ||.||_2 of a matrix read as the Frobenius norm (entrywise 2-norm) by default;
  ``norm="spectral"`` takes the operator 2-norm (largest singular value)
  instead, the other standard meaning of the symbol.
* Routing score: scale * qbar_i . kbar_j + lam * M_j with qbar_i the mean query
  of block i; the k largest are exact, ties go to the lower block index, and
  the set is returned in ascending order.  One S_i serves the whole query block.
* Keep-or-drop with an empty S_i gives o_t = 0.

Variable lengths (``seq_lens``, one valid length per batch entry).  The
block-sparse notes pad each modality to a multiple of the block size
(section 4.1) and pad a batch of different lengths to its longest sample
(section 8.2) but never say what the padding does to the statistics.
Reading: tokens at or beyond the valid length are not part of the sequence.
Block j then holds n_j = clip(len - j B, 0, B) tokens and every statistic
counts only those (centroid = their mean; the denominator weight of an
unselected block is n_j alpha instead of B alpha); Hbar is the mean over the
non-empty blocks; empty blocks are never routed (their M_j is reported as 0);
a query block with no valid token gets an all -1 row; output rows of padding
queries are 0.  If fewer than k blocks are non-empty, the row holds all of
them followed by -1.

All arithmetic is float64.  Inputs of any float dtype are upcast exactly.
"""

from __future__ import annotations

import numpy as np

MODE_APPROX = 0
MODE_DROP = 1
MODE_ZEROTH = 2
MODE_FIRST = 3


def _blocks(X: np.ndarray, B: int) -> np.ndarray:
    """[b,h,L,d] -> [b,h,nb,B,d] in float64; L must be a multiple of B.

    The block-sparse notes (section 4.1) pad each modality to a multiple of the
    block size before splitting, so blocks are never ragged.
    """
    X = np.asarray(X, dtype=np.float64)
    b, h, L, d = X.shape
    if L % B != 0:
        raise ValueError(f"sequence length {L} is not a multiple of block size {B}")
    return X.reshape(b, h, L // B, B, d)


def _valid(seq_lens, b: int, nb: int, B: int) -> np.ndarray:
    """Boolean [b, nb, B]: token n of block j of batch entry bi is in the sequence."""
    L = nb * B
    lens = np.full(b, L) if seq_lens is None else np.clip(np.asarray(seq_lens, dtype=np.int64), 0, L)
    if lens.shape != (b,):
        raise ValueError("seq_lens must hold one length per batch entry")
    pos = np.arange(L).reshape(nb, B)
    return pos[None] < lens[:, None, None]


def precompute(K: np.ndarray, V: np.ndarray, B: int, norm: str = "fro", seq_lens=None) -> dict:
    """Block statistics of the PISA precompute stage.

    PISA page, section 2, "Core algorithm": the zeroth-order term of block j
    uses the block centroid kbar_j and the block value sum sum_n v_{j,n}; the
    first-order term uses H_j = sum_n (k_{j,n} - kbar_j)^T v_{j,n} and the
    global Hbar, the mean of H_j over all blocks.  "Covariance-aware routing":
    M_j = ||H_j - Hbar||_2 (Frobenius reading, or with norm="spectral" the
    largest singular value).  "Hardware implementation": these are computed
    before the attention stages.

    Returns a dict of float64 arrays:
      centroid [b,h,nb,d], vsum [b,h,nb,d], H [b,h,nb,d,d] (row = key dim,
      column = value dim), Hbar [b,h,d,d], M [b,h,nb].

    seq_lens: optional valid length per batch entry (see the module notes);
    only the n_j valid tokens of a block enter its statistics.
    """
    Kb = _blocks(K, B)
    Vb = _blocks(V, B)
    if Kb.shape != Vb.shape:
        raise ValueError("K and V must have the same shape")
    b, _, nb, _, _ = Kb.shape
    valid = _valid(seq_lens, b, nb, B)[:, None, :, :, None]        # [b,1,nb,B,1]
    n = valid.sum(axis=3)                                          # n_j [b,1,nb,1]
    Kv = np.where(valid, Kb, 0.0)                   # padding never enters (even NaN)
    Vv = np.where(valid, Vb, 0.0)
    centroid = Kv.sum(axis=3) / np.maximum(n, 1)    # kbar_j: mean of the block's keys
    vsum = Vv.sum(axis=3)                           # sum_n v_{j,n}
    dev = np.where(valid, Kb - centroid[:, :, :, None, :], 0.0)    # k_{j,n} - kbar_j
    # H_j[a, c] = sum_n dev[n, a] * v[n, c]: a (d x B) @ (B x d) product per block
    H = np.matmul(np.swapaxes(dev, -1, -2), Vv)
    nonempty = n[..., 0] > 0                                       # [b,1,nb]
    # Hbar: mean over the (non-empty) blocks of this (b, h)
    Hbar = H.sum(axis=2) / np.maximum(nonempty.sum(axis=2), 1)[:, :, None, None]
    diff = H - Hbar[:, :, None, :, :]
    if norm == "fro":
        M = np.sqrt((diff * diff).sum(axis=(-2, -1)))   # Frobenius norm of H_j - Hbar
    elif norm == "spectral":
        M = np.linalg.norm(diff, ord=2, axis=(-2, -1))  # largest singular value (LAPACK SVD)
    else:
        raise ValueError(f"unknown norm {norm!r}")
    M = np.where(nonempty, M, 0.0)                  # empty blocks are never routed
    return {"centroid": centroid, "vsum": vsum, "H": H, "Hbar": Hbar, "M": M}


def route_scores(Q: np.ndarray, centroid: np.ndarray, M: np.ndarray, lam: float,
                 B: int, scale: float, seq_lens=None) -> np.ndarray:
    """Routing scores (PISA page, section 2, "Covariance-aware routing"):
    score_ij = scale * qbar_i . kbar_j + lam * M_j, with qbar_i the mean of the
    B queries of block i.  Returns float64 [b,h,nqb,nb].

    With seq_lens, qbar_i is the mean of block i's valid queries, and the score
    is -inf for an empty key block and on every entry of an empty query block."""
    Qb = _blocks(Q, B)
    centroid = np.asarray(centroid, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    b, _, nqb, _, _ = Qb.shape
    valid = _valid(seq_lens, b, nqb, B)[:, None, :, :, None]
    n = valid.sum(axis=3)                                           # [b,1,nqb,1]
    qbar = np.where(valid, Qb, 0.0).sum(axis=3) / np.maximum(n, 1)  # [b,h,nqb,d]
    sc = scale * np.matmul(qbar, np.swapaxes(centroid, -1, -2)) + lam * M[:, :, None, :]
    empty = n[..., 0] == 0                                          # [b,1,nqb]
    sc = np.where(empty[:, :, None, :], -np.inf, sc)                # empty key blocks
    return np.where(empty[:, :, :, None], -np.inf, sc)             # empty query blocks


def route(Q: np.ndarray, centroid: np.ndarray, M: np.ndarray, k: int, lam: float,
          B: int, scale: float, seq_lens=None) -> np.ndarray:
    """Covariance-aware top-k block selection (PISA page, section 2,
    "Covariance-aware routing").

    S_i = the k highest ``route_scores`` of query block i, ties broken towards
    the lower block index; returned ascending as int32 [b,h,nqb,k].  Blocks
    with a -inf score (empty ones, with seq_lens) are never chosen; a row with
    fewer than k candidates holds them all followed by -1.
    """
    scores = route_scores(Q, centroid, M, lam, B, scale, seq_lens)
    b, h, nqb, nb = scores.shape
    if not (1 <= k <= nb):
        raise ValueError(f"k={k} must lie in [1, {nb}]")
    idx = np.empty((b, h, nqb, k), dtype=np.int32)
    order_key = np.arange(nb)
    for bi in range(b):
        for hi in range(h):
            for i in range(nqb):
                # sort by score descending, then block index ascending
                order = np.lexsort((order_key, -scores[bi, hi, i]))
                top = np.sort([j for j in order[:k] if np.isfinite(scores[bi, hi, i, j])])
                idx[bi, hi, i] = np.concatenate([top, -np.ones(k - len(top))]).astype(np.int32)
    return idx


def attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, idx: np.ndarray,
              centroid: np.ndarray, vsum: np.ndarray, Hbar: np.ndarray,
              mode: int, scale: float, B: int, qblocks=None, H=None,
              seq_lens=None) -> np.ndarray:
    """PISA exact-or-approximate attention, or keep-or-drop block-sparse attention.

    PISA page, section 2, "Core algorithm": o_t = N_t / D_t with
      N_t = sum_{j in S_i} sum_n e^{q k_{j,n}} v_{j,n}
            + sum_{j in U_i} alpha_{t,j} sum_n v_{j,n}
            + q_t Hbar sum_{j in U_i} alpha_{t,j},      alpha_{t,j} = e^{q kbar_j}
    and (reading) D_t = sum_{S_i} sum_n e^{q k} + B sum_{U_i} alpha_{t,j}, where
    q = scale * q_t.  U_i is every block not in S_i.

    Block-sparse notes, section 3.3 (mode == MODE_DROP): only the S_i terms
    remain, i.e. softmax over the selected blocks' keys; an empty S_i gives 0.

    MODE_ZEROTH drops the q_t Hbar term.  MODE_FIRST replaces it with the
    per-block first-order terms sum_{j in U_i} alpha_{t,j} (q H_j), which needs
    ``H`` [b,h,nb,d,d] from ``precompute``; the denominator is the same in all
    three orders because the first-order term of a block sums to zero over its
    keys.

    idx: int [b,h,nqb,kmax]; entries are block ids, -1 entries are padding.
    qblocks: optional iterable of (b, h, i) triples; only those query blocks are
      computed and every other output row is NaN.
    seq_lens: optional valid length per batch entry: keys beyond it are not
      attended, block j weighs n_j alpha in D_t, empty blocks are not in U_i,
      and output rows of padding queries are 0.
    Returns float64 [b,h,L,d].
    """
    Qb = _blocks(Q, B)
    Kb = _blocks(K, B)
    Vb = _blocks(V, B)
    centroid = np.asarray(centroid, dtype=np.float64)
    vsum = np.asarray(vsum, dtype=np.float64)
    Hbar = np.asarray(Hbar, dtype=np.float64)
    idx = np.asarray(idx)
    if mode not in (MODE_APPROX, MODE_DROP, MODE_ZEROTH, MODE_FIRST):
        raise ValueError(f"unknown mode {mode}")
    if mode == MODE_FIRST:
        if H is None:
            raise ValueError("MODE_FIRST needs the per-block H_j")
        H = np.asarray(H, dtype=np.float64)
    b, h, nqb, _, d = Qb.shape
    nb = Kb.shape[2]
    dv = Vb.shape[-1]
    valid = _valid(seq_lens, b, nb, B)                              # [b, nb, B]
    count = valid.sum(axis=2)                                       # n_j [b, nb]
    out = np.full((b, h, nqb, B, dv), np.nan)
    if qblocks is None:
        qblocks = [(bi, hi, i) for bi in range(b) for hi in range(h) for i in range(nqb)]
    for bi, hi, i in qblocks:
        row = [int(j) for j in idx[bi, hi, i] if j >= 0]
        if len(set(row)) != len(row) or any(j >= nb for j in row):
            raise ValueError(f"idx row ({bi},{hi},{i}) has duplicates or out-of-range ids")
        S = sorted(j for j in row if count[bi, j] > 0)               # empty blocks hold no key
        chosen = set(S)
        U = [j for j in range(nb) if j not in chosen and count[bi, j] > 0]
        qv = valid[bi, i]                                            # valid query rows
        out[bi, hi, i] = 0.0                                         # rows of padding queries
        if not qv.any():
            continue
        q = scale * Qb[bi, hi, i][qv]                                # [n_i, d]
        # exact logits over the selected blocks' valid keys
        kv = valid[bi, S].reshape(-1)
        KS = Kb[bi, hi, S].reshape(-1, d)[kv]                        # [sum n_j, d]
        VS = Vb[bi, hi, S].reshape(-1, dv)[kv]
        ell = q @ KS.T                                               # [n_i, sum n_j]
        if mode == MODE_DROP:
            if len(S) == 0:
                continue
            m = ell.max(axis=1, keepdims=True)
            w = np.exp(ell - m)
            out[bi, hi, i, qv] = (w @ VS) / w.sum(axis=1, keepdims=True)
            continue
        # zeroth-order block terms over U_i: alpha_{t,j} = e^{q . kbar_j}
        c = q @ centroid[bi, hi, U].T                                # [B, |U|]
        parts = [x for x in (ell, c) if x.size]
        m = np.max(np.concatenate(parts, axis=1), axis=1, keepdims=True)
        w = np.exp(ell - m)                                          # exact weights
        a = np.exp(c - m)                                            # alpha, shifted by m
        asum = a.sum(axis=1, keepdims=True)                          # sum_{U} alpha
        N = w @ VS + a @ vsum[bi, hi, U]
        if mode == MODE_APPROX:
            N = N + (q @ Hbar[bi, hi]) * asum
        elif mode == MODE_FIRST and U:
            # sum_j alpha_{t,j} (q_t H_j): one (n_i x d) @ (d x dv) product per block
            qH = np.matmul(q[None, :, :], H[bi, hi, U])              # [|U|, n_i, dv]
            N = N + np.einsum("tj,jtc->tc", a, qH)
        # a block of n_j tokens weighs n_j alpha in the denominator (B when full)
        D = w.sum(axis=1, keepdims=True) + a @ count[bi, U].astype(np.float64)[:, None]
        out[bi, hi, i, qv] = N / D
    return out.reshape(b, h, nqb * B, dv)
