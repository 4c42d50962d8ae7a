"""Helpers of the GPU parity tests: device upload, the oracle side of a case,
and the tolerance checks (all comparisons are GPU result vs fp64 oracle)."""

import numpy as np

import oracle

# tolerances on attention outputs (GPU vs oracle, same idx, own statistics)
TOL = {"bf16": dict(rel_l2=1e-2, max_abs=2e-2), "fp32": dict(rel_l2=1e-5, max_abs=1e-5)}
# statistics (fp32 on both input types) against the fp64 oracle
STATS_REL = 1e-5
# routing: a differing block is accepted only if the oracle scores of the
# swapped blocks are within this gap of each other
ROUTE_GAP = 1e-6


def to_dev(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def to_np(t):
    import torch
    return t.detach().to("cpu", torch.float64).numpy()


def rel_l2(a, ref):
    return float(np.linalg.norm(a - ref) / max(np.linalg.norm(ref), 1e-300))


def check_stats(gpu: dict, ref: dict, heads=None, name=""):
    """gpu: dict of torch tensors (all heads); ref: oracle stats of `heads`."""
    sel = slice(None) if heads is None else list(heads)
    for key in ("centroid", "vsum", "Hbar", "M"):
        g = to_np(gpu[key])[:, sel]
        r = ref[key]
        err = rel_l2(g, r)
        assert err <= STATS_REL, f"{name} {key}: rel-L2 {err:.3e}"
    g = to_np(gpu["M"])[:, sel]
    mrel = float(np.max(np.abs(g - ref["M"]) / np.maximum(np.abs(ref["M"]), 1e-30)))
    assert mrel <= STATS_REL, f"{name} M: max rel {mrel:.3e}"
    if gpu.get("H") is not None:
        err = rel_l2(to_np(gpu["H"])[:, sel], ref["H"])
        assert err <= STATS_REL, f"{name} H: rel-L2 {err:.3e}"


def check_route(idx_gpu: np.ndarray, scores: np.ndarray, k: int, name=""):
    """Indices bit-exact with the oracle's top-k of `scores`, except swaps among
    blocks whose oracle scores differ by at most ROUTE_GAP.  Returns the number
    of rows that differ (all of them near-ties).
    Scores of -inf (blocks outside a shorter sequence) are never candidates:
    a row with fewer than k finite scores must hold exactly those, followed
    by -1."""
    b, h, nqb, nb = scores.shape
    keys = np.arange(nb)
    ndiff = 0
    for bi in range(b):
        for hi in range(h):
            for i in range(nqb):
                sc = scores[bi, hi, i]
                order = [j for j in np.lexsort((keys, -sc)) if np.isfinite(sc[j])]
                ref = np.sort(order[:k])
                g = idx_gpu[bi, hi, i]
                nv = len(ref)
                assert np.all(g[nv:] == -1), f"{name} row {(bi, hi, i)}: expected -1 after {nv} ids"
                g = g[:nv]
                if nv == 0:
                    continue
                assert np.all(np.diff(g) > 0), f"{name} row {(bi, hi, i)} not ascending"
                assert g.min() >= 0 and g.max() < nb and np.all(np.isfinite(sc[g]))
                if not np.array_equal(g, ref):
                    only_g = np.setdiff1d(g, ref)
                    only_r = np.setdiff1d(ref, g)
                    gap = sc[only_r].max() - sc[only_g].min()
                    assert len(only_g) == len(only_r) and gap <= ROUTE_GAP, \
                        f"{name} row {(bi, hi, i)}: differs beyond a near-tie (gap {gap:.3e})"
                    ndiff += 1
    return ndiff


def check_attention(out_gpu: np.ndarray, out_ref: np.ndarray, dtype: str, name=""):
    """Compare where the oracle computed (non-NaN rows)."""
    mask = ~np.isnan(out_ref[..., 0])
    g, r = out_gpu[mask], out_ref[mask]
    assert np.all(np.isfinite(g)), f"{name}: non-finite GPU output"
    err, mab = rel_l2(g, r), float(np.abs(g - r).max())
    tol = TOL[dtype]
    assert err <= tol["rel_l2"] and mab <= tol["max_abs"], \
        f"{name}: rel-L2 {err:.3e} (<= {tol['rel_l2']}), max-abs {mab:.3e} (<= {tol['max_abs']})"
    return err, mab


def oracle_stats(K, V, B, heads=None):
    if heads is not None:
        K, V = K[:, list(heads)], V[:, list(heads)]
    return oracle.precompute(K, V, B)
