"""Parity rules between the HIP library and the CPU oracle.

Tolerance (fixed by the benchmark spec for this path): the GPU's NN index must
equal the oracle's wherever the oracle's top-1 to top-2 similarity margin
exceeds 1e-5; elsewhere the chosen neighbour's (binary64) similarity must be
within 1e-5 of the maximum (fp32 maps) or within 1e-2 * |max| (bf16 maps).
Pointmaps (nearest points) use the relative rule derived at MARGIN_PT.
The oracle computes in binary64 on exactly the values the GPU receives.

For the fast reciprocal scheme, which is an iteration rather than a closed
form, the rules are:
  (i)   every oracle pair collected by a chain whose NN decisions all had a
        margin above 1e-5 ("clean") is in the GPU output;
  (ii)  every GPU pair (u, v) is eps-reciprocal in binary64:
        s(u, v) >= top1(u -> image 2) - eps and s(u, v) >= top1(v -> image 1) - eps;
  (iii) the GPU output is one-to-one and ascending in u;
  (iv)  if every seed's chain is clean, the GPU set equals the oracle's set, and the
        GPU's live count per iteration equals the oracle's count of first visits
        (the GPU never restarts a chain on a pixel that was live before);
  (v)   otherwise only unclean chains may end elsewhere: a chain whose decisions all
        clear the margin is followed identically on the GPU, and a chain yields at
        most one pair, so the GPU-only pairs and the oracle-only pairs each number
        at most the unclean seeds.
"""
from __future__ import annotations

import numpy as np

import oracle

MARGIN = 1e-5
# Pointmaps (metric 1, scores = -squared distance): the fp32 squared distance errs by
# at most about 4 * 2^-24 = 2.4e-7 of itself, so the index is fixed wherever the two
# smallest exact squared distances differ by more than 1e-6 of the second, and
# elsewhere the chosen point lies within 1e-6 (relative) of the nearest.
POINT = 1
MARGIN_PT = 1e-6


def tol_for(dtype: str, top1: np.ndarray) -> np.ndarray:
    if dtype == "bf16":
        return 1e-2 * np.abs(top1)
    return np.full_like(top1, 1e-5)


def margin_of(top1, top2, metric=0):
    """Decision margin from the oracle's two best scores (relative for pointmaps)."""
    top1, top2 = np.asarray(top1, np.float64), np.asarray(top2, np.float64)
    if metric != POINT:
        return top1 - top2
    with np.errstate(divide="ignore", invalid="ignore"):
        m = (top1 - top2) / -top2
    m = np.where(np.isneginf(top2), np.inf, m)
    return np.where(top2 == 0, 0.0, m)


def _near_enough(s, top1, dtype, metric):
    """Is score s (of the GPU's choice) within tolerance of the best score top1?"""
    if metric == POINT:   # -s and -top1 are squared distances
        return -s <= -top1 * (1 + MARGIN_PT) + 1e-30
    return s >= top1 - tol_for(dtype, top1)


def check_nn(gpu_idx, o_idx, o_top1, o_top2, qmap, rows, db, dtype, metric=0):
    """NN parity for queries qmap[rows] against db.  Returns a small report dict."""
    gpu_idx = np.asarray(gpu_idx).astype(np.int64)
    o_idx = np.asarray(o_idx).astype(np.int64)
    sure = margin_of(o_top1, o_top2, metric) > (MARGIN_PT if metric == POINT else MARGIN)
    bad_exact = np.nonzero(sure & (gpu_idx != o_idx))[0]
    assert bad_exact.size == 0, f"{bad_exact.size} clear-margin NN mismatches, e.g. query {rows[bad_exact[0]]}"
    amb = np.nonzero(~sure)[0]
    if amb.size:
        assert (gpu_idx[amb] >= 0).all()
        s = oracle.similarity_pairs(qmap, db, np.asarray(rows)[amb], gpu_idx[amb], metric=metric)
        ok = _near_enough(s, o_top1[amb], dtype, metric)
        assert ok.all(), f"{int((~ok).sum())} ambiguous NNs beyond tolerance"
    return dict(n=len(gpu_idx), exact=int(sure.sum()), ambiguous=int(amb.size),
                equal=int((gpu_idx == o_idx).sum()))


def check_one_to_one_sorted(pairs):
    pairs = np.asarray(pairs).reshape(-1, 2)
    if len(pairs) == 0:
        return
    u, v = pairs[:, 0], pairs[:, 1]
    assert (np.diff(u) > 0).all(), "pairs not strictly ascending in u"
    assert len(np.unique(v)) == len(v), "a pixel of image 2 is matched twice"


def _reciprocal_ok(pairs, A, B, dtype, nthreads=None, metric=0):
    """Rule (ii) per pair: (forward ok, backward ok) boolean arrays."""
    u, v = pairs[:, 0], pairs[:, 1]
    _, f1, _ = oracle.nn_rows(A, u, B, nthreads, metric=metric)
    _, b1, _ = oracle.nn_rows(B, v, A, nthreads, metric=metric)
    s = oracle.similarity_pairs(A, B, u, v, metric=metric)
    return _near_enough(s, f1, dtype, metric), _near_enough(s, b1, dtype, metric)


def check_reciprocal(pairs, A, B, dtype, nthreads=None, metric=0):
    """Rule (ii) for every listed GPU pair."""
    pairs = np.asarray(pairs).reshape(-1, 2)
    if len(pairs) == 0:
        return
    fwd, bwd = _reciprocal_ok(pairs, A, B, dtype, nthreads, metric)
    assert fwd.all(), "a GPU pair is not a forward NN within tolerance"
    assert bwd.all(), "a GPU pair is not a backward NN within tolerance"


def fast_rule_counts(gpu_pairs, orc, A, B, dtype, nthreads=None, metric=0, gpu_active=None):
    """Rules (i)-(v) counted rather than asserted, for reports.  For each rule: how many
    items pass and fail, and up to three failing items.  Items are oracle clean pairs
    (i), GPU pairs (ii), steps between consecutive GPU pairs (iii, ascending u), GPU
    pairs (iii, v used once), pairs of either set (iv, set equality), iterations (iv,
    live counts) and the one bound each of (v).  A rule that does not apply (iv when
    some chain is unclean; the live counts when none are given) counts 0 and 0."""
    gpu_pairs = np.asarray(gpu_pairs).reshape(-1, 2)
    gset = {(int(a), int(b)) for a, b in gpu_pairs}
    oset = {(int(a), int(b)) for a, b in orc["pairs"]}
    clean = {(int(a), int(b)) for (a, b), c in zip(orc["pairs"], orc["clean"]) if c}
    unclean = int((np.asarray(orc["seed_clean"]) == 0).sum())
    gpu_only, oracle_only = gset - oset, oset - gset
    rules = {}

    def put(name, passed, failed_items):
        failed_items = sorted(failed_items)
        rules[name] = dict(passed=int(passed), failed=len(failed_items),
                           examples=[[int(x) for x in np.atleast_1d(f)] for f in failed_items[:3]])

    u, v = gpu_pairs[:, 0], gpu_pairs[:, 1]
    steps = np.nonzero(np.diff(u) <= 0)[0] + 1
    put("iii_ascending_in_u", max(len(u) - 1, 0) - len(steps), [(int(u[k - 1]), int(u[k])) for k in steps])
    vals, cnt = np.unique(v, return_counts=True)
    put("iii_v_used_once", len(v) - int((cnt - 1).sum()), [int(x) for x in vals[cnt > 1]])
    missing = clean - gset
    put("i_clean_pairs_found", len(clean) - len(missing), missing)
    if len(gpu_pairs):
        fwd, bwd = _reciprocal_ok(gpu_pairs, A, B, dtype, nthreads, metric)
        ok = fwd & bwd
        put("ii_eps_reciprocal", int(ok.sum()), [tuple(map(int, gpu_pairs[k])) for k in np.nonzero(~ok)[0]])
    else:
        put("ii_eps_reciprocal", 0, [])
    if unclean == 0:
        put("iv_equal_sets", len(gset & oset), gpu_only | oracle_only)
        if gpu_active is not None:
            ga = np.asarray(gpu_active).reshape(-1)[:len(orc["fresh"])].tolist()
            fr = orc["fresh"].tolist()
            put("iv_live_counts", sum(a == b for a, b in zip(ga, fr)),
                [(t, a, b) for t, (a, b) in enumerate(zip(ga, fr)) if a != b])
        else:
            put("iv_live_counts", 0, [])
    else:
        put("iv_equal_sets", 0, [])
        put("iv_live_counts", 0, [])
    put("v_gpu_only_within_unclean", int(len(gpu_only) <= unclean),
        [] if len(gpu_only) <= unclean else [(len(gpu_only), unclean)])
    put("v_oracle_only_within_unclean", int(len(oracle_only) <= unclean),
        [] if len(oracle_only) <= unclean else [(len(oracle_only), unclean)])
    summary = dict(gpu=len(gset), oracle=len(oset), clean=len(clean), common=len(gset & oset),
                   gpu_only=len(gpu_only), oracle_only=len(oracle_only), unclean_seeds=unclean)
    return rules, summary


def check_fast(gpu_pairs, orc, A, B, dtype, nthreads=None, metric=0, gpu_active=None):
    """Rules (i)-(v) against a full oracle run `orc` (dict from oracle.fast);
    gpu_active: the GPU's live count per iteration, or None."""
    R, summary = fast_rule_counts(gpu_pairs, orc, A, B, dtype, nthreads, metric, gpu_active)
    assert not R["iii_ascending_in_u"]["failed"], "pairs not strictly ascending in u"
    assert not R["iii_v_used_once"]["failed"], "a pixel of image 2 is matched twice"
    r = R["i_clean_pairs_found"]
    assert not r["failed"], f"{r['failed']} clean oracle pairs missing, e.g. {r['examples']}"
    r = R["ii_eps_reciprocal"]
    assert not r["failed"], f"{r['failed']} GPU pairs not an NN within tolerance both ways, e.g. {r['examples']}"
    r = R["iv_equal_sets"]
    assert not r["failed"], \
        f"every chain is clean, yet {summary['gpu_only']} GPU-only and {summary['oracle_only']} oracle-only " \
        f"pairs, e.g. {r['examples']}"
    r = R["iv_live_counts"]
    assert not r["failed"], f"live counts differ from the oracle's first visits at (t, gpu, oracle) {r['examples']}"
    assert not R["v_gpu_only_within_unclean"]["failed"], \
        f"{summary['gpu_only']} GPU-only pairs but only {summary['unclean_seeds']} unclean chains"
    assert not R["v_oracle_only_within_unclean"]["failed"], \
        f"{summary['oracle_only']} oracle-only pairs but only {summary['unclean_seeds']} unclean chains"
    return summary


def oracle_chains(A, B, seeds, T, nthreads=None, eps=None, metric=0):
    """Follow the chains of the given seeds with the oracle's NN, one iteration at a time
    (for workloads too large for a full oracle run).  Returns {(u, v): clean}."""
    if eps is None:
        eps = MARGIN_PT if metric == POINT else MARGIN
    cur = {int(s): [int(s), True] for s in seeds}
    out = {}
    for _ in range(T):
        if not cur:
            break
        us = np.array(sorted({c[0] for c in cur.values()}), np.int32)
        f, f1, f2 = oracle.nn_rows(A, us, B, nthreads, metric=metric)
        fmap = {int(u): (int(v), m) for u, v, m in zip(us, f, margin_of(f1, f2, metric))}
        vs = np.array(sorted({fmap[c[0]][0] for c in cur.values()}), np.int32)
        g, g1, g2 = oracle.nn_rows(B, vs, A, nthreads, metric=metric)
        gmap = {int(v): (int(u), m) for v, u, m in zip(vs, g, margin_of(g1, g2, metric))}
        nxt = {}
        for s, (u, ok) in cur.items():
            v, m1 = fmap[u]
            u2, m2 = gmap[v]
            ok = ok and m1 > eps and m2 > eps
            if u2 == u:
                out[(u, v)] = out.get((u, v), False) or ok
            else:
                nxt[s] = [u2, ok]
        cur = nxt
    return out
