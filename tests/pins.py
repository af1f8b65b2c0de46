"""Pins for the CPU oracle: checks against facts the pages and the mathematics fix.

Each pin takes an ``oracle.Oracle`` (the real build, or a deliberately broken
copy of the same source built by the mutation test) and raises AssertionError
on failure.  None of them re-types the oracle's own code: they use hand-derived
fixtures (tests/golden), closed forms (identity, permutation, planted
noise-free fields), brute force with numpy on tiny inputs, and invariants of the
reciprocal scheme.

Run as a script (``python tests/pins.py LIBPATH``) it prints the names of the
failing pins as JSON, which is how the mutation test runs broken builds in a
child process.
"""
from __future__ import annotations

import json
import math
import os
import sys

import numpy as np

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

import workloads  # noqa: E402

GOLDEN = os.path.join(_ROOT, "tests", "golden")


def _load_golden(name):
    with open(os.path.join(GOLDEN, name + ".json")) as f:
        g = json.load(f)
    if "angles1" in g:
        a = np.radians(np.asarray(g["angles1"], np.float64))
        b = np.radians(np.asarray(g["angles2"], np.float64))
        A = np.stack([np.cos(a), np.sin(a)], 1).astype(np.float32)
        B = np.stack([np.cos(b), np.sin(b)], 1).astype(np.float32)
    else:
        A = np.asarray(g["vectors1"], np.float32)
        B = np.asarray(g["vectors2"], np.float32)
    return g, A, B


def _rand_unit(rng, n, d):
    x = rng.standard_normal((n, d))
    return (x / np.linalg.norm(x, axis=1, keepdims=True)).astype(np.float32)


def _pairs_set(p):
    return {(int(a), int(b)) for a, b in np.asarray(p).reshape(-1, 2)}


# ============================================================================ NN

def pin_golden_nn(orc):
    """Hand-derived NN maps (tests/golden)."""
    for name in ("circle_1x4", "grid_2x3", "ties_d1", "negative_scores"):
        g, A, B = _load_golden(name)
        i12, t1, t2 = orc.nn(A, B)
        i21, _, _ = orc.nn(B, A)
        assert i12.tolist() == g["nn12"], (name, i12)
        assert i21.tolist() == g["nn21"], (name, i21)
        if "top1_12" in g:
            assert np.allclose(t1, g["top1_12"], atol=1e-7), (name, t1)
            assert np.allclose(t2, g["top2_12"], atol=1e-7), (name, t2)


def pin_nn_numpy_bruteforce(orc):
    """argmax of the full float64 similarity matrix (numpy takes the first maximum)."""
    rng = np.random.default_rng(11)
    for (n1, n2, d) in ((37, 53, 24), (20, 9, 3), (5, 64, 1), (33, 31, 7)):
        A = _rand_unit(rng, n1, d)
        B = _rand_unit(rng, n2, d)
        S = A.astype(np.float64) @ B.astype(np.float64).T
        idx, t1, t2 = orc.nn(A, B)
        assert (idx == S.argmax(1)).all()
        assert np.allclose(t1, S.max(1), atol=1e-12, rtol=0)
        Ss = np.sort(S, axis=1)
        if n2 > 1:
            assert np.allclose(t2, Ss[:, -2], atol=1e-12, rtol=0)


def pin_nn_identity(orc):
    """B = A with distinct rows: every row is its own NN, top1 = |a|^2."""
    rng = np.random.default_rng(12)
    A = _rand_unit(rng, 60, 24)
    idx, t1, _ = orc.nn(A, A)
    assert (idx == np.arange(60)).all()
    sq = np.array([math.fsum(float(x) * float(x) for x in r) for r in A])
    assert np.allclose(t1, sq, atol=1e-15, rtol=0)


def pin_nn_permutation(orc):
    """B[k] = A[pi(k)]: NN21 = pi and NN12 = pi^-1 (pi is not an involution)."""
    rng = np.random.default_rng(13)
    A = _rand_unit(rng, 40, 24)
    pi = np.roll(np.arange(40), 7)
    pi = pi[rng.permutation(40)]
    assert (pi[pi] != np.arange(40)).any()
    B = A[pi]
    i21, _, _ = orc.nn(B, A)
    i12, _, _ = orc.nn(A, B)
    inv = np.empty(40, np.int64)
    inv[pi] = np.arange(40)
    assert (i21 == pi).all()
    assert (i12 == inv).all()


def pin_nn_ties_lowest_index(orc):
    """Exact duplicates: the lowest index wins and top2 == top1."""
    rng = np.random.default_rng(14)
    A = _rand_unit(rng, 4, 24)
    B = _rand_unit(rng, 12, 24)
    B[9] = A[0]
    B[3] = A[0]
    B[6] = A[1]
    B[11] = A[1]
    idx, t1, t2 = orc.nn(A[:2], B)
    assert idx.tolist() == [3, 6]
    assert (t1 == t2).all()
    ones = np.ones((7, 1), np.float32)
    idx, t1, t2 = orc.nn(ones, ones)
    assert (idx == 0).all() and (t1 == 1).all() and (t2 == 1).all()


def pin_nn_margin(orc):
    """top1/top2 against closed-form cosines: query at 0 deg, rows at 30, 10, 20, 50 deg."""
    ang = np.radians([30.0, 10.0, 20.0, 50.0])
    B = np.stack([np.cos(ang), np.sin(ang)], 1).astype(np.float32)
    A = np.array([[1.0, 0.0]], np.float32)
    idx, t1, t2 = orc.nn(A, B)
    assert idx[0] == 1
    assert abs(t1[0] - math.cos(math.radians(10))) < 1e-7
    assert abs(t2[0] - math.cos(math.radians(20))) < 1e-7


def pin_nn_rows_gather(orc):
    """nn_rows(qmap, rows) equals nn on the gathered rows."""
    rng = np.random.default_rng(15)
    A = _rand_unit(rng, 30, 24)
    B = _rand_unit(rng, 25, 24)
    rows = np.array([29, 0, 5, 5, 17], np.int32)
    S = A[rows].astype(np.float64) @ B.astype(np.float64).T
    idx, _, _ = orc.nn_rows(A, rows, B)
    assert (idx == S.argmax(1)).all()


def pin_similarity_closed_form(orc):
    """s((cos a, sin a), (cos b, sin b)) = cos(a - b), within fp32 input rounding."""
    a = np.radians([0.0, 33.0, 170.0, -80.0])
    b = np.radians([45.0, 33.0, 10.0, 100.0])
    A = np.stack([np.cos(a), np.sin(a)], 1).astype(np.float32)
    B = np.stack([np.cos(b), np.sin(b)], 1).astype(np.float32)
    s = orc.similarity_pairs(A, B, np.arange(4), np.arange(4))
    assert np.allclose(s, np.cos(a - b), atol=2e-7, rtol=0)


# ============================================================================ mutual

def pin_golden_mutual(orc):
    for name in ("circle_1x4", "grid_2x3", "ties_d1", "negative_scores"):
        g, A, B = _load_golden(name)
        pairs = orc.mutual_nn(A, B)[0]
        assert pairs.tolist() == g["mutual"], (name, pairs)


def pin_mutual_symmetry_and_one_to_one(orc):
    """M*(B, A) is M*(A, B) with each pair swapped; M* is one-to-one."""
    p = workloads.make_pair(12, 10, 24, seed=21, warp="shift", sigma=0.1, rho=0.2)
    m12 = _pairs_set(orc.mutual_nn(p.D1, p.D2)[0])
    m21 = _pairs_set(orc.mutual_nn(p.D2, p.D1)[0])
    assert m12 == {(j, i) for (i, j) in m21}
    assert len({i for i, _ in m12}) == len(m12) == len({j for _, j in m12})
    assert len(m12) > 0


def pin_mutual_planted_closed_form(orc):
    """Noise-free planted field (D2[q] = D1[src(q)] exactly, distinct D1 rows):
    M* = {(p, min{q : src(q) = p})} -- clamped borders plant exact duplicates."""
    p = workloads.make_pair(14, 11, 24, seed=22, warp="shift", sigma=0.0, rho=0.0)
    assert (p.D2 == p.D1[p.src]).all()
    first = {}
    for q, s in enumerate(p.src.tolist()):
        first.setdefault(s, q)
    expect = sorted(first.items())
    got = orc.mutual_nn(p.D1, p.D2)[0].tolist()
    assert got == [list(e) for e in expect]


# ============================================================================ fast scheme

def _chain_set(n12, n21, seeds, T):
    """The fast scheme's output by its set characterisation: every p reached from a
    seed within t <= T-1 applications of f = NN21 o NN12 with f(p) = p."""
    out = set()
    for s in seeds:
        u = int(s)
        for _ in range(T):
            v = int(n12[u])
            u2 = int(n21[v])
            if u2 == u:
                out.add((u, v))
                break
            u = u2
    return out


def _grid(H, W, stride, offset):
    return [y * W + x for y in range(offset, H, stride) for x in range(offset, W, stride)]


def pin_golden_fast(orc):
    for name in ("circle_1x4", "grid_2x3", "ties_d1", "negative_scores"):
        g, A, B = _load_golden(name)
        for case in g["fast"]:
            r = orc.fast(A, g["H1"], g["W1"], B, case["stride"], case["offset"], case["T"])
            assert r["pairs"].tolist() == case["pairs"], (name, case, r["pairs"])


def pin_fast_subset_of_mutual(orc):
    """Every fast match is a mutual NN (so the output is one-to-one)."""
    p = workloads.make_pair(24, 20, 24, seed=23, warp="shift", sigma=0.1, rho=0.2)
    mset = _pairs_set(orc.mutual_nn(p.D1, p.D2)[0])
    for stride, off, T in ((4, 2, 5), (3, 0, 2), (5, 1, 10)):
        f = _pairs_set(orc.fast(p.D1, p.H, p.W, p.D2, stride, off, T)["pairs"])
        assert f <= mset
        assert len({u for u, _ in f}) == len(f) == len({v for _, v in f})


def pin_fast_stride1_is_bruteforce(orc):
    """Stride 1 seeds every pixel; each mutual pixel is its own fixed point, so the
    scheme returns exactly the brute-force mutual set for any T >= 1."""
    p = workloads.make_pair(16, 13, 24, seed=24, warp="affine", sigma=0.15, rho=0.3)
    mset = _pairs_set(orc.mutual_nn(p.D1, p.D2)[0])
    for T in (1, 3):
        f = _pairs_set(orc.fast(p.D1, p.H, p.W, p.D2, 1, 0, T)["pairs"])
        assert f == mset


def pin_fast_set_characterisation(orc):
    """Output equals {(p, NN12(p)) : f(p) = p, p = f^t(seed), t <= T-1}, built here from
    the NN maps by walking each seed's chain."""
    p = workloads.make_pair(20, 18, 24, seed=25, warp="shift", sigma=0.1, rho=0.2)
    n12 = orc.nn(p.D1, p.D2)[0]
    n21 = orc.nn(p.D2, p.D1)[0]
    for stride, off, T in ((4, 2, 1), (4, 2, 2), (4, 2, 3), (3, 1, 10), (7, 0, 4), (2, 1, 1)):
        want = _chain_set(n12, n21, _grid(p.H, p.W, stride, off), T)
        got = _pairs_set(orc.fast(p.D1, p.H, p.W, p.D2, stride, off, T)["pairs"])
        assert got == want, (stride, off, T)


def pin_fast_monotone_ascent(orc):
    """Along a chain s(u_t, v_t) <= s(u_{t+1}, v_t) <= s(u_{t+1}, v_{t+1}); with lowest-index
    ties no chain cycles, so every chain reaches a reciprocal pair."""
    p = workloads.make_pair(20, 16, 24, seed=26, warp="shift", sigma=0.25, rho=0.4)
    n12 = orc.nn(p.D1, p.D2)[0]
    n21 = orc.nn(p.D2, p.D1)[0]
    N = p.H * p.W
    for s in range(N):
        u = s
        seen = set()
        while True:
            v = int(n12[u])
            u2 = int(n21[v])
            s0, s1 = orc.similarity_pairs(p.D1, p.D2, [u, u2], [v, v])
            assert s0 <= s1
            if u2 == u:
                break
            v2 = int(n12[u2])
            s2 = orc.similarity_pairs(p.D1, p.D2, [u2], [v2])[0]
            assert s1 <= s2
            assert u not in seen
            seen.add(u)
            u = u2


def pin_fast_planted_noise_free(orc):
    """Noise-free planted field: a seed that is a source pixel converges in the first
    iteration to min{q : src(q) = seed}; every match (u, v) has u = src(v)."""
    p = workloads.make_pair(24, 16, 24, seed=27, warp="shift", sigma=0.0, rho=0.0)
    first = {}
    for q, s in enumerate(p.src.tolist()):
        first.setdefault(s, q)
    r1 = orc.fast(p.D1, p.H, p.W, p.D2, 4, 2, 1)
    got = _pairs_set(r1["pairs"])
    seeds = _grid(p.H, p.W, 4, 2)
    assert got == {(s, first[s]) for s in seeds if s in first}
    r = orc.fast(p.D1, p.H, p.W, p.D2, 4, 2, 10)
    for u, v in r["pairs"].tolist():
        assert p.src[v] == u


def pin_fast_edges(orc):
    """T = 0 gives nothing; a stride beyond the image leaves the single seed at the
    offset; the number of live pixels starts at the seed count and never grows."""
    p = workloads.make_pair(12, 9, 24, seed=28, warp="shift", sigma=0.1, rho=0.2)
    assert orc.fast(p.D1, p.H, p.W, p.D2, 3, 1, 0)["pairs"].shape[0] == 0
    n12 = orc.nn(p.D1, p.D2)[0]
    n21 = orc.nn(p.D2, p.D1)[0]
    r = orc.fast(p.D1, p.H, p.W, p.D2, 50, 0, 6)
    assert _pairs_set(r["pairs"]) == _chain_set(n12, n21, [0], 6)
    r = orc.fast(p.D1, p.H, p.W, p.D2, 3, 1, 8)
    a = r["active"]
    assert a[0] == len(_grid(p.H, p.W, 3, 1))
    assert all(a[t + 1] <= a[t] for t in range(len(a) - 1))


def pin_fast_clean_flag(orc):
    """Chains through exact ties are not clean; well-separated chains are."""
    g, A, B = _load_golden("ties_d1")
    r = orc.fast(A, g["H1"], g["W1"], B, 1, 0, 1)
    assert r["clean"].tolist() == [0]
    g, A, B = _load_golden("circle_1x4")
    r = orc.fast(A, g["H1"], g["W1"], B, 1, 0, 1)
    assert r["clean"].tolist() == [1, 1, 1]
    # a tie only in the backward search: image-1 pixels 0 and 1 are identical
    A = np.array([[1, 0], [1, 0], [0, 1]], np.float32)
    b = np.radians([10.0, 100.0])
    B = np.stack([np.cos(b), np.sin(b)], 1).astype(np.float32)
    r = orc.fast(A, 1, 3, B, 1, 0, 1)
    assert r["pairs"].tolist() == [[0, 0], [2, 1]]
    assert r["clean"].tolist() == [0, 1]


def _numpy_nn(Q, D):
    """NN by the float64 similarity matrix (numpy takes the first maximum, i.e. the lowest
    index) with the top-1 minus top-2 margin."""
    S = Q.astype(np.float64) @ D.astype(np.float64).T
    idx = S.argmax(1)
    srt = np.sort(S, axis=1)
    top2 = srt[:, -2] if S.shape[1] > 1 else np.full(S.shape[0], -np.inf)
    return idx, srt[:, -1] - top2


def _walk_seed_records(n12, m12, n21, m21, seeds, T, eps):
    """Each seed's chain walked by hand: where it converged (-1 if not within T iterations),
    whether every decision on it cleared eps, and per iteration the number of live pixels
    that were live in no earlier iteration."""
    ends, cleans, fresh = [], [], [0] * T
    live_at = [set() for _ in range(T)]
    for s in seeds:
        u, ok, end = int(s), True, -1
        for t in range(T):
            live_at[t].add(u)
            v = int(n12[u])
            u2 = int(n21[v])
            ok = ok and m12[u] > eps and m21[v] > eps
            if u2 == u:
                end = u
                break
            u = u2
        ends.append(end)
        cleans.append(int(ok))
    ever = set()
    for t in range(T):
        fresh[t] = len(live_at[t] - ever)
        ever |= live_at[t]
    return ends, cleans, fresh


def pin_fast_seed_records(orc):
    """Per-seed end points and clean flags, and the first-visit count per iteration, against
    a hand walk of every chain over numpy brute-force NN maps and margins."""
    cases = ((20, 18, 0.1, 0.2, 4, 2, 10, 1e-5), (16, 13, 0.3, 0.5, 3, 1, 4, 1e-5),
             (24, 20, 0.2, 0.3, 5, 0, 2, 1e-5), (14, 12, 0.25, 0.4, 2, 1, 6, 0.02))
    for k, (H, W, sig, rho, stride, off, T, eps) in enumerate(cases):
        p = workloads.make_pair(H, W, 24, seed=40 + k, warp="affine", sigma=sig, rho=rho)
        n12, m12 = _numpy_nn(p.D1, p.D2)
        n21, m21 = _numpy_nn(p.D2, p.D1)
        seeds = _grid(H, W, stride, off)
        ends, cleans, fresh = _walk_seed_records(n12, m12, n21, m21, seeds, T, eps)
        r = orc.fast(p.D1, H, W, p.D2, stride, off, T, eps=eps)
        assert r["seed_u"].tolist() == ends, k
        assert r["seed_clean"].tolist() == cleans, k
        assert r["fresh"].tolist() == fresh, (k, r["fresh"], fresh)
        # the collected pairs are the end points, with the forward NN
        assert _pairs_set(r["pairs"]) == {(u, int(n12[u])) for u in ends if u >= 0}
        # a pair is clean when some clean chain collected it
        want_clean = {u for u, c in zip(ends, cleans) if u >= 0 and c}
        assert {int(u) for (u, _), c in zip(r["pairs"], r["clean"]) if c} == want_clean
    assert k == len(cases) - 1


def pin_fast_seed_records_closed_forms(orc):
    """Stride 1 and T = 1: every pixel is a seed and converges where it starts iff it is a
    mutual pixel; all N pixels are first visits.  The noise-free planted field: every seed
    that is a source pixel converges in place in the first iteration, no seed is live
    twice, and every decision is exact (large margins)."""
    p = workloads.make_pair(12, 10, 24, seed=45, warp="shift", sigma=0.1, rho=0.2)
    mutual = {int(u) for u, _ in orc.mutual_nn(p.D1, p.D2)[0]}
    r = orc.fast(p.D1, p.H, p.W, p.D2, 1, 0, 1)
    assert r["seed_u"].tolist() == [u if u in mutual else -1 for u in range(p.N)]
    assert r["fresh"].tolist() == [p.N]
    q = workloads.make_pair(24, 16, 24, seed=27, warp="shift", sigma=0.0, rho=0.0)
    srcs = set(q.src.tolist())
    seeds = _grid(q.H, q.W, 4, 2)
    r = orc.fast(q.D1, q.H, q.W, q.D2, 4, 2, 3)
    assert r["seed_u"].tolist() == [s if s in srcs else r["seed_u"][i] for i, s in enumerate(seeds)]
    assert r["fresh"][0] == len(seeds) and sum(r["fresh"]) <= q.N


# ============================================================================ pointmaps
# Metric 1: nearest = smallest Euclidean distance between 3D points ("DUSt3R and MASt3R
# explained", the paragraph on recovering the cameras); scores are -|a - b|^2.

PT = 1


def pin_point_closed_forms(orc):
    """Hand-derived distances: the nearest point is not the one of largest inner product,
    and equal distances go to the lowest index."""
    q = np.array([[1, 0, 0], [0, 0, 0], [0.5, 0.5, 0]], np.float32)
    db = np.array([[10, 0, 0], [1.5, 0, 0], [-1, 0, 0], [0, 1, 0], [0, 0, -1]], np.float32)
    idx, t1, t2 = orc.nn(q, db, metric=PT)
    # q0: squared distances 81, 0.25, 4, 2, 2 -> 1;  q1: 100, 2.25, 1, 1, 1 -> 2 (tie 2, 3, 4)
    # q2: 90.5, 1.25, 2.5, 0.5, 1.5 -> 3
    assert idx.tolist() == [1, 2, 3]
    assert t1.tolist() == [-0.25, -1.0, -0.5] and t2.tolist() == [-2.0, -1.0, -1.25]
    assert orc.nn(q, db)[0].tolist()[0] == 0          # the inner product picks (10, 0, 0)
    s = orc.similarity_pairs(q, db, [0, 2], [4, 0], metric=PT)
    assert s.tolist() == [-2.0, -90.5]


def pin_point_numpy_bruteforce(orc):
    """Against numpy's float64 pairwise distances (first index of the minimum), d = 1..4."""
    rng = np.random.default_rng(31)
    for d in (1, 2, 3, 4):
        A = rng.uniform(-3, 3, size=(29, d)).astype(np.float32)
        B = rng.uniform(-3, 3, size=(35, d)).astype(np.float32)
        idx, t1, t2 = orc.nn(A, B, metric=PT)
        D = ((A[:, None, :].astype(np.float64) - B[None, :, :].astype(np.float64)) ** 2).sum(-1)
        assert (idx == D.argmin(1)).all()
        Ds = np.sort(D, axis=1)
        assert np.abs(-t1 - Ds[:, 0]).max() < 1e-12 and np.abs(-t2 - Ds[:, 1]).max() < 1e-12


def pin_point_translation_invariance(orc):
    """Shifting both maps by the same vector changes no distance (integer coordinates,
    so every shifted value is exact)."""
    rng = np.random.default_rng(32)
    A = rng.integers(-100, 100, size=(40, 3)).astype(np.float32)
    B = rng.integers(-100, 100, size=(45, 3)).astype(np.float32)
    sh = np.array([1024, -2048, 512], np.float32)
    r0 = orc.nn(A, B, metric=PT)
    r1 = orc.nn(A + sh, B + sh, metric=PT)
    for a, b in zip(r0, r1):
        assert (a == b).all()


def pin_point_planted_closed_form(orc):
    """Noise-free planted pointmaps (X2[q] = X1[src(q)] exactly, distinct X1 points):
    M* = {(p, min{q : src(q) = p})}; the fast scheme at stride 1 returns the same set and
    every fast match (u, v) has u = src(v)."""
    p = workloads.make_pointmaps(14, 11, seed=33, warp="shift", sigma=0.0, rho=0.0)
    assert (p.D2 == p.D1[p.src]).all()
    first = {}
    for q, s in enumerate(p.src.tolist()):
        first.setdefault(s, q)
    expect = [list(e) for e in sorted(first.items())]
    assert orc.mutual_nn(p.D1, p.D2, metric=PT)[0].tolist() == expect
    assert orc.fast(p.D1, p.H, p.W, p.D2, 1, 0, 2, metric=PT)["pairs"].tolist() == expect
    for u, v in orc.fast(p.D1, p.H, p.W, p.D2, 3, 1, 10, metric=PT)["pairs"].tolist():
        assert p.src[v] == u


def pin_point_fast_invariants(orc):
    """Noisy, occluded pointmaps: fast matches are mutual, stride 1 is brute force, and the
    output equals the set characterisation walked from the NN maps."""
    p = workloads.make_pointmaps(18, 15, seed=34, warp="affine", sigma=0.02, rho=0.3)
    mset = _pairs_set(orc.mutual_nn(p.D1, p.D2, metric=PT)[0])
    assert len(mset) > 0
    assert _pairs_set(orc.fast(p.D1, p.H, p.W, p.D2, 1, 0, 3, metric=PT)["pairs"]) == mset
    n12 = orc.nn(p.D1, p.D2, metric=PT)[0]
    n21 = orc.nn(p.D2, p.D1, metric=PT)[0]
    for stride, off, T in ((4, 2, 1), (3, 1, 3), (5, 0, 10)):
        got = _pairs_set(orc.fast(p.D1, p.H, p.W, p.D2, stride, off, T, metric=PT)["pairs"])
        assert got <= mset
        assert got == _chain_set(n12, n21, _grid(p.H, p.W, stride, off), T)


def pin_point_clean_flag_relative(orc):
    """Noise-free planted pointmaps, stride 1, one iteration: a source pixel p is matched to
    its first preimage at distance 0.  The decision is a tie (margin 0, not clean) when p
    has two preimages, and otherwise has relative margin (d2 - 0) / d2 = 1 both ways, so
    it is clean even against eps = 0.5, which the squared distances themselves (< 0.5 m^2
    between neighbouring points here) would not pass."""
    p = workloads.make_pointmaps(12, 10, seed=35, warp="shift", sigma=0.0, rho=0.0)
    pre = {}
    for q, s_ in enumerate(p.src.tolist()):
        pre.setdefault(s_, []).append(q)
    r = orc.fast(p.D1, p.H, p.W, p.D2, 1, 0, 1, eps=0.5, metric=PT)
    got = {(int(u), int(v)): int(c) for (u, v), c in zip(r["pairs"].tolist(), r["clean"].tolist())}
    want = {(s_, qs[0]): int(len(qs) == 1) for s_, qs in pre.items()}
    assert got == want
    assert 0 < sum(want.values()) < len(want)


# ============================================================================ matching loss
# "MASt3R dissection", section 3: term (i, j) = log sum_k exp(<D1[i], D2[k]> / tau) - <D1[i], D2[j]> / tau.


def pin_infonce_closed_forms(orc):
    """Two database rows e0, e1 and the query e0 at tau = 0.5: the scores are 1 and 0, so the
    terms are softplus(-2) = log(1 + e^-2) for the true pair and softplus(2) for the other;
    identical database rows give log(n) whatever the query; a pair's term is never negative."""
    A = np.array([[1, 0], [0.6, 0.8]], np.float32)
    B = np.array([[1, 0], [0, 1]], np.float32)
    t, tot = orc.infonce(A, B, [[0, 0], [0, 1]], 0.5)
    assert abs(t[0] - math.log1p(math.exp(-2.0))) < 1e-13 and abs(t[1] - math.log1p(math.exp(2.0))) < 1e-13
    assert abs(tot - t.sum()) < 1e-13
    Bsame = np.tile(np.array([[0.6, 0.8]], np.float32), (7, 1))
    t2, _ = orc.infonce(A, Bsame, [[0, 3], [1, 6]], 0.1)
    assert np.abs(t2 - math.log(7)).max() < 1e-12
    assert (t >= 0).all() and (t2 >= 0).all()


def pin_infonce_scipy(orc):
    """Against scipy's log-sum-exp of numpy's float64 score matrix, several temperatures,
    including one small enough that exp(s / tau) overflows binary64 without a shift."""
    from scipy.special import logsumexp
    rng = np.random.default_rng(41)
    A = _rand_unit(rng, 23, 24).astype(np.float32)
    B = _rand_unit(rng, 31, 24).astype(np.float32)
    B[3:8] = A[:5]            # scores of about 1: exp(s / 0.001) overflows binary64 unshifted
    gt = np.stack([rng.integers(0, 23, 40), rng.integers(0, 31, 40)], 1).astype(np.int32)
    gt[:5, 0] = np.arange(5)
    S = A.astype(np.float64) @ B.astype(np.float64).T
    for tau in (1.0, 0.1, 0.001):
        t, tot = orc.infonce(A, B, gt, tau)
        ref = logsumexp(S[gt[:, 0]] / tau, axis=1) - S[gt[:, 0], gt[:, 1]] / tau
        assert np.abs(t - ref).max() < 1e-9 * max(1.0, np.abs(ref).max())
        assert abs(tot - ref.sum()) < 1e-9 * max(1.0, np.abs(ref).sum())


def pin_infonce_grad_finite_differences(orc):
    """Every component of both gradients against central differences of the oracle's own
    (pinned) loss: steps of 2^-14 are exact in fp32 for these inputs and the loss is
    binary64, so the difference quotient errs by about h^2 |L'''| / 6 (below 1e-6 here)."""
    rng = np.random.default_rng(43)
    A = _rand_unit(rng, 5, 4).astype(np.float32)
    B = _rand_unit(rng, 7, 4).astype(np.float32)
    gt = np.array([[0, 1], [2, 2], [2, 5], [4, 1], [1, 6]], np.int32)   # a repeated i and a repeated j
    h = 2.0 ** -14
    for tau in (0.5, 0.1):
        dA, dB, mass = orc.infonce_grad(A, B, gt, tau)
        for X, G in ((A, dA), (B, dB)):
            for r in range(X.shape[0]):
                for c in range(X.shape[1]):
                    v = X[r, c]
                    up, dn = np.float32(v + h), np.float32(v - h)
                    assert float(up) - float(v) == h and float(v) - float(dn) == h
                    X[r, c] = up
                    lp = orc.infonce(A, B, gt, tau)[1]
                    X[r, c] = dn
                    lm = orc.infonce(A, B, gt, tau)[1]
                    X[r, c] = v
                    fd = (lp - lm) / (2 * h)
                    assert abs(G[r, c] - fd) < 1e-6 * max(1.0, abs(fd)), (tau, r, c, G[r, c], fd)
        assert abs(mass.sum() - len(gt)) < 1e-12


def pin_infonce_grad_invariants(orc):
    """Each term's softmax sums to 1, so the image-2 gradient sums to zero over the rows and
    the column masses add up to the number of terms; scaling either map scales every score
    alike, so sum(dA * A) = sum(dB * B).  Listed rows of dB equal the full call's rows."""
    rng = np.random.default_rng(44)
    A = _rand_unit(rng, 30, 24).astype(np.float32)
    B = _rand_unit(rng, 40, 24).astype(np.float32)
    gt = np.stack([rng.integers(0, 30, 50), rng.integers(0, 40, 50)], 1).astype(np.int32)
    dA, dB, mass = orc.infonce_grad(A, B, gt, 0.1)
    assert np.abs(dB.sum(axis=0)).max() < 1e-10
    assert abs(mass.sum() - 50) < 1e-10
    lhs = float((dA * A.astype(np.float64)).sum())
    rhs = float((dB * B.astype(np.float64)).sum())
    assert abs(lhs - rhs) < 1e-9 * max(1.0, abs(lhs))
    untouched = np.setdiff1d(np.arange(30), gt[:, 0])
    assert (dA[untouched] == 0).all()
    rows = np.array([39, 3, 17], np.int32)
    _, dBr, mr = orc.infonce_grad(A, B, gt, 0.1, b_rows=rows)
    assert np.abs(dBr - dB[rows]).max() < 1e-12 and np.abs(mr - mass[rows]).max() < 1e-12


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]


def failing_pins(orc):
    bad = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except Exception:  # noqa: BLE001 -- any failure of a broken build counts
            bad.append(pin.__name__)
    return bad


if __name__ == "__main__":
    import oracle
    print(json.dumps(failing_pins(oracle.Oracle(sys.argv[1]))))
