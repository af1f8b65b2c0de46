"""Randomised property tests of the oracle (CPU only).

Hypothesis draws small maps and scheme parameters; every example is checked against
facts that do not come from the oracle's own code:

- NN and mutual NN against numpy's binary64 similarity matrix, whose argmax takes the
  first (lowest-index) maximum ("MASt3R dissection", section 3: NN as the argmax of
  the descriptor inner product; the mutual set of section 1);
- the fast scheme ("DUSt3R and MASt3R explained", the fast reciprocal matching
  paragraph) against a hand walk of every seed's chain over those numpy NN maps, and
  against the invariants that follow from it: the output is a subset of the mutual set
  and one-to-one (I1, I2); stride 1 reduces it to brute force (I3); the kept set only
  grows with the iteration budget and every chain climbs in score (I4); it equals the
  set of fixed points reached from a seed within T - 1 steps (I5); on a noise-free
  planted field every match follows the planted correspondence (I6); T = 0 gives
  nothing and a stride beyond the image leaves one seed (I7).

Two value families: unit rows with continuous components (generic, no ties), and rows
of small dyadic components (exact binary64 arithmetic in any summation order, so
numpy and the oracle agree bit for bit, with frequent exact ties and duplicate rows).
The runs are derandomised, so every run draws the same examples.
"""
from __future__ import annotations

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import workloads
from tests import pins

SETTINGS = dict(deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])


def _rows(rng, n, d, kind):
    if kind == "unit":
        return workloads.unit_rows(rng, n, d).astype(np.float32)
    # components in {-1, -1/2, 0, 1/2, 1}, drawn from a small pool of rows so that
    # duplicates (exact ties) are common
    pool = rng.integers(-2, 3, size=(max(1, n // 2), d)).astype(np.float32) / 2
    return pool[rng.integers(0, pool.shape[0], size=n)]


@st.composite
def problems(draw):
    h1, w1 = draw(st.integers(1, 9)), draw(st.integers(1, 9))
    h2, w2 = draw(st.integers(1, 9)), draw(st.integers(1, 9))
    d = draw(st.sampled_from([1, 2, 3, 8, 24]))
    kind = draw(st.sampled_from(["unit", "dyadic"]))
    seed = draw(st.integers(0, 2**31 - 1))
    rng = np.random.Generator(np.random.PCG64(seed))
    A = _rows(rng, h1 * w1, d, kind)
    B = _rows(rng, h2 * w2, d, kind)
    stride = draw(st.integers(1, 6))
    offset = draw(st.integers(0, stride - 1))
    T = draw(st.integers(0, 6))
    return dict(A=A, B=B, H=h1, W=w1, stride=stride, offset=offset, T=T, kind=kind)


def _pairs(p):
    return {(int(a), int(b)) for a, b in np.asarray(p).reshape(-1, 2)}


def _numpy_maps(A, B):
    n12, m12 = pins._numpy_nn(A, B)
    n21, m21 = pins._numpy_nn(B, A)
    return n12, m12, n21, m21


def _numpy_mutual(n12, n21):
    return {(i, int(n12[i])) for i in range(len(n12)) if int(n21[n12[i]]) == i}


@settings(max_examples=400, **SETTINGS)
@given(problems())
def test_nn_and_mutual_against_numpy(pb):
    orc = oracle.Oracle()
    A, B = pb["A"], pb["B"]
    S = A.astype(np.float64) @ B.astype(np.float64).T
    idx, t1, t2 = orc.nn(A, B)
    assert idx.tolist() == S.argmax(1).tolist()
    tol = 0.0 if pb["kind"] == "dyadic" else 1e-12
    np.testing.assert_allclose(t1, S.max(1), rtol=0, atol=tol)
    if S.shape[1] > 1:
        np.testing.assert_allclose(t2, np.sort(S, 1)[:, -2], rtol=0, atol=tol)
    n12, _, n21, _ = _numpy_maps(A, B)
    m = orc.mutual_nn(A, B)[0]
    assert _pairs(m) == _numpy_mutual(n12, n21)
    # symmetric in the maps' roles; one-to-one
    assert _pairs(orc.mutual_nn(B, A)[0]) == {(v, u) for u, v in _pairs(m)}
    assert len({u for u, _ in _pairs(m)}) == len({v for _, v in _pairs(m)}) == len(m)


@settings(max_examples=500, **SETTINGS)
@given(problems())
def test_fast_scheme_properties(pb):
    orc = oracle.Oracle()
    A, B, H, W = pb["A"], pb["B"], pb["H"], pb["W"]
    s, o, T = pb["stride"], pb["offset"], pb["T"]
    n12, m12, n21, m21 = _numpy_maps(A, B)
    seeds = pins._grid(H, W, s, o)
    r = orc.fast(A, H, W, B, s, o, T)
    got = _pairs(r["pairs"])
    # the output is sorted by u
    assert [int(u) for u, _ in r["pairs"]] == sorted(int(u) for u, _ in r["pairs"])
    # I5: the fixed points reached from a seed within T - 1 steps of f = NN21 o NN12
    assert got == pins._chain_set(n12, n21, seeds, T)
    # I1, I2: a subset of the mutual set, one-to-one
    assert got <= _numpy_mutual(n12, n21)
    assert len({u for u, _ in got}) == len({v for _, v in got}) == len(got)
    # I4: one more iteration keeps every pair
    assert got <= _pairs(orc.fast(A, H, W, B, s, o, T + 1)["pairs"])
    # per-seed records and first visits against the hand walk
    ends, cleans, fresh = pins._walk_seed_records(n12, m12, n21, m21, seeds, T, 1e-5)
    assert r["seed_u"].tolist() == ends
    assert r["seed_clean"].tolist() == cleans
    assert r["fresh"].tolist() == fresh
    # I7 and the live counts: T = 0 gives nothing; iteration 0 holds every seed; the
    # live set never grows
    if T == 0:
        assert len(got) == 0
    else:
        a = r["active"].tolist()
        assert a[0] == len(seeds)
        assert all(a[t + 1] <= a[t] for t in range(T - 1))


@settings(max_examples=300, **SETTINGS)
@given(problems())
def test_fast_chains_climb(pb):
    """I4: along every chain s(u_t, v_t) <= s(u_t+1, v_t) <= s(u_t+1, v_t+1), and no chain
    revisits a pixel before it converges (lowest-index ties rule out cycles)."""
    A, B = pb["A"], pb["B"]
    S = A.astype(np.float64) @ B.astype(np.float64).T
    n12, _, n21, _ = _numpy_maps(A, B)
    for u0 in range(A.shape[0]):
        u, seen = u0, set()
        while True:
            v = int(n12[u])
            u2 = int(n21[v])
            assert S[u, v] <= S[u2, v]
            if u2 == u:
                break
            assert S[u2, v] <= S[u2, int(n12[u2])]
            assert u not in seen
            seen.add(u)
            u = u2


@settings(max_examples=150, **SETTINGS)
@given(problems())
def test_fast_stride1_is_bruteforce(pb):
    """I3: seeding every pixel returns exactly the mutual set for any T >= 1."""
    orc = oracle.Oracle()
    A, B, H, W = pb["A"], pb["B"], pb["H"], pb["W"]
    T = max(1, pb["T"])
    n12, _, n21, _ = _numpy_maps(A, B)
    assert _pairs(orc.fast(A, H, W, B, 1, 0, T)["pairs"]) == _numpy_mutual(n12, n21)


@settings(max_examples=150, **SETTINGS)
@given(problems(), st.integers(10, 40))
def test_fast_single_seed_beyond_stride(pb, stride):
    """I7: a stride at least the image size leaves the one seed at the offset."""
    orc = oracle.Oracle()
    A, B, H, W = pb["A"], pb["B"], pb["H"], pb["W"]
    T = max(1, pb["T"])
    r = orc.fast(A, H, W, B, stride, 0, T)
    assert r["active"][0] == 1
    n12, _, n21, _ = _numpy_maps(A, B)
    assert _pairs(r["pairs"]) == pins._chain_set(n12, n21, [0], T)


@settings(max_examples=100, **SETTINGS)
@given(st.integers(2, 14), st.integers(2, 14), st.sampled_from(["shift", "affine", "identity"]),
       st.integers(0, 2**31 - 1), st.integers(1, 5), st.integers(1, 6))
def test_fast_planted_noise_free(H, W, warp, seed, stride, T):
    """I6: on a noise-free planted field every match (u, v) has u = src(v), and a seed that
    is a source pixel converges in the first iteration to the lowest pixel planted from
    it."""
    orc = oracle.Oracle()
    p = workloads.make_pair(H, W, 24, seed=seed, warp=warp, sigma=0.0, rho=0.0)
    off = stride // 2
    r = orc.fast(p.D1, H, W, p.D2, stride, off, T)
    for u, v in r["pairs"].tolist():
        assert p.src[v] == u
    first = {}
    for q, s in enumerate(p.src.tolist()):
        first.setdefault(s, q)
    r1 = orc.fast(p.D1, H, W, p.D2, stride, off, 1)
    assert _pairs(r1["pairs"]) == {(s, first[s]) for s in pins._grid(H, W, stride, off) if s in first}


def test_properties_reject_a_planted_mistake():
    """The hand walk is sharp enough to see an off-by-one iteration budget: running the
    oracle with T + 1 iterations disagrees with the T-iteration walk on some example."""
    rng = np.random.Generator(np.random.PCG64(5))
    found = False
    for _ in range(50):
        A = _rows(rng, 36, 3, "unit")
        B = _rows(rng, 36, 3, "unit")
        n12, _, n21, _ = _numpy_maps(A, B)
        seeds = pins._grid(6, 6, 3, 1)
        r = oracle.Oracle().fast(A, 6, 6, B, 3, 1, 2)
        if _pairs(r["pairs"]) != pins._chain_set(n12, n21, seeds, 1):
            found = True
            break
    assert found
