"""The fast-scheme parity rules (tests/checks.py) catch the mistakes they are meant to.

Stand-in "GPU" outputs are made on the CPU from oracle runs: the correct output
passes; one iteration too many, an extra seed row, a dropped pair, and a live
count one iteration off each fail.  The planted mistakes live in these inputs,
never in the library."""
import numpy as np
import pytest

import oracle
import workloads
from tests import checks


def _pair():
    # 40x32 shift pair: at T = 1 about half the seeds are still live, so one more
    # iteration adds pairs; every chain is clean
    return workloads.make_pair(40, 32, 24, seed=61, warp="affine", sigma=0.15, rho=0.3)


def test_correct_output_passes():
    p = _pair()
    for T in (1, 2, 10):
        orc = oracle.fast(p.D1, p.H, p.W, p.D2, 4, 2, T)
        assert orc["seed_clean"].all()
        rep = checks.check_fast(orc["pairs"], orc, p.D1, p.D2, "f32", gpu_active=orc["fresh"])
        assert rep["gpu_only"] == rep["oracle_only"] == 0


def test_one_iteration_too_many_fails():
    p = _pair()
    o1 = oracle.fast(p.D1, p.H, p.W, p.D2, 4, 2, 1)
    o2 = oracle.fast(p.D1, p.H, p.W, p.D2, 4, 2, 2)
    assert len(o2["pairs"]) > len(o1["pairs"])
    with pytest.raises(AssertionError, match="every chain is clean"):
        checks.check_fast(o2["pairs"], o1, p.D1, p.D2, "f32")


def test_extra_seed_row_fails():
    p = _pair()
    orc = oracle.fast(p.D1, p.H, p.W, p.D2, 4, 2, 10)
    more = oracle.fast(p.D1, p.H, p.W, p.D2, 2, 0, 10)     # a denser grid: extra, genuinely mutual pairs
    extra = sorted({tuple(x) for x in more["pairs"].tolist()} | {tuple(x) for x in orc["pairs"].tolist()})
    assert len(extra) > len(orc["pairs"])
    with pytest.raises(AssertionError, match="every chain is clean"):
        checks.check_fast(np.array(extra), orc, p.D1, p.D2, "f32")


def test_dropped_pair_fails():
    p = _pair()
    orc = oracle.fast(p.D1, p.H, p.W, p.D2, 4, 2, 10)
    with pytest.raises(AssertionError, match="clean oracle pairs missing"):
        checks.check_fast(orc["pairs"][1:], orc, p.D1, p.D2, "f32")


def test_live_count_off_by_one_iteration_fails():
    p = _pair()
    orc = oracle.fast(p.D1, p.H, p.W, p.D2, 4, 2, 10)
    shifted = np.concatenate([orc["fresh"][:1], orc["fresh"][:-1]])
    with pytest.raises(AssertionError, match="live counts"):
        checks.check_fast(orc["pairs"], orc, p.D1, p.D2, "f32", gpu_active=shifted)


def test_unclean_chains_bound_the_difference():
    """With a coarse margin many chains are unclean; a stand-in output that differs by
    more pairs than there are unclean chains fails, one within the bound passes."""
    p = _pair()
    orc = oracle.fast(p.D1, p.H, p.W, p.D2, 4, 2, 10, eps=0.02)
    unclean = int((orc["seed_clean"] == 0).sum())
    assert 0 < unclean < len(orc["pairs"])
    dirty = [tuple(x) for x, c in zip(orc["pairs"].tolist(), orc["clean"]) if not c]
    kept = sorted(set(map(tuple, orc["pairs"].tolist())) - set(dirty[:1]))
    checks.check_fast(np.array(kept), orc, p.D1, p.D2, "f32")
    more = oracle.fast(p.D1, p.H, p.W, p.D2, 1, 0, 1)      # the whole mutual set
    big = sorted({tuple(x) for x in more["pairs"].tolist()})
    assert len(set(big) - set(map(tuple, orc["pairs"].tolist()))) > unclean
    with pytest.raises(AssertionError, match="GPU-only pairs"):
        checks.check_fast(np.array(big), orc, p.D1, p.D2, "f32")


def test_rule_counts_report_each_planted_mistake():
    """The counted form of the rules (used in the benchmark's report) counts every item:
    all pass on the oracle's own output, and each planted mistake shows up in its rule
    with the right number of failing items."""
    p = _pair()
    orc = oracle.fast(p.D1, p.H, p.W, p.D2, 4, 2, 10)
    n = len(orc["pairs"])
    R, s = checks.fast_rule_counts(orc["pairs"], orc, p.D1, p.D2, "f32", gpu_active=orc["fresh"])
    assert all(r["failed"] == 0 for r in R.values()), R
    assert R["i_clean_pairs_found"]["passed"] == R["ii_eps_reciprocal"]["passed"] == n
    assert R["iv_equal_sets"]["passed"] == n and R["iv_live_counts"]["passed"] == 10
    assert R["iii_ascending_in_u"]["passed"] == n - 1 and R["iii_v_used_once"]["passed"] == n
    # two pairs dropped: (i) and (iv) fail by two, nothing else
    R, _ = checks.fast_rule_counts(orc["pairs"][2:], orc, p.D1, p.D2, "f32")
    assert R["i_clean_pairs_found"]["failed"] == 2 and R["iv_equal_sets"]["failed"] == 2
    assert R["i_clean_pairs_found"]["examples"] == sorted(map(list, orc["pairs"][:2].tolist()))
    assert R["ii_eps_reciprocal"]["failed"] == 0 and R["iv_live_counts"]["failed"] == 0
    # a pair that is not mutual, placed out of order, and reusing a pixel of image 2
    v0 = int(orc["pairs"][0, 1])
    used_u = set(orc["pairs"][:, 0].tolist())
    free_u = next(x for x in range(p.N) if x not in used_u)   # below the last u: out of order
    assert free_u < orc["pairs"][-1, 0]
    bad = np.concatenate([orc["pairs"], [[free_u, v0]]])
    R, _ = checks.fast_rule_counts(bad, orc, p.D1, p.D2, "f32")
    assert R["iii_v_used_once"]["failed"] == 1 and R["iii_v_used_once"]["examples"] == [[v0]]
    assert R["iii_ascending_in_u"]["failed"] == 1
    assert R["ii_eps_reciprocal"]["failed"] >= 1
    # live counts one iteration off: the iterations whose counts differ
    shifted = np.concatenate([orc["fresh"][:1], orc["fresh"][:-1]])
    R, _ = checks.fast_rule_counts(orc["pairs"], orc, p.D1, p.D2, "f32", gpu_active=shifted)
    diff = int((shifted != orc["fresh"]).sum())
    assert diff > 0 and R["iv_live_counts"]["failed"] == diff
