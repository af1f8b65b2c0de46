"""The accuracy study's GPU runs against the oracle: on a pair small enough for the
oracle, every configuration's match set obeys the fast-scheme parity rules, and where
all of the oracle's decisions are clean the two studies report the same numbers."""
import time

import numpy as np
import pytest

import oracle
import workloads
from tests import checks

pytestmark = pytest.mark.gpu
pytest.importorskip("torch")
from dense_grounded_image_amd import study_accuracy as st  # noqa: E402


def oracle_matcher():
    """The study's matcher interface on the CPU oracle."""
    def fast(A, B, H, W, stride, offset, T):
        t = time.perf_counter()
        r = oracle.fast(A, H, W, B, stride, offset, T)
        return r["pairs"].astype(np.int64), time.perf_counter() - t
    return fast


def test_study_matches_oracle():
    H, W = 64, 48
    kw = dict(H=H, W=W, d=24, seed=3, strides=(1, 4, 8), iters=(1, 3, 10), sigmas=(0.1,), rhos=(0.2,))
    g = st.study(fast=st.gpu_matcher(), **kw)
    o = st.study(fast=oracle_matcher(), **kw)
    p = workloads.make_pair(H, W, 24, 3, warp="affine", sigma=0.1, rho=0.2)
    for rg, ro in zip(g, o):
        assert (rg["stride"], rg["T"]) == (ro["stride"], ro["T"])
        orc = oracle.fast(p.D1, H, W, p.D2, rg["stride"], rg["stride"] // 2, rg["T"])
        gp = st.gpu_matcher()(p.D1, p.D2, H, W, rg["stride"], rg["stride"] // 2, rg["T"])[0]
        rep = checks.check_fast(gp, orc, p.D1, p.D2, "f32")
        if rep["unclean_seeds"] == 0:
            assert rg["matches"] == ro["matches"] and rg["correct"] == ro["correct"]
