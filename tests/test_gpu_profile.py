"""The measurement aid's per-launch query counts on the fast scheme.

Over one call, the forward launches must count the live pixels of each iteration, and
the backward launches the pixels of image 2 first reached in that iteration (the
backward NN of a pixel is searched once per call: "DUSt3R and MASt3R explained", the
fast reciprocal matching paragraph, with NN fixed per pixel, "MASt3R dissection",
section 3). The expected counts come from a walk over the oracle's NN; their total must
equal the number of distinct NN queries the oracle itself makes on the same pair.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.pins import _grid

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import dense_grounded_image_amd as mr  # noqa: E402

DEV = torch.device("cuda:0")


def _walk_counts(p):
    """Per iteration: live pixels, and pixels of image 2 landed on for the first time."""
    seeds = np.array(_grid(p.H, p.W, p.stride, p.offset), np.int32)
    visited = np.zeros(p.N, bool)
    visited[seeds] = True
    live, seen_v = seeds, set()
    fwd, bwd = [], []
    for _ in range(p.max_iters):
        fwd.append(len(live))
        if len(live) == 0:
            bwd.append(0)
            continue
        v = oracle.nn_rows(p.D1, live, p.D2)[0].astype(np.int64)
        new = sorted(set(v.tolist()) - seen_v)
        bwd.append(len(new))
        seen_v.update(new)
        uniq = np.unique(v)
        u2 = dict(zip(uniq.tolist(), oracle.nn_rows(p.D2, uniq.astype(np.int32), p.D1)[0].tolist()))
        nxt = []
        for u, x in zip(live.tolist(), v.tolist()):
            w = u2[x]
            if w != u and not visited[w]:
                visited[w] = True
                nxt.append(w)
        live = np.array(sorted(nxt), np.int32)
    return fwd, bwd


@pytest.mark.parametrize("seed", [0, 5])
def test_profile_counts_the_queries_each_launch_searched(seed):
    p = workloads.make_pair(64, 48, 24, seed=seed, warp="shift", sigma=0.1, rho=0.2, stride=8, max_iters=10) \
        if seed else workloads.config_pair(0)
    A = torch.from_numpy(p.D1.reshape(1, p.H, p.W, p.d)).to(DEV)
    B = torch.from_numpy(p.D2.reshape(1, p.H, p.W, p.d)).to(DEV)
    f = mr.FastReciprocal(A, B, p.stride, p.offset, p.max_iters)
    f(A, B)
    torch.cuda.synchronize()
    mr.profile_begin(64)
    _, _, act = f(A, B)
    torch.cuda.synchronize()
    _, n, each, qs = mr.profile_end_queries(64)
    assert n == 2 * p.max_iters and len(qs) == n and all(t >= 0 for t in each)
    fwd, bwd = _walk_counts(p)
    assert qs[0::2] == act[0].cpu().tolist() == fwd
    assert qs[1::2] == bwd
    r = oracle.fast(p.D1, p.H, p.W, p.D2, p.stride, p.offset, p.max_iters)
    assert sum(qs) == r["nn_queries"]
    assert sum(bwd) < sum(fwd)   # pixels of image 2 are reached more than once


def test_profile_counts_sum_over_the_batch():
    small = [workloads.make_pair(48, 40, 24, seed=70 + b, warp="affine", sigma=0.15, rho=0.3, stride=4,
                                 max_iters=6) for b in range(3)]
    A = torch.from_numpy(np.stack([q.D1.reshape(q.H, q.W, q.d) for q in small])).to(DEV)
    B = torch.from_numpy(np.stack([q.D2.reshape(q.H, q.W, q.d) for q in small])).to(DEV)
    q0 = small[0]
    f = mr.FastReciprocal(A, B, q0.stride, q0.offset, q0.max_iters)
    mr.profile_begin(32)
    _, _, act = f(A, B)
    torch.cuda.synchronize()
    _, n, _, qs = mr.profile_end_queries(32)
    walks = [_walk_counts(q) for q in small]
    assert qs[0::2] == [sum(w[0][t] for w in walks) for t in range(q0.max_iters)]
    assert qs[1::2] == [sum(w[1][t] for w in walks) for t in range(q0.max_iters)]
    assert act.sum(0).cpu().tolist() == qs[0::2]
