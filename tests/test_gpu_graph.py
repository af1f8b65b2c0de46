"""GPU: the fast scheme over a pair graph on one image collection equals the per-pair
call on each edge's two maps, and obeys the fast-scheme parity rules against the oracle."""
import numpy as np
import pytest

import oracle
import workloads
from tests import checks

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import dense_grounded_image_amd as mr  # noqa: E402

DEV = torch.device("cuda:0")


def log(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_graph_equals_per_pair_and_oracle(dtype):
    n, H, W = 6, 33, 29
    maps, bits, _ = workloads.make_collection(n, H, W, 24, seed=800, dtype=dtype)
    if bits is not None:
        imgs = torch.from_numpy(np.ascontiguousarray(bits).reshape(n, H, W, 24)).view(torch.bfloat16).to(DEV)
    else:
        imgs = torch.from_numpy(maps.reshape(n, H, W, 24)).to(DEV)
    edges = workloads.all_edges(n)
    edges = np.concatenate([edges, edges[::-1, ::-1], [[2, 2]]]).astype(np.int32)   # both orders, a self-pair
    pairs, npairs, act = mr.fast_reciprocal_graph(imgs, edges, 4, 2, 6)
    torch.cuda.synchronize()
    for e, (i, j) in enumerate(edges.tolist()):
        got = mr.matches(pairs, npairs, e)
        rp, rn, ra = mr.fast_reciprocal(imgs[i], imgs[j], 4, 2, 6)
        assert got.tolist() == mr.matches(rp, rn).tolist(), (e, i, j)
        assert act[e].cpu().tolist() == ra[0].cpu().tolist()
        if e % 5 == 0:
            orc = oracle.fast(maps[i], H, W, maps[j], 4, 2, 6)
            rep = checks.check_fast(got, orc, maps[i], maps[j], dtype, gpu_active=act[e].cpu().numpy())
            log("graph edge", e, i, j, rep)


def test_graph_full_size_sampled():
    """8 images of 512x384 fp32, all 28 edges: three edges against the per-pair call, and
    one of them against a full oracle run."""
    n, H, W = 8, 512, 384
    maps, _, _ = workloads.make_collection(n, H, W, 24, seed=801)
    imgs = torch.from_numpy(maps.reshape(n, H, W, 24)).to(DEV)
    edges = workloads.all_edges(n)
    pairs, npairs, act = mr.fast_reciprocal_graph(imgs, edges, 8, 4, 10)
    torch.cuda.synchronize()
    for e in (0, 13, len(edges) - 1):
        i, j = edges[e]
        rp, rn, _ = mr.fast_reciprocal(imgs[i], imgs[j], 8, 4, 10)
        assert mr.matches(pairs, npairs, e).tolist() == mr.matches(rp, rn).tolist()
    # one full-size edge against a full oracle run
    e = 13
    i, j = edges[e]
    orc = oracle.fast(maps[i], H, W, maps[j], 8, 4, 10)
    rep = checks.check_fast(mr.matches(pairs, npairs, e), orc, maps[i], maps[j], "f32",
                            gpu_active=act[e].cpu().numpy())
    log("graph 8x512x384", [int(x) for x in npairs.cpu()[:5]], "edge", e, rep)
