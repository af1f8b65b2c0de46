"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Small and medium cases are compared in full (every NN, every pair), with ragged
sizes that span several 16-row tiles and a partial last tile.  The workloads at
full size are checked on sampled outputs the oracle can compute one by one and
through properties that hold at any size (rules in tests/checks.py).
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads
from tests import checks
from tests.pins import _load_golden

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import dense_grounded_image_amd as mr  # noqa: E402

DEV = torch.device("cuda:0")


def log(*a):
    print(*a, flush=True)


def dev_map(arr, H, W, bits=None):
    """numpy [N, d] fp32 (or bf16 bit patterns) -> device tensor [H, W, d]."""
    if bits is not None:
        t = torch.from_numpy(np.ascontiguousarray(bits).reshape(H, W, -1)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32).reshape(H, W, -1))
    return t.to(DEV)


def pair_maps(p):
    return dev_map(p.D1, p.H, p.W, p.D1_bits), dev_map(p.D2, p.H, p.W, p.D2_bits)


def seeds_of(H, W, stride, offset):
    return [y * W + x for y in range(offset, H, stride) for x in range(offset, W, stride)]


# ============================================================================ NN argmax

@pytest.mark.parametrize("dtype,d", [("f32", 24), ("bf16", 24), ("f32", 1), ("f32", 3), ("f32", 17),
                                     ("f32", 64), ("bf16", 8), ("bf16", 64), ("f32", 8), ("f32", 16),
                                     ("f32", 32)])
def test_nn_argmax_ragged(dtype, d):
    """All queries, 37x29 against 41x23 pixels (neither a multiple of the 32-row tile).
    fp32 maps with d = 8, 16, 24, 32 take the exact three-way bf16 split (three query
    tiles per wave, two at d = 32), the others fp32 products."""
    rng = np.random.default_rng(100 + d)
    p = workloads.make_pair(37, 29, d, seed=100 + d, warp="shift", sigma=0.1, rho=0.2, dtype=dtype)
    q = workloads.make_pair(41, 23, d, seed=200 + d, warp="shift", sigma=0.1, rho=0.2, dtype=dtype)
    A = dev_map(p.D1, p.H, p.W, p.D1_bits)
    B = dev_map(q.D2, q.H, q.W, q.D2_bits)
    gi, gs = mr.nn_argmax(A, B, with_score=True)
    torch.cuda.synchronize()
    oi, o1, o2 = oracle.nn(p.D1, q.D2)
    rep = checks.check_nn(gi.cpu().numpy(), oi, o1, o2, p.D1, np.arange(p.N), q.D2, dtype)
    # the reported score is the GPU's fp32 similarity of its own choice
    s = oracle.similarity_pairs(p.D1, q.D2, np.arange(p.N), gi.cpu().numpy())
    assert np.abs(gs.cpu().numpy().astype(np.float64) - s).max() < 3e-6
    log("nn", dtype, d, rep)
    del rng


def test_nn_argmax_query_list_batch():
    """Batched maps, explicit query lists with repeats and out-of-order ids."""
    B_, H, W, d = 3, 19, 21, 24
    ps = [workloads.make_pair(H, W, d, seed=300 + b, warp="shift", sigma=0.1, rho=0.2) for b in range(B_)]
    A = torch.stack([dev_map(p.D1, H, W) for p in ps])
    Bm = torch.stack([dev_map(p.D2, H, W) for p in ps])
    rng = np.random.default_rng(7)
    rows = rng.integers(0, H * W, size=(B_, 150)).astype(np.int32)
    rows[:, 5] = rows[:, 6]
    gi = mr.nn_argmax(A, Bm, q_idx=torch.from_numpy(rows))
    torch.cuda.synchronize()
    gi = gi.cpu().numpy()
    for b, p in enumerate(ps):
        oi, o1, o2 = oracle.nn_rows(p.D1, rows[b], p.D2)
        checks.check_nn(gi[b], oi, o1, o2, p.D1, rows[b], p.D2, "f32")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_batch16_xcd_packed_grid(dtype):
    """16 pairs of ragged 37x29 maps in one call.  Each pair then gets only a few dozen
    workgroups, so the search runs on the one-dimensional grid that keeps a pair's
    workgroups on one XCD.  Every pair's NN map and fast-scheme output against the
    oracle, and three pairs equal to single-pair calls."""
    B_, d, s, o, T = 16, 24, 4, 2, 6
    ps = [workloads.make_pair(37, 29, d, seed=900 + b, warp="shift", sigma=0.1, rho=0.2, dtype=dtype)
          for b in range(B_)]
    A = torch.stack([dev_map(p.D1, p.H, p.W, p.D1_bits) for p in ps])
    Bm = torch.stack([dev_map(p.D2, p.H, p.W, p.D2_bits) for p in ps])
    gi = mr.nn_argmax(A, Bm)
    fp, fn, act = mr.fast_reciprocal(A, Bm, s, o, T)
    torch.cuda.synchronize()
    gi = gi.cpu().numpy()
    for b, p in enumerate(ps):
        oi, o1, o2 = oracle.nn(p.D1, p.D2)
        checks.check_nn(gi[b], oi, o1, o2, p.D1, np.arange(p.N), p.D2, dtype)
        orc = oracle.fast(p.D1, p.H, p.W, p.D2, s, o, T)
        checks.check_fast(mr.matches(fp, fn, b), orc, p.D1, p.D2, dtype, gpu_active=act[b].cpu().numpy())
    for b in (0, 9, 15):
        sp, sn, _ = mr.fast_reciprocal(A[b], Bm[b], s, o, T)
        assert mr.matches(sp, sn).tolist() == mr.matches(fp, fn, b).tolist()
    log("batch16", dtype, [int(x) for x in fn.cpu()][:4], "...")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("db_hw", [(64, 48), (50, 60)])
def test_nn_argmax_query_counts_across_modes(dtype, db_hw):
    """Query lists of 1 .. 545 rows against a database of whole 32-row tiles (64x48)
    or with a ragged last tile (50x60): fewer query tiles than waves (the per-wave
    mode), one partial or full query group (the general mode; for bf16 the register
    stream with zero operands in empty slots), and two groups."""
    d = 24
    p = workloads.make_pair(64, 48, d, seed=41, warp="shift", sigma=0.1, rho=0.2, dtype=dtype)
    q = workloads.make_pair(db_hw[0], db_hw[1], d, seed=42, warp="shift", sigma=0.1, rho=0.2, dtype=dtype)
    A = dev_map(p.D1, p.H, p.W, p.D1_bits)
    B = dev_map(q.D2, q.H, q.W, q.D2_bits)
    rng = np.random.default_rng(43)
    for n in (1, 33, 96, 97, 127, 200, 385, 480, 512, 545):
        rows = rng.integers(0, p.N, size=n).astype(np.int32)
        gi = mr.nn_argmax(A, B, q_idx=torch.from_numpy(rows).to(DEV))
        torch.cuda.synchronize()
        oi, o1, o2 = oracle.nn_rows(p.D1, rows, q.D2)
        rep = checks.check_nn(gi.cpu().numpy(), oi, o1, o2, p.D1, rows, q.D2, dtype)
        log("query count", dtype, db_hw, n, rep)


def test_scores_bitwise_symmetric():
    """For every mutual pair the forward and backward searches report the same fp32 score
    bit for bit: the similarity does not depend on which map is the query side."""
    for dtype in ("f32", "bf16"):
        p = workloads.make_pair(48, 40, 24, seed=400, warp="affine", sigma=0.15, rho=0.3, dtype=dtype)
        A, B = pair_maps(p)
        i12, s12 = mr.nn_argmax(A, B, with_score=True)
        i21, s21 = mr.nn_argmax(B, A, with_score=True)
        torch.cuda.synchronize()
        i12, s12, i21, s21 = (x.cpu().numpy() for x in (i12, s12, i21, s21))
        u = np.nonzero(i21[i12] == np.arange(p.N))[0]
        assert len(u) > 100
        assert (s12[u].view(np.uint32) == s21[i12[u]].view(np.uint32)).all()


# ============================================================================ mutual NN

@pytest.mark.parametrize("H,W,dtype", [(64, 48, "f32"), (37, 29, "f32"), (33, 50, "bf16")])
def test_mutual_full(H, W, dtype):
    p = workloads.make_pair(H, W, 24, seed=500 + H, warp="shift", sigma=0.1, rho=0.2, dtype=dtype)
    A, B = pair_maps(p)
    pairs, n, nn_ab, nn_ba = mr.mutual_nn(A, B)
    torch.cuda.synchronize()
    o_pairs, o12, a1, a2, o21, b1, b2 = oracle.mutual_nn(p.D1, p.D2)
    checks.check_nn(nn_ab[0].cpu().numpy(), o12, a1, a2, p.D1, np.arange(p.N), p.D2, dtype)
    checks.check_nn(nn_ba[0].cpu().numpy(), o21, b1, b2, p.D2, np.arange(p.N), p.D1, dtype)
    gp = mr.matches(pairs, n)
    checks.check_one_to_one_sorted(gp)
    # the pair list is exactly the reciprocal subset of the GPU's own NN maps
    g12, g21 = nn_ab[0].cpu().numpy(), nn_ba[0].cpu().numpy()
    i = np.nonzero(g21[g12] == np.arange(p.N))[0]
    assert (gp[:, 0] == i).all() and (gp[:, 1] == g12[i]).all()
    clean = (a1 - a2 > checks.MARGIN) & (b1[o12] - b2[o12] > checks.MARGIN)
    if clean.all():
        assert gp.tolist() == o_pairs.tolist()
    log("mutual", H, W, dtype, len(gp), len(o_pairs))


@pytest.mark.parametrize("H,W,dtype", [(40, 35, "f32"), (40, 35, "bf16"), (64, 64, "bf16")])
def test_mutual_planted_noise_free_ties(H, W, dtype):
    """Noise-free planted field: clamped borders duplicate descriptors exactly, so the
    lowest-index tie-break decides; the result is the closed form.  For bf16 the ties go
    through the tile-level search and the row recovery; 64x64 (whole query groups, no
    ragged tile) takes the direct-load stream, 40x35 the staged one."""
    p = workloads.make_pair(H, W, 24, seed=600, warp="shift", sigma=0.0, rho=0.0, dtype=dtype)
    A, B = pair_maps(p)
    pairs, n, _, _ = mr.mutual_nn(A, B)
    torch.cuda.synchronize()
    first = {}
    for q, s in enumerate(p.src.tolist()):
        first.setdefault(s, q)
    assert mr.matches(pairs, n).tolist() == [list(x) for x in sorted(first.items())]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nn_all_scores_negative(dtype):
    """Every similarity negative (the maps point into opposite half-spaces): the integer
    key order does not hold there, so this takes the exact fallback (fp32) and the
    float comparisons of the tile-level search and the row recovery (bf16)."""
    rng = np.random.default_rng(5)
    d, (h1, w1), (h2, w2) = 24, (37, 29), (41, 23)
    e = np.zeros(d)
    e[0] = 1.0

    def unit(x):
        return (x / np.linalg.norm(x, axis=1, keepdims=True)).astype(np.float32)

    A = unit(0.9 * e + 0.25 * rng.standard_normal((h1 * w1, d)) / np.sqrt(d))
    B = unit(-0.9 * e + 0.25 * rng.standard_normal((h2 * w2, d)) / np.sqrt(d))
    Ab = Bb = None
    if dtype == "bf16":
        Ab, Bb = workloads.f32_to_bf16_bits(A), workloads.f32_to_bf16_bits(B)
        A, B = workloads.bf16_bits_to_f32(Ab), workloads.bf16_bits_to_f32(Bb)
    gi, gs = mr.nn_argmax(dev_map(A, h1, w1, Ab), dev_map(B, h2, w2, Bb), with_score=True)
    torch.cuda.synchronize()
    oi, o1, o2 = oracle.nn(A, B)
    assert o1.max() < 0
    rep = checks.check_nn(gi.cpu().numpy(), oi, o1, o2, A, np.arange(len(A)), B, dtype)
    s = oracle.similarity_pairs(A, B, np.arange(len(A)), gi.cpu().numpy())
    assert np.abs(gs.cpu().numpy().astype(np.float64) - s).max() < 3e-6
    log("negative", dtype, rep)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nn_mixed_sign_best_scores(dtype):
    """Full query groups (64x48 queries against a 64x48 map) where every other row of
    image 1 points away from all of image 2 (best score negative) and the rest toward
    it: one workgroup holds lanes of both kinds, so the keyed search, its exact
    fallback and the tile epilogue run one unit behind the products all meet."""
    rng = np.random.default_rng(15)
    d, (h, w) = 24, (64, 48)
    e = np.zeros(d)
    e[0] = 1.0

    def unit(x):
        return (x / np.linalg.norm(x, axis=1, keepdims=True)).astype(np.float32)

    sign = np.where(np.arange(h * w) % 2 == 0, 1.0, -1.0)[:, None]
    A = unit(sign * 0.9 * e + 0.25 * rng.standard_normal((h * w, d)) / np.sqrt(d))
    B = unit(0.9 * e + 0.25 * rng.standard_normal((h * w, d)) / np.sqrt(d))
    Ab = Bb = None
    if dtype == "bf16":
        Ab, Bb = workloads.f32_to_bf16_bits(A), workloads.f32_to_bf16_bits(B)
        A, B = workloads.bf16_bits_to_f32(Ab), workloads.bf16_bits_to_f32(Bb)
    gi, gs = mr.nn_argmax(dev_map(A, h, w, Ab), dev_map(B, h, w, Bb), with_score=True)
    torch.cuda.synchronize()
    oi, o1, o2 = oracle.nn(A, B)
    assert o1[1::2].max() < 0 < o1[0::2].min()
    rep = checks.check_nn(gi.cpu().numpy(), oi, o1, o2, A, np.arange(len(A)), B, dtype)
    s = oracle.similarity_pairs(A, B, np.arange(len(A)), gi.cpu().numpy())
    assert np.abs(gs.cpu().numpy().astype(np.float64) - s).max() < 3e-6
    log("mixed sign", dtype, rep)


@pytest.mark.parametrize("d", [8, 16, 24, 32])
@pytest.mark.parametrize("sizes", [((37, 29), (41, 23)), ((70, 50), (64, 48)), ((64, 64), (64, 64)),
                                   ((1, 1), (9, 7)), ((9, 7), (1, 1)), ((96, 96), (50, 61))])
def test_mutual_fused_bf16_equals_two_searches(d, sizes):
    """bf16 maps (d <= 32) take the fused row + column pass.  Its two NN maps must equal,
    element by element, the two separate searches of mr_nn_argmax (the same scores and
    the same comparison rule), and both must pass the oracle rule.  Sizes cover ragged
    query and database tiles, a partial second query group (70x50 = 3500 queries), whole
    tiles, single-pixel maps, and several database segments per query group."""
    (h1, w1), (h2, w2) = sizes
    p = workloads.make_pair(h1, w1, d, seed=1000 + d + h1, warp="shift", sigma=0.1, rho=0.2, dtype="bf16")
    q = workloads.make_pair(h2, w2, d, seed=2000 + d + h2, warp="shift", sigma=0.1, rho=0.2, dtype="bf16")
    A = dev_map(p.D1, h1, w1, p.D1_bits)
    B = dev_map(q.D2, h2, w2, q.D2_bits)
    pairs, n, nn_ab, nn_ba = mr.mutual_nn(A, B)
    i12 = mr.nn_argmax(A, B)
    i21 = mr.nn_argmax(B, A)
    torch.cuda.synchronize()
    g12, g21 = nn_ab[0].cpu().numpy(), nn_ba[0].cpu().numpy()
    assert (g12 == i12.cpu().numpy()).all()
    assert (g21 == i21.cpu().numpy()).all()
    oi, o1, o2 = oracle.nn(p.D1, q.D2)
    checks.check_nn(g12, oi, o1, o2, p.D1, np.arange(len(p.D1)), q.D2, "bf16")
    oj, b1, b2 = oracle.nn(q.D2, p.D1)
    checks.check_nn(g21, oj, b1, b2, q.D2, np.arange(len(q.D2)), p.D1, "bf16")
    gp = mr.matches(pairs, n)
    i = np.nonzero(g21[g12] == np.arange(len(g12)))[0]
    assert gp.tolist() == np.stack([i, g12[i]], 1).tolist()


def test_mutual_fused_bf16_batch_and_negative_scores():
    """The fused pass with a batch of three pairs (each against its own maps), and with
    every similarity negative (maxima below zero go through the same comparison)."""
    Bn, H, W, d = 3, 23, 19, 24
    ps = [workloads.make_pair(H, W, d, seed=1300 + b, warp="shift", sigma=0.1, rho=0.2, dtype="bf16")
          for b in range(Bn)]
    A = torch.stack([dev_map(p.D1, H, W, p.D1_bits) for p in ps])
    Bm = torch.stack([dev_map(p.D2, H, W, p.D2_bits) for p in ps])
    pairs, n, nn_ab, nn_ba = mr.mutual_nn(A, Bm)
    torch.cuda.synchronize()
    for b, p in enumerate(ps):
        o_pairs, o12, a1, a2, o21, c1, c2 = oracle.mutual_nn(p.D1, p.D2)
        checks.check_nn(nn_ab[b].cpu().numpy(), o12, a1, a2, p.D1, np.arange(p.N), p.D2, "bf16")
        checks.check_nn(nn_ba[b].cpu().numpy(), o21, c1, c2, p.D2, np.arange(p.N), p.D1, "bf16")
    rng = np.random.default_rng(6)
    e = np.zeros(d)
    e[0] = 1.0

    def unit(x):
        return (x / np.linalg.norm(x, axis=1, keepdims=True)).astype(np.float32)

    Ab = workloads.f32_to_bf16_bits(unit(0.9 * e + 0.25 * rng.standard_normal((37 * 29, d)) / np.sqrt(d)))
    Bb = workloads.f32_to_bf16_bits(unit(-0.9 * e + 0.25 * rng.standard_normal((41 * 23, d)) / np.sqrt(d)))
    Af, Bf = workloads.bf16_bits_to_f32(Ab), workloads.bf16_bits_to_f32(Bb)
    pairs, n, nn_ab, nn_ba = mr.mutual_nn(dev_map(Af, 37, 29, Ab), dev_map(Bf, 41, 23, Bb))
    torch.cuda.synchronize()
    o_pairs, o12, a1, a2, o21, c1, c2 = oracle.mutual_nn(Af, Bf)
    assert a1.max() < 0 and c1.max() < 0
    checks.check_nn(nn_ab[0].cpu().numpy(), o12, a1, a2, Af, np.arange(len(Af)), Bf, "bf16")
    checks.check_nn(nn_ba[0].cpu().numpy(), o21, c1, c2, Bf, np.arange(len(Bf)), Af, "bf16")


def test_mutual_c2_bf16_full_size_sampled():
    """512x384 bf16 pair, full 196608^2 brute force; the oracle checks 4096 random rows and
    4096 random columns (and the reciprocity of the sampled rows)."""
    p = workloads.config_pair(2)
    A, B = pair_maps(p)
    pairs, n, nn_ab, nn_ba = mr.mutual_nn(A, B)
    torch.cuda.synchronize()
    g12, g21 = nn_ab[0].cpu().numpy(), nn_ba[0].cpu().numpy()
    gp = mr.matches(pairs, n)
    rng = np.random.default_rng(2)
    rows = np.sort(rng.choice(p.N, 4096, replace=False)).astype(np.int32)
    cols = np.sort(rng.choice(p.N, 4096, replace=False)).astype(np.int32)
    oi, o1, o2 = oracle.nn_rows(p.D1, rows, p.D2)
    r1 = checks.check_nn(g12[rows], oi, o1, o2, p.D1, rows, p.D2, "bf16")
    oj, q1, q2 = oracle.nn_rows(p.D2, cols, p.D1)
    r2 = checks.check_nn(g21[cols], oj, q1, q2, p.D2, cols, p.D1, "bf16")
    # reciprocity of the sampled rows: the oracle's NN of their GPU partners
    back, c1, c2 = oracle.nn_rows(p.D2, g12[rows], p.D1)
    checks.check_nn(g21[g12[rows]], back, c1, c2, p.D2, g12[rows], p.D1, "bf16")
    # the pair list is the reciprocal subset of the GPU's own maps, over all pixels
    i = np.nonzero(g21[g12] == np.arange(p.N))[0]
    assert (gp[:, 0] == i).all() and (gp[:, 1] == g12[i]).all()
    # the fused pass equals the two separate searches everywhere
    s12 = mr.nn_argmax(A, B)
    s21 = mr.nn_argmax(B, A)
    torch.cuda.synchronize()
    assert (g12 == s12.cpu().numpy()).all() and (g21 == s21.cpu().numpy()).all()
    log("c2", r1, r2, "pairs", len(gp))


# ============================================================================ fast reciprocal

@pytest.mark.parametrize("name", ["circle_1x4", "grid_2x3", "ties_d1", "negative_scores"])
def test_fast_golden(name):
    """The hand-derived fixtures, through the GPU path."""
    g, A, B = _load_golden(name)
    H1, W1 = g["H1"], g["W1"]
    Ad = dev_map(A, H1, W1)
    Bd = dev_map(B, 1, B.shape[0])
    pairs, n, nn_ab, nn_ba = mr.mutual_nn(Ad, Bd)
    torch.cuda.synchronize()
    assert nn_ab[0].cpu().tolist() == g["nn12"]
    assert nn_ba[0].cpu().tolist() == g["nn21"]
    assert mr.matches(pairs, n).tolist() == g["mutual"]
    for case in g["fast"]:
        fp, fn, _ = mr.fast_reciprocal(Ad, Bd, case["stride"], case["offset"], case["T"])
        torch.cuda.synchronize()
        assert mr.matches(fp, fn).tolist() == case["pairs"], case


@pytest.mark.parametrize("cfg", [
    dict(H=64, W=48, warp="shift", sigma=0.1, rho=0.2, stride=8, offset=4, T=10),
    dict(H=64, W=48, warp="shift", sigma=0.1, rho=0.2, stride=8, offset=0, T=1),
    dict(H=53, W=47, warp="affine", sigma=0.15, rho=0.3, stride=5, offset=2, T=3),
    dict(H=53, W=47, warp="affine", sigma=0.3, rho=0.5, stride=3, offset=1, T=15),
    dict(H=90, W=70, warp="homography", sigma=0.2, rho=0.4, stride=7, offset=3, T=6),
    dict(H=29, W=31, warp="shift", sigma=0.1, rho=0.2, stride=1, offset=0, T=2),
])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fast_full(cfg, dtype):
    p = workloads.make_pair(cfg["H"], cfg["W"], 24, seed=700 + cfg["H"] + cfg["stride"], warp=cfg["warp"],
                            sigma=cfg["sigma"], rho=cfg["rho"], dtype=dtype)
    A, B = pair_maps(p)
    fp, fn, act = mr.fast_reciprocal(A, B, cfg["stride"], cfg["offset"], cfg["T"])
    torch.cuda.synchronize()
    orc = oracle.fast(p.D1, p.H, p.W, p.D2, cfg["stride"], cfg["offset"], cfg["T"])
    act = act[0].cpu().numpy()
    rep = checks.check_fast(mr.matches(fp, fn), orc, p.D1, p.D2, dtype, gpu_active=act)
    assert act[0] == len(seeds_of(p.H, p.W, cfg["stride"], cfg["offset"]))
    assert (np.diff(act) <= 0).all()
    log("fast", cfg, dtype, rep, act.tolist())


@pytest.mark.parametrize("d", [8, 16, 32])
def test_fast_split_fp32_other_d(d):
    """The fast scheme on fp32 maps with d = 8, 16, 32 (the split products with three
    query tiles per wave, two at d = 32): 720 seeds fill whole query groups, so the
    interleaved full-tile path runs, against the oracle."""
    p = workloads.make_pair(90, 70, d, seed=900 + d, warp="affine", sigma=0.15, rho=0.3, dtype="f32")
    A, B = pair_maps(p)
    fp, fn, act = mr.fast_reciprocal(A, B, 3, 1, 6)
    torch.cuda.synchronize()
    orc = oracle.fast(p.D1, p.H, p.W, p.D2, 3, 1, 6)
    act = act[0].cpu().numpy()
    rep = checks.check_fast(mr.matches(fp, fn), orc, p.D1, p.D2, "f32", gpu_active=act)
    assert act[0] == len(seeds_of(p.H, p.W, 3, 1))
    log("fast split fp32", d, rep, act.tolist())


def test_fast_is_subset_of_gpu_mutual_and_stride1_equals_it():
    """In the GPU's own arithmetic: fast matches are mutual NNs, and seeding every pixel
    returns the brute-force mutual set exactly."""
    p = workloads.make_pair(57, 45, 24, seed=800, warp="affine", sigma=0.15, rho=0.3)
    A, B = pair_maps(p)
    mp, mn, _, _ = mr.mutual_nn(A, B)
    m = {tuple(x) for x in mr.matches(mp, mn).tolist()}
    for stride, off, T in ((4, 2, 10), (6, 1, 3)):
        fp, fn, _ = mr.fast_reciprocal(A, B, stride, off, T)
        assert {tuple(x) for x in mr.matches(fp, fn).tolist()} <= m
    fp, fn, _ = mr.fast_reciprocal(A, B, 1, 0, 1)
    assert {tuple(x) for x in mr.matches(fp, fn).tolist()} == m


def test_fast_edges():
    """max_iters = 0, a stride beyond the image, a 1x1 image, images of different sizes,
    an offset beyond the image (no seeds)."""
    p = workloads.make_pair(30, 20, 24, seed=900, warp="shift", sigma=0.1, rho=0.2)
    A, B = pair_maps(p)
    fp, fn, act = mr.fast_reciprocal(A, B, 4, 1, 0)
    assert int(fn[0]) == 0
    fp, fn, _ = mr.fast_reciprocal(A, B, 100, 0, 6)
    orc = oracle.fast(p.D1, p.H, p.W, p.D2, 100, 0, 6)
    assert mr.matches(fp, fn).tolist() == orc["pairs"].tolist()
    fp, fn, act = mr.fast_reciprocal(A, B, 4, 40, 5)
    assert int(fn[0]) == 0 and (act[0].cpu().numpy() == 0).all()
    one = dev_map(p.D1[:1], 1, 1)
    fp, fn, _ = mr.fast_reciprocal(one, B, 1, 0, 3)
    orc = oracle.fast(p.D1[:1], 1, 1, p.D2, 1, 0, 3)
    assert mr.matches(fp, fn).tolist() == orc["pairs"].tolist()
    q = workloads.make_pair(17, 33, 24, seed=901, warp="shift", sigma=0.1, rho=0.2)
    Bq = dev_map(q.D2, q.H, q.W)
    fp, fn, _ = mr.fast_reciprocal(A, Bq, 3, 1, 8)
    torch.cuda.synchronize()
    orc = oracle.fast(p.D1, p.H, p.W, q.D2, 3, 1, 8)
    checks.check_fast(mr.matches(fp, fn), orc, p.D1, q.D2, "f32")


def test_fast_deterministic():
    p = workloads.make_pair(96, 80, 24, seed=950, warp="affine", sigma=0.15, rho=0.3)
    A, B = pair_maps(p)
    f = mr.FastReciprocal(A.unsqueeze(0), B.unsqueeze(0), 4, 2, 10)
    outs = []
    for _ in range(3):
        pr, n, act = f(A.unsqueeze(0), B.unsqueeze(0))
        torch.cuda.synchronize()
        outs.append((pr[0, :int(n[0])].cpu().numpy().copy(), act.cpu().numpy().copy()))
    for o in outs[1:]:
        assert (o[0] == outs[0][0]).all() and (o[1] == outs[0][1]).all()


def test_fast_c1_full_size():
    """One 512x384 fp32 pair, stride 8 (3072 seeds), 10 iterations, against a full oracle run."""
    p = workloads.config_pair(1)
    A, B = pair_maps(p)
    fp, fn, act = mr.fast_reciprocal(A, B, p.stride, p.offset, p.max_iters)
    torch.cuda.synchronize()
    orc = oracle.fast(p.D1, p.H, p.W, p.D2, p.stride, p.offset, p.max_iters)
    rep = checks.check_fast(mr.matches(fp, fn), orc, p.D1, p.D2, "f32", gpu_active=act[0].cpu().numpy())
    log("c1", rep, act[0].cpu().tolist(), orc["fresh"].tolist())


def test_c0_workload_mutual_and_fast():
    """The tiny pair exactly as the bench configuration defines it (64x48 fp32, seed 0):
    brute-force mutual NN in full against the oracle, and the fast scheme (stride 8,
    offset 4, 10 iterations) against a full oracle run, live counts included."""
    p = workloads.config_pair(0)
    A, B = pair_maps(p)
    pairs, n, nn_ab, nn_ba = mr.mutual_nn(A, B)
    fp, fn, act = mr.fast_reciprocal(A, B, p.stride, p.offset, p.max_iters)
    torch.cuda.synchronize()
    o_pairs, o12, a1, a2, o21, b1, b2 = oracle.mutual_nn(p.D1, p.D2)
    checks.check_nn(nn_ab[0].cpu().numpy(), o12, a1, a2, p.D1, np.arange(p.N), p.D2, p.dtype)
    checks.check_nn(nn_ba[0].cpu().numpy(), o21, b1, b2, p.D2, np.arange(p.N), p.D1, p.dtype)
    gp = mr.matches(pairs, n)
    clean = (a1 - a2 > checks.MARGIN) & (b1[o12] - b2[o12] > checks.MARGIN)
    assert clean.all()
    assert gp.tolist() == o_pairs.tolist()
    orc = oracle.fast(p.D1, p.H, p.W, p.D2, p.stride, p.offset, p.max_iters)
    rep = checks.check_fast(mr.matches(fp, fn), orc, p.D1, p.D2, p.dtype, gpu_active=act[0].cpu().numpy())
    assert rep["unclean_seeds"] == 0 and rep["gpu"] == rep["oracle"] == rep["common"]
    log("c0", len(gp), rep, act[0].cpu().tolist())


def test_fast_c4_full_size_sampled():
    """1024x768 bf16 pair, stride 8 (12288 seeds), 15 iterations: 256 sampled seed chains
    followed by the oracle, and every GPU pair's reciprocity for 384 sampled pairs."""
    p = workloads.config_pair(4)
    A, B = pair_maps(p)
    fp, fn, act = mr.fast_reciprocal(A, B, p.stride, p.offset, p.max_iters)
    torch.cuda.synchronize()
    gp = mr.matches(fp, fn)
    checks.check_one_to_one_sorted(gp)
    gset = {tuple(x) for x in gp.tolist()}
    rng = np.random.default_rng(4)
    seeds = np.array(seeds_of(p.H, p.W, p.stride, p.offset))
    sample = rng.choice(seeds, 256, replace=False)
    chains = checks.oracle_chains(p.D1, p.D2, sample, p.max_iters)
    missing = [k for k, clean in chains.items() if clean and k not in gset]
    assert not missing, missing[:3]
    pick = gp[rng.choice(len(gp), min(384, len(gp)), replace=False)]
    checks.check_reciprocal(pick, p.D1, p.D2, "bf16")
    log("c4", len(gp), "sampled chains", len(chains), act[0].cpu().tolist())


def test_fast_c3_batch64():
    """64 independent 512x384 fp32 pairs in one call: pairs 0 and 63 against full oracle
    runs, 64 sampled GPU pairs of every pair for reciprocity, and pair 17 equal to a
    single-pair call."""
    ps = []
    for b in range(64):
        ps.append(workloads.config_pair(3, b))
    A = torch.stack([dev_map(p.D1, p.H, p.W) for p in ps])
    B = torch.stack([dev_map(p.D2, p.H, p.W) for p in ps])
    log("c3 data ready")
    p0 = ps[0]
    fp, fn, act = mr.fast_reciprocal(A, B, p0.stride, p0.offset, p0.max_iters)
    torch.cuda.synchronize()
    for b in (0, 63):
        orc = oracle.fast(ps[b].D1, p0.H, p0.W, ps[b].D2, p0.stride, p0.offset, p0.max_iters)
        checks.check_fast(mr.matches(fp, fn, b), orc, ps[b].D1, ps[b].D2, "f32", gpu_active=act[b].cpu().numpy())
    rng = np.random.default_rng(3)
    for b in range(64):
        gp = mr.matches(fp, fn, b)
        checks.check_one_to_one_sorted(gp)
        pick = gp[rng.choice(len(gp), min(64, len(gp)), replace=False)]
        checks.check_reciprocal(pick, ps[b].D1, ps[b].D2, "f32")
    sp, sn, _ = mr.fast_reciprocal(A[17], B[17], p0.stride, p0.offset, p0.max_iters)
    assert mr.matches(sp, sn).tolist() == mr.matches(fp, fn, 17).tolist()
    log("c3", [int(x) for x in fn.cpu()][:8], "...")
