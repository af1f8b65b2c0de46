"""GPU parity of the matching loss (InfoNCE) against the CPU oracle.

Term of ground-truth pair (i, j): log sum_k exp(<a_i, b_k>/tau) - <a_i, b_j>/tau over
every row k of b ("MASt3R dissection", section 3 "Napkin Formula"); the loss of an
image pair is the sum of its terms.  The oracle evaluates each term in binary64.

Tolerance (unit rows, tau >= 0.05, up to 2^18 rows in b): a score carries at most
about d * 2^-24 of error in fp32 (the split-fp32 products are exact to 2^-23), i.e.
1.4e-6 at d = 24, which moves the log-sum-exp and the positive term by at most
1.4e-5 each at tau = 0.1 (2.8e-5 at tau = 0.05); the fp32 sums of the exponentials are
compensated (Kahan) per lane and per segment merge, so they add a few units of fp32
rounding whatever their length, as do v_exp and the final log and products for a term
below 30.  atol = 1e-4 covers that worst case; rows scaled by c multiply the score
errors by c^2.  The loss is checked against the binary64 sum of the oracle's
terms within n_gt * atol, and against the binary64 sum of the GPU's own terms to
1e-12 (the reduction itself).
"""
import math

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import dense_grounded_image_amd as mr  # noqa: E402

DEV = torch.device("cuda:0")
ATOL = 1e-4


def log(*a):
    print(*a, flush=True)


def dev_map(arr, H, W, bits=None):
    if bits is not None:
        t = torch.from_numpy(np.ascontiguousarray(bits).reshape(H, W, -1)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32).reshape(H, W, -1))
    return t.to(DEV)


def run(A, B, gt, tau, H1, W1, H2, W2, bits=(None, None)):
    a = dev_map(A, H1, W1, bits[0])
    b = dev_map(B, H2, W2, bits[1])
    g = torch.from_numpy(np.ascontiguousarray(gt, dtype=np.int32)).to(DEV)
    terms, loss = mr.infonce(a, b, g, tau)
    torch.cuda.synchronize()
    return terms[0].cpu().numpy().astype(np.float64), float(loss[0].cpu())


def check(gt_terms, gt_loss, A, B, gt, tau, atol=ATOL):
    o_terms, o_total = oracle.infonce(A, B, gt, float(np.float32(tau)))
    err = np.abs(gt_terms - o_terms)
    assert np.isfinite(gt_terms).all()
    assert err.max() <= atol, (err.max(), int(err.argmax()))
    assert abs(gt_loss - o_total) <= len(gt) * atol
    assert abs(gt_loss - math.fsum(gt_terms)) <= 1e-12 * max(1.0, math.fsum(np.abs(gt_terms)))
    return err.max()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nce_tiny_planted(dtype):
    """64x48 planted pair, every non-occluded pixel of image 2 as ground truth."""
    p = workloads.make_pair(64, 48, 24, 0, warp="shift", sigma=0.1, rho=0.2, dtype=dtype)
    gt = workloads.gt_pairs(p)
    terms, loss = run(p.D1, p.D2, gt, 0.1, p.H, p.W, p.H, p.W, (p.D1_bits, p.D2_bits))
    e = check(terms, loss, p.D1, p.D2, gt, 0.1)
    log("tiny", dtype, len(gt), "max err", e, "loss", loss)


@pytest.mark.parametrize("dtype,d", [("f32", 8), ("f32", 16), ("f32", 32), ("bf16", 8), ("bf16", 40),
                                     ("bf16", 64)])
def test_nce_ragged_sizes(dtype, d):
    """Maps of 37x29 and 23x41 pixels (ragged 32-row tiles), a ragged ground-truth count,
    repeated rows i, and every supported descriptor length class."""
    rng = np.random.default_rng(100 + d)
    A = workloads.unit_rows(rng, 37 * 29, d).astype(np.float32)
    B = workloads.unit_rows(rng, 23 * 41, d).astype(np.float32)
    bits = (None, None)
    if dtype == "bf16":
        bits = (workloads.f32_to_bf16_bits(A), workloads.f32_to_bf16_bits(B))
        A, B = workloads.bf16_bits_to_f32(bits[0]), workloads.bf16_bits_to_f32(bits[1])
    n_gt = 517
    gt = np.stack([rng.integers(0, len(A), n_gt), rng.integers(0, len(B), n_gt)], axis=1).astype(np.int32)
    gt[5:9, 0] = gt[4, 0]
    terms, loss = run(A, B, gt, 0.1, 37, 29, 23, 41, bits)
    e = check(terms, loss, A, B, gt, 0.1)
    log("ragged", dtype, d, "max err", e)


@pytest.mark.parametrize("n_gt", [1, 5, 31, 33, 4000])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nce_counts(n_gt, dtype):
    """Few ground-truth pairs spread each query over many database segments; many fill
    several query groups (partial ones too: for bf16 the register stream then runs zero
    operands in the empty query slots)."""
    rng = np.random.default_rng(n_gt)
    A = workloads.unit_rows(rng, 96 * 64, 24).astype(np.float32)
    B = workloads.unit_rows(rng, 80 * 72, 24).astype(np.float32)
    bits = (None, None)
    if dtype == "bf16":
        bits = (workloads.f32_to_bf16_bits(A), workloads.f32_to_bf16_bits(B))
        A, B = workloads.bf16_bits_to_f32(bits[0]), workloads.bf16_bits_to_f32(bits[1])
    gt = np.stack([rng.integers(0, len(A), n_gt), rng.integers(0, len(B), n_gt)], axis=1).astype(np.int32)
    terms, loss = run(A, B, gt, 0.1, 96, 64, 80, 72, bits)
    e = check(terms, loss, A, B, gt, 0.1)
    log("count", dtype, n_gt, "max err", e)


@pytest.mark.parametrize("tau", [0.05, 0.1, 1.0])
def test_nce_temperatures(tau):
    p = workloads.make_pair(48, 40, 24, 7, warp="affine", sigma=0.15, rho=0.3)
    gt = workloads.gt_pairs(p)
    terms, loss = run(p.D1, p.D2, gt, tau, p.H, p.W, p.H, p.W)
    e = check(terms, loss, p.D1, p.D2, gt, tau)
    log("tau", tau, "max err", e)


def test_nce_large_scores_do_not_overflow():
    """Rows of norm 3 at tau = 0.05: scores / tau reach 180, far past the fp32 range of
    exp; the online shift keeps every exponential finite.  Score errors grow by 9x."""
    rng = np.random.default_rng(9)
    A = (3.0 * workloads.unit_rows(rng, 40 * 40, 24)).astype(np.float32)
    B = (3.0 * workloads.unit_rows(rng, 40 * 40, 24)).astype(np.float32)
    B[:200] = A[:200]   # strong positives
    gt = np.stack([np.arange(300), np.arange(300)], axis=1).astype(np.int32)
    terms, loss = run(A, B, gt, 0.05, 40, 40, 40, 40)
    e = check(terms, loss, A, B, gt, 0.05, atol=20 * ATOL)
    log("large", "max err", e)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nce_scores_rising_along_the_database(dtype):
    """Database row k is alpha_t * a[k mod 300], alpha stepping up by 0.97 from one
    32-row tile to the next in runs of four tiles (0.1 .. 3.0): at tau = 0.02 a query's
    best score then rises by about 70 in base-2 exponent units per tile, so the
    log-sum-exp offset is raised inside segments, again and again, where it would
    otherwise stay.  Scores reach 3, so score errors grow by 3x and the exponent errors
    by 5x against tau = 0.1."""
    rng = np.random.default_rng(21)
    A = workloads.unit_rows(rng, 40 * 40, 24).astype(np.float32)
    k = np.arange(64 * 64)
    alpha = (0.1 + 0.97 * ((k // 32) % 4)).astype(np.float32)
    B = (alpha[:, None] * A[k % 300]).astype(np.float32)
    bits = (None, None)
    if dtype == "bf16":
        bits = (workloads.f32_to_bf16_bits(A), workloads.f32_to_bf16_bits(B))
        A, B = workloads.bf16_bits_to_f32(bits[0]), workloads.bf16_bits_to_f32(bits[1])
    gt = np.stack([np.arange(300), np.arange(300) + 3 * 32], axis=1).astype(np.int32)
    terms, loss = run(A, B, gt, 0.02, 40, 40, 64, 64, bits)
    e = check(terms, loss, A, B, gt, 0.02, atol=10 * ATOL)
    log("rising", dtype, "max err", e)


def test_nce_batch_and_invalid_pairs():
    """Three image pairs in one call; pair 1 holds an out-of-range ground-truth row, whose
    term (and that pair's loss) is NaN while the others are unaffected."""
    ps = [workloads.make_pair(40, 36, 24, 20 + b, warp="shift", sigma=0.1, rho=0.2) for b in range(3)]
    n_gt = 700
    gts = [workloads.gt_pairs(p)[:n_gt] for p in ps]
    assert all(len(g) == n_gt for g in gts)
    gts[1] = gts[1].copy()
    gts[1][17] = (40 * 36, 3)
    A = torch.from_numpy(np.stack([p.D1 for p in ps]).reshape(3, 40, 36, 24)).to(DEV)
    B = torch.from_numpy(np.stack([p.D2 for p in ps]).reshape(3, 40, 36, 24)).to(DEV)
    g = torch.from_numpy(np.stack(gts)).to(DEV)
    terms, loss = mr.infonce(A, B, g, 0.1)
    torch.cuda.synchronize()
    terms, loss = terms.cpu().numpy().astype(np.float64), loss.cpu().numpy()
    for b in (0, 2):
        check(terms[b], float(loss[b]), ps[b].D1, ps[b].D2, gts[b], 0.1)
    assert np.isnan(terms[1][17]) and np.isnan(loss[1])
    ok = np.ones(n_gt, bool)
    ok[17] = False
    o_terms, _ = oracle.infonce(ps[1].D1, ps[1].D2, gts[1][ok], float(np.float32(0.1)))
    assert np.abs(terms[1][ok] - o_terms).max() <= ATOL


def test_nce_empty_ground_truth():
    p = workloads.make_pair(32, 32, 24, 3)
    a = dev_map(p.D1, 32, 32)
    b = dev_map(p.D2, 32, 32)
    terms, loss = mr.infonce(a, b, torch.zeros((0, 2), dtype=torch.int32, device=DEV), 0.1)
    torch.cuda.synchronize()
    assert terms.shape == (1, 0) and float(loss[0].cpu()) == 0.0


def test_nce_deterministic():
    p = workloads.make_pair(64, 48, 24, 5, warp="affine", sigma=0.15, rho=0.3, dtype="bf16")
    gt = workloads.gt_pairs(p)
    r1 = run(p.D1, p.D2, gt, 0.1, p.H, p.W, p.H, p.W, (p.D1_bits, p.D2_bits))
    r2 = run(p.D1, p.D2, gt, 0.1, p.H, p.W, p.H, p.W, (p.D1_bits, p.D2_bits))
    assert (r1[0] == r2[0]).all() and r1[1] == r2[1]


def test_nce_full_size_bf16_sampled():
    """512x384 bf16 planted pair, every non-occluded pixel as ground truth (about 137k
    terms against 196608 rows each); the oracle checks 1500 sampled terms, and the loss
    is the sum of the GPU's terms."""
    p = workloads.config_pair(2)
    gt = workloads.gt_pairs(p)
    terms, loss = run(p.D1, p.D2, gt, 0.1, p.H, p.W, p.H, p.W, (p.D1_bits, p.D2_bits))
    assert np.isfinite(terms).all() and (terms > -1e-3).all()
    rng = np.random.default_rng(4)
    pick = np.sort(rng.choice(len(gt), 1500, replace=False))
    o_terms, _ = oracle.infonce(p.D1, p.D2, gt[pick], float(np.float32(0.1)))
    err = np.abs(terms[pick] - o_terms)
    assert err.max() <= ATOL, err.max()
    assert abs(loss - math.fsum(terms)) <= 1e-12 * math.fsum(np.abs(terms))
    log("c2 nce", len(gt), "max err", err.max(), "loss", loss)
