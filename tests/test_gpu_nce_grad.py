"""GPU parity of the matching loss's gradient against the CPU oracle.

With p[t][k] the softmax of term t over the rows k of image 2 ("MASt3R dissection",
section 3 "Napkin Formula": the loss; its gradient is the derivative of each term's
log-sum-exp, the softmax):
    dL/dA[i] = (1/tau) sum_{t: i_t = i} (sum_k p[t][k] B[k] - B[j_t]),
    dL/dB[k] = (1/tau) sum_t p[t][k] A[i_t] - (1/tau) sum_{t: j_t = k} A[i_t].
The oracle (binary64, pinned against central differences of its own loss) gives both.

Tolerance, unit rows, tau = 0.1: a score errs by about d * 2^-24 (1.4e-6 at d = 24) and
the log-sum-exp by as much again, so each softmax value carries a relative error near
ln 2 * k2 * 3e-6 = 3e-5; the two-part bf16 split of p adds 2^-17 = 7.6e-6 relative; the
fp32 accumulation on the matrix cores over up to 2.5e4 steps adds, as a random walk,
about 1e-5 of the sum (its worst case is far larger and is not what is checked).  With
|B[k][c]| <= 1 and sum_k p = 1 the softmax-weighted sum errs by about 5e-5 per term, so a
row of dA is checked to 1e-4 / tau per ground-truth pair naming it, and a row k of dB to
1e-4 / tau * (1 + its column mass sum_t p[t][k]).  Rows of A that no pair names must be
exactly 0.
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import dense_grounded_image_amd as mr  # noqa: E402

DEV = torch.device("cuda:0")
EPS = 1e-4


def log(*a):
    print(*a, flush=True)


def bf16_pair(rng, n1, n2, d, dtype="bf16"):
    """Unit rows; for bf16 the oracle reads the exactly widened values.  Returns the fp32
    arrays and the arrays the device gets (bf16 bit patterns, or the fp32 arrays)."""
    A = workloads.unit_rows(rng, n1, d).astype(np.float32)
    B = workloads.unit_rows(rng, n2, d).astype(np.float32)
    if dtype == "f32":
        return A, B, A, B
    ba, bb = workloads.f32_to_bf16_bits(A), workloads.f32_to_bf16_bits(B)
    return workloads.bf16_bits_to_f32(ba), workloads.bf16_bits_to_f32(bb), ba, bb


def dev_bits(arr, H, W):
    t = torch.from_numpy(np.ascontiguousarray(arr).reshape(H, W, -1))
    return (t.view(torch.bfloat16) if arr.dtype == np.int16 else t).to(DEV)


def run(bits_a, bits_b, gt, tau, H1, W1, H2, W2):
    a, b = dev_bits(bits_a, H1, W1), dev_bits(bits_b, H2, W2)
    g = torch.from_numpy(np.ascontiguousarray(gt, dtype=np.int32)).to(DEV)
    terms, loss, ga, gb = mr.infonce_backward(a, b, g, tau)
    fterms, floss = mr.infonce(a, b, g, tau)
    torch.cuda.synchronize()
    # the gradient call's loss stage is the forward call's
    assert torch.equal(terms, fterms) and torch.equal(loss, floss)
    return (terms[0].cpu().numpy(), float(loss[0].cpu()), ga[0].reshape(-1, ga.shape[-1]).cpu().numpy(),
            gb[0].reshape(-1, gb.shape[-1]).cpu().numpy())


def check_grads(ga, gb, A, B, gt, tau, b_rows=None, a_rows=None):
    dA, dB, mass = oracle.infonce_grad(A, B, gt, float(np.float32(tau)), b_rows=b_rows)
    counts = np.bincount(gt[:, 0], minlength=len(A))
    rows_a = np.arange(len(A)) if a_rows is None else a_rows
    ea = np.abs(ga[rows_a] - dA[rows_a]).max(axis=1)
    tol_a = EPS / tau * counts[rows_a]
    assert (ea <= tol_a).all(), (float(ea.max()), int(np.argmax(ea - tol_a)))
    assert (ga[rows_a][counts[rows_a] == 0] == 0).all()
    gbr = gb if b_rows is None else gb[b_rows]
    eb = np.abs(gbr - dB).max(axis=1)
    tol_b = EPS / tau * (1.0 + mass)
    assert (eb <= tol_b).all(), (float(eb.max()), int(np.argmax(eb - tol_b)))
    return float((ea / np.maximum(tol_a, 1e-30)).max()), float((eb / tol_b).max())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_grad_tiny_planted(dtype):
    """64x48 planted pair, every non-occluded pixel of image 2 as ground truth."""
    p = workloads.make_pair(64, 48, 24, 0, warp="shift", sigma=0.1, rho=0.2, dtype=dtype)
    gt = workloads.gt_pairs(p)
    da, db = (p.D1_bits, p.D2_bits) if dtype == "bf16" else (p.D1, p.D2)
    terms, loss, ga, gb = run(da, db, gt, 0.1, p.H, p.W, p.H, p.W)
    ra, rb = check_grads(ga, gb, p.D1, p.D2, gt, 0.1)
    log("grad tiny", dtype, len(gt), "err/tol", ra, rb)


@pytest.mark.parametrize("dtype,d", [("bf16", 8), ("bf16", 16), ("bf16", 24), ("bf16", 32), ("f32", 8), ("f32", 16),
                                     ("f32", 24), ("f32", 32)])
def test_grad_ragged(dtype, d):
    """37x29 against 23x41 pixels (ragged tiles), 517 pairs with repeated rows on both sides."""
    rng = np.random.default_rng(200 + d)
    A, B, ba, bb = bf16_pair(rng, 37 * 29, 23 * 41, d, dtype)
    n_gt = 517
    gt = np.stack([rng.integers(0, len(A), n_gt), rng.integers(0, len(B), n_gt)], axis=1).astype(np.int32)
    gt[5:9, 0] = gt[4, 0]
    gt[20:25, 1] = gt[19, 1]
    terms, loss, ga, gb = run(ba, bb, gt, 0.1, 37, 29, 23, 41)
    ra, rb = check_grads(ga, gb, A, B, gt, 0.1)
    log("grad ragged", dtype, d, "err/tol", ra, rb)


@pytest.mark.parametrize("n_gt", [1, 5, 33, 3000])
def test_grad_counts(n_gt):
    rng = np.random.default_rng(300 + n_gt)
    A, B, ba, bb = bf16_pair(rng, 64 * 64, 72 * 56, 24)
    gt = np.stack([rng.integers(0, len(A), n_gt), rng.integers(0, len(B), n_gt)], axis=1).astype(np.int32)
    terms, loss, ga, gb = run(ba, bb, gt, 0.1, 64, 64, 72, 56)
    ra, rb = check_grads(ga, gb, A, B, gt, 0.1)
    log("grad count", n_gt, "err/tol", ra, rb)


def test_grad_batch():
    """Two image pairs in one call: each pair's gradient is its own loss's."""
    rng = np.random.default_rng(400)
    pairs = [bf16_pair(rng, 40 * 36, 40 * 36, 24) for _ in range(2)]
    gts = [np.stack([rng.integers(0, 40 * 36, 300), rng.integers(0, 40 * 36, 300)], 1).astype(np.int32)
           for _ in range(2)]
    a = torch.from_numpy(np.stack([q[2] for q in pairs]).reshape(2, 40, 36, 24)).view(torch.bfloat16).to(DEV)
    b = torch.from_numpy(np.stack([q[3] for q in pairs]).reshape(2, 40, 36, 24)).view(torch.bfloat16).to(DEV)
    g = torch.from_numpy(np.stack(gts)).to(DEV)
    terms, loss, ga, gb = mr.infonce_backward(a, b, g, 0.1)
    torch.cuda.synchronize()
    for k in range(2):
        check_grads(ga[k].reshape(-1, 24).cpu().numpy(), gb[k].reshape(-1, 24).cpu().numpy(), pairs[k][0],
                    pairs[k][1], gts[k], 0.1)


def test_grad_empty_ground_truth():
    rng = np.random.default_rng(5)
    A, B, ba, bb = bf16_pair(rng, 32 * 32, 32 * 32, 24)
    a, b = dev_bits(ba, 32, 32), dev_bits(bb, 32, 32)
    terms, loss, ga, gb = mr.infonce_backward(a, b, torch.zeros((0, 2), dtype=torch.int32, device=DEV), 0.1)
    torch.cuda.synchronize()
    assert float(loss[0].cpu()) == 0.0 and not ga.any() and not gb.any()


@pytest.mark.parametrize("cfg", [2, 1])
def test_grad_full_size_sampled(cfg):
    """512x384 maps (bf16, then fp32) with 2048 ground-truth pairs of the planted field:
    every named row of dA and 512 sampled rows of dB against the oracle."""
    p = workloads.config_pair(cfg)
    gt_all = workloads.gt_pairs(p)
    rng = np.random.default_rng(6)
    gt = gt_all[np.sort(rng.choice(len(gt_all), 2048, replace=False))]
    da, db = (p.D1_bits, p.D2_bits) if p.dtype == "bf16" else (p.D1, p.D2)
    terms, loss, ga, gb = run(da, db, gt, 0.1, p.H, p.W, p.H, p.W)
    b_rows = np.sort(np.concatenate([rng.choice(p.N, 448, replace=False), gt[:64, 1]])).astype(np.int32)
    a_rows = np.unique(gt[:, 0])
    ra, rb = check_grads(ga, gb, p.D1, p.D2, gt, 0.1, b_rows=b_rows, a_rows=a_rows)
    log("grad 512x384", p.dtype, "err/tol", ra, rb)


def test_grad_bench_size_invariants():
    """The bench's workload (137626 pairs on the 512x384 bf16 pair): every softmax sums to
    1, so dB sums to zero over its rows; scaling either map scales all scores alike, so
    sum(dA * A) = sum(dB * B).  Both within the accumulated fp32 rounding."""
    p = workloads.config_pair(2)
    gt = workloads.gt_pairs(p)
    terms, loss, ga, gb = run(p.D1_bits, p.D2_bits, gt, 0.1, p.H, p.W, p.H, p.W)
    assert np.isfinite(ga).all() and np.isfinite(gb).all()
    colsum = np.abs(gb.astype(np.float64).sum(axis=0)).max()
    scale = np.abs(gb.astype(np.float64)).sum(axis=0).max()
    assert colsum <= 1e-4 * scale, (colsum, scale)
    lhs = float((ga.astype(np.float64) * p.D1).sum())
    rhs = float((gb.astype(np.float64) * p.D2).sum())
    assert abs(lhs - rhs) <= 1e-4 * max(abs(lhs), 1.0), (lhs, rhs)
    log("grad bench size", colsum, scale, lhs, rhs)
