"""Accuracy of fast reciprocal matching against a planted correspondence field.

"DUSt3R and MASt3R explained" (the paragraph on MASt3R's fast reciprocal matching)
reports that matching from a sparse grid of seeds is not only faster than the full
mutual-NN set but more accurate: the points that survive the iterated reciprocal
test are disproportionately correct.  This study measures that claim on synthetic
planted pairs (workloads.make_pair: image 2 is a warped, noisy, partly occluded copy
of image 1, so the true source pixel src(q) of every image-2 pixel is known):

  precision = correct matches / matches, a match (u, v) being correct when
              src(v) = u;
  recall    = correct matches / recoverable pixels, the image-1 pixels that are the
              source of some unoccluded image-2 pixel (each can be matched once);

as functions of the seed stride s (s = 1 seeds every pixel and returns the brute-force
mutual set), the iteration cap T, the noise sigma and the occlusion rate rho, with the
GPU time of each call.  An optional symmetric pass also seeds image 2 and keeps the
union of both directions' matches.

Run:  python -m dense_grounded_image_amd.study_accuracy [--quick]
"""
from __future__ import annotations

import argparse
import json
import sys

import numpy as np


def planted_scores(pairs, src):
    """(matches, correct, precision, recall) of a match list against src()."""
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    recoverable = np.unique(src[src >= 0]).size
    if len(pairs) == 0:
        return 0, 0, float("nan"), 0.0
    correct = int((src[pairs[:, 1]] == pairs[:, 0]).sum())
    return len(pairs), correct, correct / len(pairs), correct / max(recoverable, 1)


def gpu_matcher():
    """fast(A, B, H, W, stride, offset, T) -> (pairs [m, 2] int64, seconds) on cuda:0."""
    import torch
    import dense_grounded_image_amd as mr

    def fast(A, B, H, W, stride, offset, T):
        a = torch.from_numpy(np.ascontiguousarray(A).reshape(H, W, -1)).cuda()[None]
        b = torch.from_numpy(np.ascontiguousarray(B).reshape(H, W, -1)).cuda()[None]
        f = mr.FastReciprocal(a, b, stride, offset, T)
        f(a, b)                                  # warm-up (and workspace first touch)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        pairs, n, _ = f(a, b)
        t1.record()
        torch.cuda.synchronize()
        return mr.matches(pairs, n), t0.elapsed_time(t1) * 1e-3
    return fast


def study(H, W, d, seed, strides, iters, sigmas, rhos, fast, symmetric=False, warp="affine"):
    """One row per (sigma, rho, stride, T)."""
    import workloads
    rows = []
    for sigma in sigmas:
        for rho in rhos:
            p = workloads.make_pair(H, W, d, seed, warp=warp, sigma=sigma, rho=rho)
            for s in strides:
                for T in iters:
                    off = s // 2
                    pairs, sec = fast(p.D1, p.D2, H, W, s, off, T)
                    row = dict(sigma=sigma, rho=rho, stride=s, T=T, seconds=sec)
                    m, c, prec, rec = planted_scores(pairs, p.src)
                    row.update(matches=m, correct=c, precision=prec, recall=rec)
                    if symmetric:
                        back, sec2 = fast(p.D2, p.D1, H, W, s, off, T)
                        both = {tuple(x) for x in pairs.tolist()} | {(int(v), int(u)) for u, v in back.tolist()}
                        m2, c2, prec2, rec2 = planted_scores(sorted(both), p.src)
                        row.update(sym_matches=m2, sym_precision=prec2, sym_recall=rec2, sym_seconds=sec + sec2)
                    rows.append(row)
    return rows


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--quick", action="store_true", help="a 128x96 pair and a smaller grid")
    ap.add_argument("--symmetric", action="store_true", help="also seed image 2 and take the union")
    args = ap.parse_args(argv)
    if args.quick:
        H, W, strides, iters, sigmas, rhos = 128, 96, (1, 4, 8), (1, 10), (0.15,), (0.3,)
    else:
        H, W = 512, 384
        strides, iters, sigmas, rhos = (1, 2, 4, 8, 16), (1, 2, 3, 10), (0.05, 0.15, 0.3), (0.0, 0.3)
    rows = study(H, W, 24, 1, strides, iters, sigmas, rhos, gpu_matcher(), symmetric=args.symmetric)
    for r in rows:
        print(json.dumps(r), flush=True)
    print("| sigma | rho | stride | T | matches | precision | recall | ms |", file=sys.stderr)
    for r in rows:
        print("| %.2f | %.1f | %d | %d | %d | %.4f | %.4f | %.3f |" % (
            r["sigma"], r["rho"], r["stride"], r["T"], r["matches"], r["precision"], r["recall"],
            r["seconds"] * 1e3), file=sys.stderr)


if __name__ == "__main__":
    main()
