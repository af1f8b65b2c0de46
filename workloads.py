"""Seeded synthetic descriptor-map pairs shaped like MASt3R's matching workloads
(and pointmap pairs shaped like DUSt3R's, see make_pointmaps).

This module only makes inputs.  It holds none of the matching arithmetic (no
similarity, no nearest-neighbour search, no reciprocity test): the CPU oracle
and the HIP library both consume exactly the arrays built here.

Shape of the data, after the pages:
  * one d = 24 local descriptor per pixel, L2-normalised ("Grounding Image
    Matching in 3D" / MASt3R dissection, section 3 "Napkin Formula": the matching
    head's output D_v[i] is L2-normalised and d is deliberately small, 24;
    DUSt3R/MASt3R explained, the paragraph on MASt3R's dense local-feature head);
  * pairs at MASt3R's 512-pixel working resolution (DUSt3R/MASt3R explained,
    the training paragraph: trained at 224 then 512 pixels).
Real descriptors come from a trained network and are spatially smooth; here
image 1 holds i.i.d. random unit vectors and image 2 is a warped, noisy,
partly occluded copy of it, so the planted correspondence src() is known.

Recipe (all draws from numpy's PCG64 generator seeded per pair, in this order:
image-1 normals, warp parameters, jitter, noise, occlusion subset, occluder
vectors):
  1. D1[p] = g / |g| with g ~ N(0, 1)^d in float64.
  2. Backward warp: every image-2 pixel q gets an integer source pixel
     src(q) in image 1 (clamped to the image), D2[q] = D1[src(q)].
  3. D2 += sigma * N(0, 1) per component.
  4. floor(rho * N) image-2 pixels, a uniformly random subset, are replaced by
     fresh unit vectors; their src is -1 (occluded: no true match).
  5. If sigma > 0 every D2 row is renormalised (rows left untouched stay exact
     copies, which the noise-free pins rely on).  Both maps are cast to fp32.
  6. bf16 workloads round both fp32 maps to bf16 (round to nearest even) and do
     not renormalise; the oracle receives the rounded values widened exactly.
round(x) = floor(x + 0.5); clamp() clips to [0, H-1] x [0, W-1].
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

D_DEFAULT = 24


@dataclasses.dataclass
class Pair:
    """One synthetic image pair.  Maps are row-major [H*W, d], pixel p = y*W + x."""
    name: str
    H: int
    W: int
    d: int
    dtype: str                      # "f32" or "bf16"
    D1: np.ndarray                  # float32 [N, d]; for bf16 the exact widened values
    D2: np.ndarray                  # float32 [N, d]
    D1_bits: Optional[np.ndarray]   # int16 [N, d] bf16 bit patterns (bf16 only)
    D2_bits: Optional[np.ndarray]
    src: np.ndarray                 # int32 [N]: planted source pixel in image 1, -1 if occluded
    seed: int
    stride: int = 8
    offset: int = 4
    max_iters: int = 10

    @property
    def N(self) -> int:
        return self.H * self.W


# ----------------------------------------------------------------------------- helpers

def unit_rows(rng: np.random.Generator, n: int, d: int) -> np.ndarray:
    g = rng.standard_normal((n, d))
    return g / np.linalg.norm(g, axis=1, keepdims=True)


def _round_half_up(x: np.ndarray) -> np.ndarray:
    return np.floor(x + 0.5).astype(np.int64)


def _clamp_pix(y: np.ndarray, x: np.ndarray, H: int, W: int) -> np.ndarray:
    y = np.clip(y, 0, H - 1)
    x = np.clip(x, 0, W - 1)
    return (y * W + x).astype(np.int64)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 -> bf16 to nearest, ties to even (finite inputs); int16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    return r.astype(np.uint16).view(np.int16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    u = b.view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


# ----------------------------------------------------------------------------- warps

def _warp_shift(rng, H, W, shift=(3, 2)):
    ys, xs = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    ys, xs = ys.ravel(), xs.ravel()
    j = rng.integers(-1, 2, size=(H * W, 2))          # +-1 jitter per pixel
    return _clamp_pix(ys - shift[0] - j[:, 0], xs - shift[1] - j[:, 1], H, W)


def _affine_params(rng, H, W, max_disp=30.0):
    M = rng.uniform(-0.06, 0.06, size=(2, 2))
    t = rng.uniform(-20.0, 20.0, size=2)
    c = np.array([(H - 1) / 2.0, (W - 1) / 2.0])
    corners = np.array([[0, 0], [0, W - 1], [H - 1, 0], [H - 1, W - 1]], dtype=np.float64)
    disp = (corners - c) @ M.T + t
    m = np.abs(disp).max()
    if m > max_disp:                                    # an affine field peaks at a corner
        M = M * (max_disp / m)
        t = t * (max_disp / m)
    return M, t, c


def _warp_affine(rng, H, W, max_disp=30.0):
    M, t, c = _affine_params(rng, H, W, max_disp)
    ys, xs = np.meshgrid(np.arange(H, dtype=np.float64), np.arange(W, dtype=np.float64), indexing="ij")
    q = np.stack([ys.ravel(), xs.ravel()], axis=1)
    delta = (q - c) @ M.T + t
    s = q - delta
    return _clamp_pix(_round_half_up(s[:, 0]), _round_half_up(s[:, 1]), H, W)


def _warp_homography(rng, H, W, max_rot_deg=25.0, scale=(0.7, 1.4), max_t=30.0, max_p=0.1):
    theta = math.radians(rng.uniform(-max_rot_deg, max_rot_deg))
    s = math.exp(rng.uniform(math.log(scale[0]), math.log(scale[1])))
    t = rng.uniform(-max_t, max_t, size=2)
    p = rng.uniform(-max_p, max_p, size=2) / max(H, W)
    cx, cy = (W - 1) / 2.0, (H - 1) / 2.0
    A = np.array([[s * math.cos(theta), -s * math.sin(theta), t[0]],
                  [s * math.sin(theta), s * math.cos(theta), t[1]],
                  [p[0], p[1], 1.0]])
    Tc = np.array([[1, 0, cx], [0, 1, cy], [0, 0, 1.0]])
    Tm = np.array([[1, 0, -cx], [0, 1, -cy], [0, 0, 1.0]])
    Hm = Tc @ A @ Tm                                   # image-2 (x, y, 1) -> image-1
    ys, xs = np.meshgrid(np.arange(H, dtype=np.float64), np.arange(W, dtype=np.float64), indexing="ij")
    P = np.stack([xs.ravel(), ys.ravel(), np.ones(H * W)], axis=0)
    Q = Hm @ P
    x1 = Q[0] / Q[2]
    y1 = Q[1] / Q[2]
    return _clamp_pix(_round_half_up(y1), _round_half_up(x1), H, W)


# ----------------------------------------------------------------------------- generic pair

def make_pair(H: int, W: int, d: int, seed: int, warp: str = "shift", sigma: float = 0.1,
              rho: float = 0.2, dtype: str = "f32", name: str = "custom", stride: int = 8,
              offset: Optional[int] = None, max_iters: int = 10) -> Pair:
    """A planted pair following the module recipe; warp in {"shift", "affine", "homography", "identity"}."""
    N = H * W
    rng = np.random.Generator(np.random.PCG64(seed))
    D1 = unit_rows(rng, N, d)
    if warp == "shift":
        src = _warp_shift(rng, H, W)
    elif warp == "affine":
        src = _warp_affine(rng, H, W)
    elif warp == "homography":
        src = _warp_homography(rng, H, W)
    elif warp == "identity":
        src = np.arange(N, dtype=np.int64)
    else:
        raise ValueError(f"unknown warp {warp!r}")
    D2 = D1[src].copy()
    if sigma > 0:
        D2 += sigma * rng.standard_normal((N, d))
    src = src.astype(np.int32)
    k = int(math.floor(rho * N))
    if k > 0:
        occ = rng.choice(N, size=k, replace=False)
        D2[occ] = unit_rows(rng, k, d)
        src[occ] = -1
    if sigma > 0:
        D2 /= np.linalg.norm(D2, axis=1, keepdims=True)
    D1f = D1.astype(np.float32)
    D2f = D2.astype(np.float32)
    b1 = b2 = None
    if dtype == "bf16":
        b1, b2 = f32_to_bf16_bits(D1f), f32_to_bf16_bits(D2f)
        D1f, D2f = bf16_bits_to_f32(b1), bf16_bits_to_f32(b2)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    if offset is None:
        offset = stride // 2
    return Pair(name=name, H=H, W=W, d=d, dtype=dtype, D1=D1f, D2=D2f, D1_bits=b1, D2_bits=b2,
                src=src, seed=seed, stride=stride, offset=offset, max_iters=max_iters)


# ----------------------------------------------------------------------------- image collections

def make_collection(n_images: int, H: int, W: int, d: int, seed: int, sigma: float = 0.15, rho: float = 0.3,
                    dtype: str = "f32"):
    """A collection of n_images maps that all view one scene: a base map D0 of unit rows,
    and image k = D0 warped by its own random affine field (the pair recipe's warp), plus
    sigma noise and rho occlusion, renormalised.  Any two images therefore share content,
    as the pairs of a reconstruction's pair graph do.  Returns (maps float32 [n, N, d],
    bf16 bits [n, N, d] or None, src int32 [n, N]: the D0 pixel each pixel shows, -1 if
    occluded).  Draw order: D0, then per image: warp, noise, occlusion subset, occluders."""
    N = H * W
    rng = np.random.Generator(np.random.PCG64(seed))
    D0 = unit_rows(rng, N, d)
    maps = np.empty((n_images, N, d), np.float32)
    srcs = np.empty((n_images, N), np.int32)
    for k in range(n_images):
        src = _warp_affine(rng, H, W)
        X = D0[src]
        if sigma > 0:
            X = X + sigma * rng.standard_normal((N, d))
        src = src.astype(np.int32)
        m = int(math.floor(rho * N))
        if m > 0:
            occ = rng.choice(N, size=m, replace=False)
            X[occ] = unit_rows(rng, m, d)
            src[occ] = -1
        X /= np.linalg.norm(X, axis=1, keepdims=True)
        maps[k] = X.astype(np.float32)
        srcs[k] = src
    bits = None
    if dtype == "bf16":
        bits = f32_to_bf16_bits(maps)
        maps = bf16_bits_to_f32(bits)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return maps, bits, srcs


def all_edges(n_images: int):
    """Every unordered pair (i, j), i < j, in lexicographic order (the complete pair graph)."""
    return np.array([(i, j) for i in range(n_images) for j in range(i + 1, n_images)], np.int32)


# ----------------------------------------------------------------------------- pointmaps

def make_pointmaps(H: int, W: int, seed: int, warp: str = "affine", sigma: float = 0.005, rho: float = 0.3,
                   name: str = "pointmaps", stride: int = 8, offset: Optional[int] = None,
                   max_iters: int = 10) -> Pair:
    """A planted pair of pointmaps (d = 3, metres, both in camera 1's frame).

    After the pages (DUSt3R/MASt3R explained: a pointmap holds, per pixel, the 3D
    point that pixel observes; both views are expressed in the first camera's frame,
    so where the images overlap their pointmaps hold the same 3D points):
      1. image 1 sees a smooth surface: depth z(y, x) = 3 + 0.4 sin(a) cos(b) + 0.3 (x/W - 1/2)
         with a, b linear in the pixel coordinates (random frequencies and phases), back-
         projected through a pinhole camera with focal length W pixels and the principal
         point at the image centre: X1[p] = z ((x - cx)/W, (y - cy)/W, 1);
      2. image 2 is a backward warp of it (the descriptor warps): X2[q] = X1[src(q)];
      3. X2 += sigma * N(0, 1) per coordinate (metres);
      4. floor(rho N) image-2 pixels are replaced by points drawn uniformly in the
         bounding box of X1 (src = -1);
      5. both maps are cast to fp32 (no normalisation: pointmaps are not unit vectors).
    Draw order: surface parameters, warp, noise, occlusion subset, occluder points."""
    N = H * W
    rng = np.random.Generator(np.random.PCG64(seed))
    fa, fb = rng.uniform(1.0, 3.0, size=2)
    pa, pb = rng.uniform(0.0, 2.0 * math.pi, size=2)
    ys, xs = np.meshgrid(np.arange(H, dtype=np.float64), np.arange(W, dtype=np.float64), indexing="ij")
    ys, xs = ys.ravel(), xs.ravel()
    z = 3.0 + 0.4 * np.sin(2 * math.pi * fa * xs / W + pa) * np.cos(2 * math.pi * fb * ys / H + pb) \
        + 0.3 * (xs / W - 0.5)
    cx, cy = (W - 1) / 2.0, (H - 1) / 2.0
    X1 = np.stack([z * (xs - cx) / W, z * (ys - cy) / W, z], axis=1)
    if warp == "shift":
        src = _warp_shift(rng, H, W)
    elif warp == "affine":
        src = _warp_affine(rng, H, W)
    elif warp == "identity":
        src = np.arange(N, dtype=np.int64)
    else:
        raise ValueError(f"unknown warp {warp!r}")
    X2 = X1[src].copy()
    if sigma > 0:
        X2 += sigma * rng.standard_normal((N, 3))
    src = src.astype(np.int32)
    k = int(math.floor(rho * N))
    if k > 0:
        occ = rng.choice(N, size=k, replace=False)
        lo, hi = X1.min(axis=0), X1.max(axis=0)
        X2[occ] = lo + (hi - lo) * rng.uniform(size=(k, 3))
        src[occ] = -1
    if offset is None:
        offset = stride // 2
    return Pair(name=name, H=H, W=W, d=3, dtype="f32", D1=X1.astype(np.float32), D2=X2.astype(np.float32),
                D1_bits=None, D2_bits=None, src=src, seed=seed, stride=stride, offset=offset,
                max_iters=max_iters)


# ----------------------------------------------------------------------------- the five workloads

CONFIGS = {
    0: dict(name="tiny-64x48-f32", H=64, W=48, warp="shift", sigma=0.1, rho=0.2, dtype="f32",
            seed=0, stride=8, max_iters=10, op="mutual+fast"),
    1: dict(name="pair-512x384-f32", H=512, W=384, warp="affine", sigma=0.15, rho=0.3, dtype="f32",
            seed=1, stride=8, max_iters=10, op="fast"),
    2: dict(name="pair-512x384-bf16-bruteforce", H=512, W=384, warp="affine", sigma=0.15, rho=0.3,
            dtype="bf16", seed=1, stride=8, max_iters=10, op="mutual"),
    3: dict(name="batch64-512x384-f32", H=512, W=384, warp="affine", sigma=0.15, rho=0.3, dtype="f32",
            seed=1000, stride=8, max_iters=10, op="fast", batch=64),
    4: dict(name="pair-1024x768-bf16", H=1024, W=768, warp="homography", sigma=0.2, rho=0.4,
            dtype="bf16", seed=4, stride=8, max_iters=15, op="fast"),
}


def config_pair(cfg: int, b: int = 0, d: int = D_DEFAULT) -> Pair:
    """Pair b of workload cfg (b > 0 only for the 64-pair batch, seeded 1000 + b)."""
    c = CONFIGS[cfg]
    seed = c["seed"] + b
    return make_pair(c["H"], c["W"], d, seed, warp=c["warp"], sigma=c["sigma"], rho=c["rho"],
                     dtype=c["dtype"], name=c["name"], stride=c["stride"], max_iters=c["max_iters"])


def gt_pairs(p: Pair) -> np.ndarray:
    """Ground-truth correspondences of a planted pair: (src[j], j) for every pixel j of
    image 2 that is not occluded, int32 [n_gt, 2] ascending in j (several j may share
    one source pixel)."""
    j = np.nonzero(p.src >= 0)[0]
    return np.stack([p.src[j], j], axis=1).astype(np.int32)


def stack_pairs(pairs):
    """Stack pairs into [B, N, d] fp32 arrays (and bf16 bits if any)."""
    D1 = np.stack([p.D1 for p in pairs])
    D2 = np.stack([p.D2 for p in pairs])
    if pairs[0].dtype == "bf16":
        return D1, D2, np.stack([p.D1_bits for p in pairs]), np.stack([p.D2_bits for p in pairs])
    return D1, D2, None, None

