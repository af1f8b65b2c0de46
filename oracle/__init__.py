"""CPU oracle for dense NN search and reciprocal matching -- TEST INFRASTRUCTURE ONLY.

Loads ``liboracle.so`` (plain C, binary64; source ``oracle.c`` beside this file)
with ctypes.  Only the test suite, the smoke check and the benchmark's CPU
baseline may import this package; the matching library never does.

Inputs are fp32 numpy arrays holding exactly the values the GPU library
receives (bf16 maps are passed as their exact fp32 widening).

``metric`` selects what "nearest" means: INNER (0, descriptor maps: largest
inner product) or NEG_SQ_L2 (1, pointmaps: smallest Euclidean distance; the
returned scores are minus the squared distances).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

INNER, NEG_SQ_L2 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (-O2, no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _bind(lib):
    P = ctypes.c_void_p
    i64, i32, f64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    lib.orc_nn.argtypes = [P, i64, P, i64, i32, i32, P, P, P]
    lib.orc_nn.restype = ctypes.c_int
    lib.orc_nn_rows.argtypes = [P, P, i64, P, i64, i32, i32, P, P, P]
    lib.orc_nn_rows.restype = ctypes.c_int
    lib.orc_similarity_pairs.argtypes = [P, P, i32, P, P, i64, P]
    lib.orc_similarity_pairs.restype = ctypes.c_int
    lib.orc_mutual.argtypes = [P, i64, P, i64, P, i64]
    lib.orc_mutual.restype = ctypes.c_int64
    lib.orc_fast.argtypes = [P, i32, i32, P, i64, i32, i32, i32, i32, i32, i32, f64, P, i64, P, P,
                             P, P]
    lib.orc_fast.restype = ctypes.c_int
    lib.orc_nn_metric.argtypes = [P, i64, P, i64, i32, i32, i32, P, P, P]
    lib.orc_nn_metric.restype = ctypes.c_int
    lib.orc_nn_rows_metric.argtypes = [P, P, i64, P, i64, i32, i32, i32, P, P, P]
    lib.orc_nn_rows_metric.restype = ctypes.c_int
    lib.orc_similarity_pairs_metric.argtypes = [P, P, i32, i32, P, P, i64, P]
    lib.orc_similarity_pairs_metric.restype = ctypes.c_int
    lib.orc_fast_metric.argtypes = [P, i32, i32, P, i64, i32, i32, i32, i32, i32, i32, i32, f64, P, i64,
                                    P, P, P, P]
    lib.orc_fast_metric.restype = ctypes.c_int
    lib.orc_fast_ex.argtypes = lib.orc_fast_metric.argtypes + [P, P, P]
    lib.orc_fast_ex.restype = ctypes.c_int
    lib.orc_infonce.argtypes = [P, i64, P, i64, i32, P, i64, f64, i32, P, P]
    lib.orc_infonce.restype = ctypes.c_int
    lib.orc_infonce_grad.argtypes = [P, i64, P, i64, i32, P, i64, f64, P, i64, i32, P, P, P]
    lib.orc_infonce_grad.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a.reshape(a.shape[0], -1) if a.ndim != 2 else a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


class Oracle:
    """The oracle's entry points bound to one compiled library (the default one, or
    another build of the same source, e.g. a deliberately broken copy in a test)."""

    def __init__(self, libpath=None):
        self._path = libpath
        self._own = None

    @property
    def lib(self):
        if self._path is None:
            return _load()
        if self._own is None:
            self._own = _bind(ctypes.CDLL(self._path))
        return self._own

    def nn(self, q, db, nthreads=None, metric=INNER):
        """Lowest-index argmax_k score(q[i], db[k]) per query row; returns (idx, top1, top2)."""
        lib = self.lib
        q, db = _f32(q), _f32(db)
        assert q.shape[1] == db.shape[1]
        nq = q.shape[0]
        idx = np.empty(nq, np.int32)
        t1 = np.empty(nq, np.float64)
        t2 = np.empty(nq, np.float64)
        rc = lib.orc_nn_metric(_ptr(q), nq, _ptr(db), db.shape[0], q.shape[1], metric,
                               nthreads or default_threads(), _ptr(idx), _ptr(t1), _ptr(t2))
        assert rc == 0, rc
        return idx, t1, t2

    def nn_rows(self, qmap, rows, db, nthreads=None, metric=INNER):
        """nn() for the query rows qmap[rows]."""
        lib = self.lib
        qmap, db = _f32(qmap), _f32(db)
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        n = rows.shape[0]
        idx = np.empty(n, np.int32)
        t1 = np.empty(n, np.float64)
        t2 = np.empty(n, np.float64)
        rc = lib.orc_nn_rows_metric(_ptr(qmap), _ptr(rows), n, _ptr(db), db.shape[0], qmap.shape[1], metric,
                                    nthreads or default_threads(), _ptr(idx), _ptr(t1), _ptr(t2))
        assert rc == 0, rc
        return idx, t1, t2

    def similarity_pairs(self, A, B, ia, ib, metric=INNER):
        """binary64 score(A[ia[t]], B[ib[t]]) for each t."""
        lib = self.lib
        A, B = _f32(A), _f32(B)
        ia = np.ascontiguousarray(ia, dtype=np.int32)
        ib = np.ascontiguousarray(ib, dtype=np.int32)
        out = np.empty(ia.shape[0], np.float64)
        rc = lib.orc_similarity_pairs_metric(_ptr(A), _ptr(B), A.shape[1], metric, _ptr(ia), _ptr(ib),
                                             ia.shape[0], _ptr(out))
        assert rc == 0, rc
        return out

    def mutual(self, nn12, nn21):
        """Reciprocal pairs (i, nn12[i]) with nn21[nn12[i]] == i, ascending i; int32 [m, 2]."""
        lib = self.lib
        nn12 = np.ascontiguousarray(nn12, dtype=np.int32)
        nn21 = np.ascontiguousarray(nn21, dtype=np.int32)
        cap = max(1, min(nn12.shape[0], nn21.shape[0]))
        pairs = np.empty((cap, 2), np.int32)
        m = lib.orc_mutual(_ptr(nn12), nn12.shape[0], _ptr(nn21), nn21.shape[0], _ptr(pairs), cap)
        assert m >= 0, m
        return pairs[:m].copy()

    def mutual_nn(self, A, B, nthreads=None, metric=INNER):
        """Brute-force mutual NN of two maps: (pairs, nn12, top1_12, top2_12, nn21, top1_21, top2_21)."""
        n12, a1, a2 = self.nn(A, B, nthreads, metric)
        n21, b1, b2 = self.nn(B, A, nthreads, metric)
        return self.mutual(n12, n21), n12, a1, a2, n21, b1, b2

    def fast(self, A, H1, W1, B, stride, offset, max_iters, seed_limit=-1, nthreads=None, eps=1e-5,
             metric=INNER):
        """Fast reciprocal matching seeded on image 1's grid.

        Returns dict(pairs int32 [m,2] ascending in u, clean uint8 [m], active int64 [T],
        nn_queries int, fresh int64 [T] (pixels live at iteration t and in no earlier one),
        seed_u int32 [ns] (where seed c's chain converged, -1 if it did not within T),
        seed_clean uint8 [ns] (every decision on seed c's chain cleared eps))."""
        lib = self.lib
        A, B = _f32(A), _f32(B)
        assert A.shape[0] == H1 * W1 and A.shape[1] == B.shape[1]
        ns = len(range(offset, H1, stride)) * len(range(offset, W1, stride)) if stride > 0 else 0
        if seed_limit >= 0:
            ns = min(ns, seed_limit)
        cap = max(1, ns)
        pairs = np.empty((cap, 2), np.int32)
        clean = np.zeros(cap, np.uint8)
        active = np.zeros(max(1, max_iters), np.int64)
        fresh = np.zeros(max(1, max_iters), np.int64)
        seed_u = np.full(cap, -1, np.int32)
        seed_clean = np.ones(cap, np.uint8)
        npairs = ctypes.c_int64(0)
        nq = ctypes.c_int64(0)
        rc = lib.orc_fast_ex(_ptr(A), H1, W1, _ptr(B), B.shape[0], A.shape[1], metric, stride, offset,
                             max_iters, seed_limit, nthreads or default_threads(), eps, _ptr(pairs), cap,
                             ctypes.byref(npairs), _ptr(clean), _ptr(active), ctypes.byref(nq), _ptr(fresh),
                             _ptr(seed_u), _ptr(seed_clean))
        assert rc == 0, rc
        m = npairs.value
        return dict(pairs=pairs[:m].copy(), clean=clean[:m].copy(), active=active[:max_iters].copy(),
                    nn_queries=nq.value, fresh=fresh[:max_iters].copy(), seed_u=seed_u[:ns].copy(),
                    seed_clean=seed_clean[:ns].copy())


    def infonce(self, A, B, gt, tau, nthreads=None):
        """Matching loss terms LSE_i - <A[i], B[j]> / tau per ground-truth pair (i, j), the
        log-sum-exp over every row of B; returns (terms float64 [n_gt], total)."""
        lib = self.lib
        A, B = _f32(A), _f32(B)
        gt = np.ascontiguousarray(np.asarray(gt, dtype=np.int32).reshape(-1, 2))
        terms = np.empty(gt.shape[0], np.float64)
        total = ctypes.c_double(0.0)
        rc = lib.orc_infonce(_ptr(A), A.shape[0], _ptr(B), B.shape[0], A.shape[1], _ptr(gt), gt.shape[0],
                             float(tau), nthreads or default_threads(), _ptr(terms), ctypes.byref(total))
        assert rc == 0, rc
        return terms, total.value


    def infonce_grad(self, A, B, gt, tau, b_rows=None, nthreads=None):
        """Gradient of the summed matching loss: (dA float64 [n1, d], dB float64 [len(b_rows), d],
        colmass float64 [len(b_rows)] = sum_t softmax_t[k]) for the listed rows k of B (all
        rows when b_rows is None)."""
        lib = self.lib
        A, B = _f32(A), _f32(B)
        gt = np.ascontiguousarray(np.asarray(gt, dtype=np.int32).reshape(-1, 2))
        rows = np.arange(B.shape[0], dtype=np.int32) if b_rows is None else \
            np.ascontiguousarray(b_rows, dtype=np.int32)
        d = A.shape[1]
        dA = np.empty((A.shape[0], d), np.float64)
        dB = np.empty((max(1, rows.shape[0]), d), np.float64)
        mass = np.empty(max(1, rows.shape[0]), np.float64)
        rc = lib.orc_infonce_grad(_ptr(A), A.shape[0], _ptr(B), B.shape[0], d, _ptr(gt), gt.shape[0], float(tau),
                                  _ptr(rows), rows.shape[0], nthreads or default_threads(), _ptr(dA), _ptr(dB),
                                  _ptr(mass))
        assert rc == 0, rc
        return dA, dB[:rows.shape[0]], mass[:rows.shape[0]]


_default = Oracle()
nn = _default.nn
nn_rows = _default.nn_rows
similarity_pairs = _default.similarity_pairs
mutual = _default.mutual
mutual_nn = _default.mutual_nn
fast = _default.fast
infonce = _default.infonce
infonce_grad = _default.infonce_grad
