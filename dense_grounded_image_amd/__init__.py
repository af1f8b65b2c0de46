"""Dense NN search and reciprocal matching of per-pixel descriptor maps on MI355X.

A thin ctypes binding over ``libmr.so`` (C ABI declared in include/mr.h).  Every
step of the computation runs in the library's HIP kernels; this module only
marshals torch tensors (device memory and the current stream) into the C calls.
There is no CPU fallback: if the library is missing or no GPU is present, the
calls raise.

Maps are torch tensors [H, W, d] or [B, H, W, d] (float32 or bfloat16, d <= 64,
bf16 needs d % 8 == 0), contiguous, on a ROCm device, one L2-normalised
descriptor per pixel; pixel id p = y*W + x.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmr.so")

MR_F32, MR_BF16 = 0, 1
MR_OP_NN_ARGMAX, MR_OP_MUTUAL_NN, MR_OP_FAST_RECIPROCAL = 0, 1, 2
MR_OP_POINT_NN, MR_OP_POINT_MUTUAL_NN, MR_OP_POINT_FAST_RECIPROCAL = 3, 4, 5
MR_OP_FAST_RECIPROCAL_GRAPH = 6
MR_OP_INFONCE = 7
MR_OP_INFONCE_BACKWARD = 8
STATUS = {0: "MR_OK", 1: "MR_ERR_NULL", 2: "MR_ERR_SHAPE", 3: "MR_ERR_DTYPE", 4: "MR_ERR_PARAM",
          5: "MR_ERR_WORKSPACE", 6: "MR_ERR_CAPACITY", 7: "MR_ERR_DEVICE", 8: "MR_ERR_SCRATCH"}

EXPORTS = ("mr_workspace_bytes", "mr_status_str", "mr_seed_count", "mr_nn_argmax", "mr_mutual_nn",
           "mr_fast_reciprocal", "mr_fast_reciprocal_static", "mr_fast_reciprocal_graph", "mr_point_nn", "mr_point_mutual_nn",
           "mr_point_fast_reciprocal", "mr_infonce_forward", "mr_infonce_backward",
           "mr_profile_begin", "mr_profile_end", "mr_profile_end_each", "mr_profile_end_queries")


class MrMap(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("batch", ctypes.c_int32), ("h", ctypes.c_int32),
                ("w", ctypes.c_int32), ("d", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class MrError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({status_str(code)})")


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmr.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    MP = ctypes.POINTER(MrMap)
    lib.mr_workspace_bytes.argtypes = [ctypes.c_int, MP, MP, i64, i32, i32]
    lib.mr_workspace_bytes.restype = sz
    lib.mr_status_str.argtypes = [ctypes.c_int]
    lib.mr_status_str.restype = ctypes.c_char_p
    lib.mr_seed_count.argtypes = [i32, i32, i32, i32]
    lib.mr_seed_count.restype = i64
    lib.mr_nn_argmax.argtypes = [MP, MP, P, i64, P, P, P, sz, P]
    lib.mr_nn_argmax.restype = ctypes.c_int
    lib.mr_mutual_nn.argtypes = [MP, MP, P, P, P, i64, P, P, sz, P]
    lib.mr_mutual_nn.restype = ctypes.c_int
    lib.mr_fast_reciprocal.argtypes = [MP, MP, i32, i32, i32, P, i64, P, P, P, sz, P]
    lib.mr_fast_reciprocal.restype = ctypes.c_int
    lib.mr_fast_reciprocal_static.argtypes = [MP, MP, i32, i32, i32, P, i64, P, P, P]
    lib.mr_fast_reciprocal_static.restype = ctypes.c_int
    lib.mr_fast_reciprocal_graph.argtypes = [MP, P, i32, i32, i32, i32, P, i64, P, P, P, sz, P]
    lib.mr_fast_reciprocal_graph.restype = ctypes.c_int
    lib.mr_point_nn.argtypes = lib.mr_nn_argmax.argtypes
    lib.mr_point_nn.restype = ctypes.c_int
    lib.mr_point_mutual_nn.argtypes = lib.mr_mutual_nn.argtypes
    lib.mr_point_mutual_nn.restype = ctypes.c_int
    lib.mr_point_fast_reciprocal.argtypes = lib.mr_fast_reciprocal.argtypes
    lib.mr_point_fast_reciprocal.restype = ctypes.c_int
    lib.mr_infonce_forward.argtypes = [MP, MP, P, i64, ctypes.c_float, P, P, P, sz, P]
    lib.mr_infonce_forward.restype = ctypes.c_int
    lib.mr_infonce_backward.argtypes = [MP, MP, P, i64, ctypes.c_float, P, P, P, P, P, sz, P]
    lib.mr_infonce_backward.restype = ctypes.c_int
    lib.mr_profile_begin.argtypes = [i32]
    lib.mr_profile_begin.restype = ctypes.c_int
    lib.mr_profile_end.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    lib.mr_profile_end.restype = ctypes.c_int
    lib.mr_profile_end_each.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64), P, i32]
    lib.mr_profile_end_each.restype = ctypes.c_int
    lib.mr_profile_end_queries.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64), P, P, i32]
    lib.mr_profile_end_queries.restype = ctypes.c_int
    _lib = lib
    return lib


def status_str(code: int) -> str:
    return load_library().mr_status_str(code).decode()


def seed_count(h: int, w: int, stride: int, offset: int) -> int:
    return int(load_library().mr_seed_count(h, w, stride, offset))


# ----------------------------------------------------------------------------- marshalling

def _torch():
    import torch
    return torch


def _as_map(t) -> MrMap:
    torch = _torch()
    if t.dim() == 3:
        t = t.unsqueeze(0)
    if t.dim() != 4:
        raise ValueError("a descriptor map is [H, W, d] or [B, H, W, d]")
    if not t.is_cuda:
        raise ValueError("descriptor maps must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("descriptor maps must be contiguous")
    if t.dtype == torch.float32:
        dt = MR_F32
    elif t.dtype == torch.bfloat16:
        dt = MR_BF16
    else:
        raise ValueError(f"unsupported dtype {t.dtype}")
    B, H, W, d = t.shape
    return MrMap(t.data_ptr(), B, H, W, d, dt)


def _stream(t) -> int:
    return _torch().cuda.current_stream(t.device).cuda_stream


def _check(fn, rc):
    if rc != 0:
        raise MrError(fn, rc)


def _workspace(nbytes: int, device, ws=None):
    torch = _torch()
    nbytes = max(int(nbytes), 256)
    if ws is not None and ws.numel() >= nbytes:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _batched(t):
    return t.unsqueeze(0) if t.dim() == 3 else t


def workspace_bytes(op: int, a, b, n_q: int = 0, stride: int = 1, offset: int = 0) -> int:
    ma, mb = _as_map(a), _as_map(b)
    return int(load_library().mr_workspace_bytes(op, ctypes.byref(ma), ctypes.byref(mb), n_q, stride, offset))


# ----------------------------------------------------------------------------- entry points

def _nn(point, q, db, q_idx, with_score, ws):
    torch = _torch()
    lib = load_library()
    squeeze = q.dim() == 3
    mq, mdb = _as_map(q), _as_map(db)
    B = mq.batch
    if q_idx is None:
        n = mq.h * mq.w
        qptr = None
    else:
        q_idx = q_idx.to(device=q.device, dtype=torch.int32).reshape(B, -1).contiguous()
        n = q_idx.shape[1]
        qptr = q_idx.data_ptr()
    out_idx = torch.empty((B, n), dtype=torch.int32, device=q.device)
    out_score = torch.empty((B, n), dtype=torch.float32, device=q.device) if with_score else None
    op, fn = (MR_OP_POINT_NN, "mr_point_nn") if point else (MR_OP_NN_ARGMAX, "mr_nn_argmax")
    need = lib.mr_workspace_bytes(op, ctypes.byref(mq), ctypes.byref(mdb), n, 1, 0)
    ws = _workspace(need, q.device, ws)
    rc = getattr(lib, fn)(ctypes.byref(mq), ctypes.byref(mdb), qptr, n, out_idx.data_ptr(),
                          out_score.data_ptr() if with_score else None, ws.data_ptr(), ws.numel(), _stream(q))
    _check(fn, rc)
    if squeeze:
        out_idx = out_idx[0]
        out_score = out_score[0] if with_score else None
    return (out_idx, out_score) if with_score else out_idx


def nn_argmax(q, db, q_idx=None, with_score: bool = False, ws=None):
    """NN in db of every (or every listed) pixel of q, lowest index on ties.

    q, db: [H, W, d] or [B, H, W, d].  q_idx: None or int32 [n] / [B, n] pixel ids of q.
    Returns idx int32 [B, n] (and fp32 scores if with_score); B dim dropped for 3-D input."""
    return _nn(False, q, db, q_idx, with_score, ws)


def point_nn(q, db, q_idx=None, with_dist2: bool = False, ws=None):
    """Nearest point in pointmap db of every (or every listed) pixel of pointmap q (fp32,
    d <= 4), lowest index on ties; with_dist2 also returns the fp32 squared distances."""
    return _nn(True, q, db, q_idx, with_dist2, ws)


def _mutual(point, a, b, ws):
    torch = _torch()
    lib = load_library()
    ma, mb = _as_map(a), _as_map(b)
    B, Na, Nb = ma.batch, ma.h * ma.w, mb.h * mb.w
    cap = max(1, min(Na, Nb))
    dev = a.device
    nn_ab = torch.empty((B, Na), dtype=torch.int32, device=dev)
    nn_ba = torch.empty((B, Nb), dtype=torch.int32, device=dev)
    pairs = torch.empty((B, cap, 2), dtype=torch.int32, device=dev)
    n_pairs = torch.empty((B,), dtype=torch.int64, device=dev)
    op, fn = (MR_OP_POINT_MUTUAL_NN, "mr_point_mutual_nn") if point else (MR_OP_MUTUAL_NN, "mr_mutual_nn")
    need = lib.mr_workspace_bytes(op, ctypes.byref(ma), ctypes.byref(mb), 0, 1, 0)
    ws = _workspace(need, dev, ws)
    rc = getattr(lib, fn)(ctypes.byref(ma), ctypes.byref(mb), nn_ab.data_ptr(), nn_ba.data_ptr(),
                          pairs.data_ptr(), cap, n_pairs.data_ptr(), ws.data_ptr(), ws.numel(), _stream(a))
    _check(fn, rc)
    return pairs, n_pairs, nn_ab, nn_ba


def mutual_nn(a, b, ws=None):
    """Brute-force reciprocal NN.  Returns (pairs int32 [B, cap, 2], n_pairs int64 [B],
    nn_ab int32 [B, Na], nn_ba int32 [B, Nb]); pairs[b, :n_pairs[b]] ascending in i."""
    return _mutual(False, a, b, ws)


def point_mutual_nn(a, b, ws=None):
    """Brute-force reciprocal nearest points of two pointmaps; returns as mutual_nn."""
    return _mutual(True, a, b, ws)


class FastReciprocal:
    """Reusable call of the fast reciprocal scheme for fixed shapes: output and
    workspace buffers are allocated once, so repeated calls allocate nothing.
    static_scratch=True calls mr_fast_reciprocal_static, which takes no workspace (the
    library's fixed per-GPU scratch; descriptor maps only)."""

    def __init__(self, a, b, stride: int = 8, offset: Optional[int] = None, max_iters: int = 10,
                 record_active: bool = True, point: bool = False, static_scratch: bool = False):
        torch = _torch()
        self.lib = load_library()
        if static_scratch and point:
            raise ValueError("the static-scratch call covers descriptor maps only")
        self.static = bool(static_scratch)
        self.fn = self.lib.mr_point_fast_reciprocal if point else self.lib.mr_fast_reciprocal
        op = MR_OP_POINT_FAST_RECIPROCAL if point else MR_OP_FAST_RECIPROCAL
        self.stride = int(stride)
        self.offset = int(stride // 2 if offset is None else offset)
        self.max_iters = int(max_iters)
        ma, mb = _as_map(a), _as_map(b)
        self.B = ma.batch
        self.cap = max(1, seed_count(ma.h, ma.w, self.stride, self.offset))
        dev = a.device
        self.pairs = torch.empty((self.B, self.cap, 2), dtype=torch.int32, device=dev)
        self.n_pairs = torch.empty((self.B,), dtype=torch.int64, device=dev)
        self.active = (torch.empty((self.B, max(1, self.max_iters)), dtype=torch.int32, device=dev)
                       if record_active else None)
        need = self.lib.mr_workspace_bytes(op, ctypes.byref(ma), ctypes.byref(mb), 0, self.stride, self.offset)
        self.ws = None if self.static else _workspace(need, dev)
        self.shape = (tuple(a.shape), tuple(b.shape), a.dtype)

    def __call__(self, a, b):
        if (tuple(a.shape), tuple(b.shape), a.dtype) != self.shape:
            raise ValueError("shapes differ from the ones this FastReciprocal was built for")
        ma, mb = _as_map(a), _as_map(b)
        if self.static:
            rc = self.lib.mr_fast_reciprocal_static(
                ctypes.byref(ma), ctypes.byref(mb), self.stride, self.offset, self.max_iters,
                self.pairs.data_ptr(), self.cap, self.n_pairs.data_ptr(),
                self.active.data_ptr() if self.active is not None else None, _stream(a))
            _check("mr_fast_reciprocal_static", rc)
            return self.pairs, self.n_pairs, self.active
        rc = self.fn(ctypes.byref(ma), ctypes.byref(mb), self.stride, self.offset, self.max_iters,
                     self.pairs.data_ptr(), self.cap, self.n_pairs.data_ptr(),
                     self.active.data_ptr() if self.active is not None else None,
                     self.ws.data_ptr(), self.ws.numel(), _stream(a))
        _check(self.fn.__name__, rc)
        return self.pairs, self.n_pairs, self.active


def fast_reciprocal(a, b, stride: int = 8, offset: Optional[int] = None, max_iters: int = 10):
    """Fast reciprocal matching seeded on a's grid.  Returns (pairs int32 [B, cap, 2],
    n_pairs int64 [B], iter_active int32 [B, max_iters]); pairs ascending in the a-pixel."""
    return FastReciprocal(_batched(a), _batched(b), stride, offset, max_iters)(_batched(a), _batched(b))


class FastReciprocalGraph:
    """Reusable fast reciprocal matching over the edges of a pair graph on one image
    collection (images [n, H, W, d]; edges: host int array [E, 2] of image ids)."""

    def __init__(self, images, edges, stride: int = 8, offset: Optional[int] = None, max_iters: int = 10):
        import numpy as np
        torch = _torch()
        self.lib = load_library()
        self.stride = int(stride)
        self.offset = int(stride // 2 if offset is None else offset)
        self.max_iters = int(max_iters)
        self.edges = np.ascontiguousarray(np.asarray(edges, dtype=np.int32).reshape(-1, 2))
        E = self.edges.shape[0]
        m = _as_map(images)
        self.cap = max(1, seed_count(m.h, m.w, self.stride, self.offset))
        dev = images.device
        self.pairs = torch.empty((E, self.cap, 2), dtype=torch.int32, device=dev)
        self.n_pairs = torch.empty((E,), dtype=torch.int64, device=dev)
        self.active = torch.empty((E, max(1, self.max_iters)), dtype=torch.int32, device=dev)
        need = self.lib.mr_workspace_bytes(MR_OP_FAST_RECIPROCAL_GRAPH, ctypes.byref(m), ctypes.byref(m), E,
                                           self.stride, self.offset)
        if need == 0:
            raise MrError("mr_workspace_bytes", 4)
        self.ws = _workspace(need, dev)
        self.shape = (tuple(images.shape), images.dtype)

    def __call__(self, images):
        if (tuple(images.shape), images.dtype) != self.shape:
            raise ValueError("shapes differ from the ones this FastReciprocalGraph was built for")
        m = _as_map(images)
        rc = self.lib.mr_fast_reciprocal_graph(
            ctypes.byref(m), self.edges.ctypes.data_as(ctypes.c_void_p), self.edges.shape[0], self.stride,
            self.offset, self.max_iters, self.pairs.data_ptr(), self.cap, self.n_pairs.data_ptr(),
            self.active.data_ptr(), self.ws.data_ptr(), self.ws.numel(), _stream(images))
        _check("mr_fast_reciprocal_graph", rc)
        return self.pairs, self.n_pairs, self.active


def fast_reciprocal_graph(images, edges, stride: int = 8, offset: Optional[int] = None, max_iters: int = 10):
    """Fast reciprocal matching on every edge (i, j) of a pair graph over images [n, H, W, d];
    returns (pairs [E, cap, 2], n_pairs [E], iter_active [E, max_iters]) like fast_reciprocal."""
    return FastReciprocalGraph(images, edges, stride, offset, max_iters)(images)


def point_fast_reciprocal(a, b, stride: int = 8, offset: Optional[int] = None, max_iters: int = 10):
    """The fast reciprocal scheme on two pointmaps (nearest points); returns as fast_reciprocal."""
    return FastReciprocal(_batched(a), _batched(b), stride, offset, max_iters,
                          point=True)(_batched(a), _batched(b))


class InfoNCE:
    """Reusable matching-loss forward for fixed shapes (workspace and outputs allocated
    once): terms[b, t] = logsumexp_k(<a_i, b_k> / tau) - <a_i, b_j> / tau for the
    ground-truth pair gt[b, t] = (i, j), and loss[b] = sum_t terms[b, t] (float64)."""

    def __init__(self, a, b, n_gt: int, tau: float = 0.1, backward: bool = False):
        torch = _torch()
        self.lib = load_library()
        self.tau = float(tau)
        self.n_gt = int(n_gt)
        self.backward = bool(backward)
        ma, mb = _as_map(a), _as_map(b)
        self.B = ma.batch
        dev = a.device
        self.terms = torch.empty((self.B, self.n_gt), dtype=torch.float32, device=dev)
        self.loss = torch.empty((self.B,), dtype=torch.float64, device=dev)
        if self.backward:
            self.grad_a = torch.empty(_batched(a).shape, dtype=torch.float32, device=dev)
            self.grad_b = torch.empty(_batched(b).shape, dtype=torch.float32, device=dev)
        op = MR_OP_INFONCE_BACKWARD if self.backward else MR_OP_INFONCE
        need = self.lib.mr_workspace_bytes(op, ctypes.byref(ma), ctypes.byref(mb), self.n_gt, 0, 0)
        if need == 0:
            raise MrError("mr_workspace_bytes", 2)
        self.ws = _workspace(need, dev)
        self.shape = (tuple(_batched(a).shape), tuple(_batched(b).shape), a.dtype)

    def __call__(self, a, b, gt):
        """(terms, loss), plus (grad_a, grad_b) of each pair's loss when built with backward=True."""
        torch = _torch()
        if (tuple(_batched(a).shape), tuple(_batched(b).shape), a.dtype) != self.shape:
            raise ValueError("shapes differ from the ones this InfoNCE was built for")
        gt = gt.to(device=a.device, dtype=torch.int32).reshape(self.B, self.n_gt, 2).contiguous()
        ma, mb = _as_map(a), _as_map(b)
        if self.backward:
            rc = self.lib.mr_infonce_backward(ctypes.byref(ma), ctypes.byref(mb), gt.data_ptr(), self.n_gt,
                                              self.tau, self.terms.data_ptr(), self.loss.data_ptr(),
                                              self.grad_a.data_ptr(), self.grad_b.data_ptr(), self.ws.data_ptr(),
                                              self.ws.numel(), _stream(a))
            _check("mr_infonce_backward", rc)
            return self.terms, self.loss, self.grad_a, self.grad_b
        rc = self.lib.mr_infonce_forward(ctypes.byref(ma), ctypes.byref(mb), gt.data_ptr(), self.n_gt, self.tau,
                                         self.terms.data_ptr(), self.loss.data_ptr(), self.ws.data_ptr(),
                                         self.ws.numel(), _stream(a))
        _check("mr_infonce_forward", rc)
        return self.terms, self.loss


def infonce(a, b, gt, tau: float = 0.1):
    """Matching loss (InfoNCE) of maps a, b over ground-truth pixel pairs gt (int [n_gt, 2] or
    [B, n_gt, 2] of (i in a, j in b)); returns (terms float32 [B, n_gt], loss float64 [B])."""
    B = _batched(a).shape[0]
    n_gt = gt.numel() // (2 * B)
    return InfoNCE(a, b, n_gt, tau)(a, b, gt)


def infonce_backward(a, b, gt, tau: float = 0.1):
    """The matching loss and its gradient (bf16 maps, d <= 32): returns (terms float32
    [B, n_gt], loss float64 [B], grad_a float32 like a, grad_b float32 like b)."""
    B = _batched(a).shape[0]
    n_gt = gt.numel() // (2 * B)
    return InfoNCE(a, b, n_gt, tau, backward=True)(a, b, gt)


def matches(pairs, n_pairs, b: int = 0):
    """The n_pairs[b] valid rows of pairs[b] as a host int64 array [m, 2]."""
    m = int(n_pairs[b].item())
    return pairs[b, :m].cpu().numpy().astype("int64")


# ----------------------------------------------------------------------------- measurement aid

def profile_begin(max_launches: int):
    _check("mr_profile_begin", load_library().mr_profile_begin(max_launches))


def profile_end():
    """Returns (summed similarity-kernel milliseconds, launches timed)."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check("mr_profile_end", load_library().mr_profile_end(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def profile_end_each(cap: int):
    """Returns (summed milliseconds, launches timed, list of each launch's milliseconds
    in launch order, at most cap of them)."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    each = (ctypes.c_float * max(1, cap))()
    _check("mr_profile_end_each", load_library().mr_profile_end_each(ctypes.byref(ms), ctypes.byref(n), each, cap))
    return ms.value, n.value, [float(x) for x in each[:min(cap, n.value)]]


def profile_end_queries(cap: int):
    """Returns (summed milliseconds, launches timed, each launch's milliseconds, each
    launch's query count summed over the batch (-1: not counted)), at most cap of each."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    each = (ctypes.c_float * max(1, cap))()
    qs = (ctypes.c_int64 * max(1, cap))()
    _check("mr_profile_end_queries",
           load_library().mr_profile_end_queries(ctypes.byref(ms), ctypes.byref(n), each, qs, cap))
    k = min(cap, n.value)
    return ms.value, n.value, [float(x) for x in each[:k]], [int(x) for x in qs[:k]]
