"""The workspace-free fast scheme (mr_fast_reciprocal_static, a static per-GPU scratch
array) against the workspace call (mr_fast_reciprocal), through the C ABI: element by
element equal pairs, counts and live counts on three calls in a row -- a 1024x768 bf16
pair (T = 15), then a smaller 512x384 fp32 pair, then the 64x48 fp32 pair -- so that a
call reusing the static buffer after a larger one is covered, and a rejected oversize
call in between changes nothing."""
import ctypes

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import dense_grounded_image_amd as mr  # noqa: E402

DEV = torch.device("cuda:0")
SCRATCH = 8


def log(*a):
    print(*a, flush=True)


def dev_maps(p):
    if p.dtype == "bf16":
        A = torch.from_numpy(np.ascontiguousarray(p.D1_bits).reshape(1, p.H, p.W, p.d)).view(torch.bfloat16)
        B = torch.from_numpy(np.ascontiguousarray(p.D2_bits).reshape(1, p.H, p.W, p.d)).view(torch.bfloat16)
    else:
        A = torch.from_numpy(p.D1.reshape(1, p.H, p.W, p.d))
        B = torch.from_numpy(p.D2.reshape(1, p.H, p.W, p.d))
    return A.to(DEV), B.to(DEV)


def run_both(lib, p):
    A, B = dev_maps(p)
    ma, mb = mr._as_map(A), mr._as_map(B)
    cap = lib.mr_seed_count(p.H, p.W, p.stride, p.offset)
    st = torch.cuda.current_stream(DEV).cuda_stream
    out = []
    for static in (False, True):
        pairs = torch.full((1, cap, 2), -7, dtype=torch.int32, device=DEV)
        n = torch.full((1,), -7, dtype=torch.int64, device=DEV)
        act = torch.full((1, p.max_iters), -7, dtype=torch.int32, device=DEV)
        if static:
            rc = lib.mr_fast_reciprocal_static(ctypes.byref(ma), ctypes.byref(mb), p.stride, p.offset, p.max_iters,
                                               pairs.data_ptr(), cap, n.data_ptr(), act.data_ptr(), st)
        else:
            need = lib.mr_workspace_bytes(2, ctypes.byref(ma), ctypes.byref(mb), 0, p.stride, p.offset)
            ws = torch.empty(need, dtype=torch.uint8, device=DEV)
            rc = lib.mr_fast_reciprocal(ctypes.byref(ma), ctypes.byref(mb), p.stride, p.offset, p.max_iters,
                                        pairs.data_ptr(), cap, n.data_ptr(), act.data_ptr(), ws.data_ptr(), need, st)
        assert rc == 0, (static, rc)
        torch.cuda.synchronize()
        m = int(n[0])
        out.append((m, pairs[0, :m].cpu().numpy(), act[0].cpu().numpy()))
    return out


def test_static_scratch_equals_workspace_call():
    lib = mr.load_library()
    for cfg in (4, 1, 0):
        p = workloads.config_pair(cfg)
        log("static scratch: workload", cfg, p.H, p.W, p.dtype, "T", p.max_iters)
        (n0, p0, a0), (n1, p1, a1) = run_both(lib, p)
        assert n0 == n1 and n0 > 0, (cfg, n0, n1)
        assert (p0 == p1).all(), cfg
        assert (a0 == a1).all(), (cfg, a0, a1)
        log("  equal:", n0, "pairs, live", a0.tolist())
        if cfg == 4:
            # an oversize problem is refused before anything is launched
            big = torch.empty((10, 512, 384, 8), dtype=torch.float32, device=DEV)
            mb = mr._as_map(big)
            cap = 3072
            pairs = torch.empty((10, cap, 2), dtype=torch.int32, device=DEV)
            n = torch.empty((10,), dtype=torch.int64, device=DEV)
            rc = lib.mr_fast_reciprocal_static(ctypes.byref(mb), ctypes.byref(mb), 8, 4, 10, pairs.data_ptr(), cap,
                                               n.data_ptr(), None, torch.cuda.current_stream(DEV).cuda_stream)
            assert rc == SCRATCH, rc
