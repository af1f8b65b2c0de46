#!/usr/bin/env python3
"""Benchmark: fast reciprocal matching of one 512x384 d=24 fp32 descriptor-map pair.

One step = one mr_fast_reciprocal call on inputs already resident in HBM:
seed grid (stride 8, 3072 seeds), up to 10 forward/backward NN iterations with
cycle check and frontier compaction, and the ordered match list.  The JSON line
reports image pairs/s, NN queries/s, the similarity kernel's fraction of the
ceiling of fp32-accurate products on the matrix cores (timed live with HIP events
around each launch), and the CPU oracle timed on the host for the same pair.
Other workloads (brute-force bf16 mutual NN, the 64-pair batch, the 1024x768 bf16
pair, pointmaps, the pair graph, the matching loss) are reported under "other"
unless --main-only.
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "image pairs/sec fast reciprocal NN @512×384 d=24; NN-queries/sec; %MFMA peak"
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}   # MI355X dense matrix-core peaks
# fp32 maps never use the fp32 matrix instruction: each fp32 product is formed as six
# exact bf16 products (an exact three-way split of both operands) on the bf16 matrix
# cores, so the ceiling of fp32-accurate products is the bf16 peak over six.
SPLIT_PRODUCTS = 6
PEAK_SPLIT_TFLOPS = PEAK_TFLOPS["bf16"] / SPLIT_PRODUCTS
PEAK_HBM_GBPS = 8000.0
# fp32 VALU lane-operations per second: the published fp32 vector peak, 157.3 TFLOP/s,
# is 78.6 T fused multiply-adds per second (32 fp32 lanes per SIMD per clock, 256 CUs x
# 4 SIMDs x 2.4 GHz); a plain fp32 VALU operation (subtract, multiply, minimum) counts as
# one lane-operation like an FMA.  Measured without packed instructions: one instruction
# type issues at 16 lanes per clock, the point kernel's mix at up to 23 (56 T/s), so the
# published figure is an upper bound.
PEAK_VALU_TOPS = 157.3 / 2
# Algorithmic VALU work of one (query, point) pair of 3D pointmaps: 3 subtractions, a
# multiply and 2 fused multiply-adds for the squared distance, and half of a 3-input
# minimum for the selection.
POINT_OPS_PER_PAIR = 6.5
# Transcendental (v_exp_f32) lane-operations per second: 8 lanes per SIMD per clock, a
# quarter of the published rate (measured: 19.3 T/s at 2.39 GHz).
PEAK_EXP_TOPS = PEAK_VALU_TOPS / 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # defaults: about 27 ms of timed calls after 20 warm-up calls (about 11 ms), which
    # leave the first calls' lower clock out of the mean
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--main-only", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", choices=OTHER, default=None,
                    help="run just this one of the other workloads and print its record (for profiling)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB (calibrates HBM byte counters)")
    return ap.parse_args()


def copy_calibration(mib, torch):
    """A plain device-to-device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 3}), flush=True)


def dev_maps(p, torch, dev):
    import numpy as np
    if p.dtype == "bf16":
        A = torch.from_numpy(np.ascontiguousarray(p.D1_bits).reshape(p.H, p.W, p.d)).view(torch.bfloat16)
        B = torch.from_numpy(np.ascontiguousarray(p.D2_bits).reshape(p.H, p.W, p.d)).view(torch.bfloat16)
    else:
        A = torch.from_numpy(p.D1.reshape(p.H, p.W, p.d))
        B = torch.from_numpy(p.D2.reshape(p.H, p.W, p.d))
    return A.to(dev).unsqueeze(0), B.to(dev).unsqueeze(0)


def time_steps(fn, steps, warmup, torch, prof_launches=0, each=None, queries=None):
    """Warm up, then time exactly `steps` calls between two synchronisations with nothing
    else on the stream.  With prof_launches, the same steps run once more with the
    library's per-launch hipEvents on (they cost a few microseconds per launch, so they
    stay out of the pass that gives the step time) for the similarity kernel's average
    launch duration; `each` receives every launch's milliseconds and `queries` every
    search launch's query count (summed over the batch).  Returns (ms per step, summed
    similarity-kernel ms, launches timed)."""
    import dense_grounded_image_amd as mr
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        fn()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    kms, kn = 0.0, 0
    if prof_launches:
        mr.profile_begin(prof_launches)
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        if queries is not None:
            kms, kn, per, qs = mr.profile_end_queries(prof_launches)
            queries.extend(qs)
            if each is not None:
                each.extend(per)
        elif each is None:
            kms, kn = mr.profile_end()
        else:
            kms, kn, per = mr.profile_end_each(prof_launches)
            each.extend(per)
    return ms, kms, kn


def step_percentiles(fn, steps, torch):
    """Per-step times (one hipEvent pair around each call, nothing else on the stream):
    p10, median and p90 in ms over `steps` calls."""
    import numpy as np
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return [round(float(x), 4) for x in np.percentile(t, [10, 50, 90])]


def oracle_host():
    """CPU model string and the core count the host shows."""
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cpu, os.cpu_count() or 0


def fast_work(searched, N, d):
    """Algorithmic work of one fast-scheme call: every NN query the call searched costs
    2*N*d flops against the other map.  A call searches the forward NN of each live
    pixel and the backward NN of each pixel of image 2 it lands on, once per call (an
    answer already found is reused), so `searched` comes from the library's per-launch
    query counts, not from the live counts."""
    return searched, 2.0 * N * d * searched


def searched_per_step(queries, steps):
    """NN queries the search launches ran per call (uncounted launches excluded)."""
    return sum(q for q in queries if q >= 0) / steps


def run_fast(p, batch_pairs, args, torch, dev, prof=True, point=False):
    import dense_grounded_image_amd as mr
    if batch_pairs is None:
        A, B = dev_maps(p, torch, dev)
    else:
        A, B = batch_pairs
    f = mr.FastReciprocal(A, B, p.stride, p.offset, p.max_iters, point=point)
    launches = 2 * p.max_iters * args.steps
    each, queries = [], []
    ms, kms, kn = time_steps(lambda: f(A, B), args.steps, args.warmup, torch, launches if prof else 0, each,
                             queries)
    pairs, n_pairs, active = f(A, B)
    torch.cuda.synchronize()
    act = active.cpu().numpy()
    q, flops = fast_work(searched_per_step(queries, args.steps), p.N, p.d)
    return dict(ms=ms, kernel_ms=kms, launches=kn, nn_queries=q, flops=flops, each=each, queries=queries,
                nn_answers=2 * int(act.sum()),
                active=act[0].tolist(), matches=[int(x) for x in n_pairs.cpu()], batch=A.shape[0],
                pairs0=pairs[0, :int(n_pairs[0])].cpu().numpy())


def rounds_roofline(r, N, d, elem_bytes, peak_tflops):
    """Per round of the fast scheme: its two similarity launches' measured time (averaged
    over the timed calls) against the round's lower bound max(flops / matrix peak,
    bytes / HBM), flops 2*N*d per query the two launches searched (the forward NN of the
    |U_t| live pixels, the backward NN of the landing pixels not searched before) and
    bytes two map reads of N*d elements; overall, the summed bounds over the summed
    kernel time.  peak_tflops is the ceiling of the arithmetic the kernel executes (for
    fp32 maps the split ceiling, bf16 peak / 6)."""
    each, act, qs = r["each"], r["active"], r["queries"]
    per_call = 2 * len(act)
    if not each or len(each) % per_call or len(qs) != len(each):
        return None
    calls = len(each) // per_call
    out, lb_sum, t_sum = [], 0.0, 0.0
    for t, u in enumerate(act):
        ms = sum(each[c * per_call + 2 * t] + each[c * per_call + 2 * t + 1] for c in range(calls)) / calls
        qf = sum(qs[c * per_call + 2 * t] for c in range(calls)) / calls
        qb = sum(qs[c * per_call + 2 * t + 1] for c in range(calls)) / calls
        fl = 2.0 * (qf + qb) * N * d
        by = 2.0 * N * d * elem_bytes if u else 0.0
        lb = max(fl / (peak_tflops * 1e12), by / (PEAK_HBM_GBPS * 1e9)) * 1e3
        lb_sum += lb
        t_sum += ms
        out.append({"t": t, "active": int(u), "backward_searched": int(round(qb)), "ms": round(ms, 4),
                    "lb_ms": round(lb, 4), "frac": round(lb / ms, 4) if ms > 0 else None})
    return {"rounds": out, "lb_ms": round(lb_sum, 4), "kernel_ms": round(t_sum, 4),
            "frac": round(lb_sum / t_sum, 4) if t_sum else None}


def measured_traffic(name):
    """HBM bytes per launch of the similarity kernel from a committed counter summary, or
    None when the kernel source has changed since the counters were taken."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            rec = json.load(f)
        with open(os.path.join(ROOT, "dense_grounded_image_amd", "csrc", "mr.hip"), "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    return rec["hbm_bytes_per_launch"] if rec.get("source_sha256") == sha else None


def roofline(flops_per_step, steps, kernel_ms, launches, dtype, traffic=None, kernel="nn_argmax_kernel"):
    """Algorithmic flops (2*N*d per NN query; a brute-force call counts the similarity
    matrix once) per launch of the similarity kernel over its average launch time,
    against the ceiling of the arithmetic the kernel executes.  bf16 maps: the bf16
    matrix-core peak.  fp32 maps: every fp32 product is six exact bf16 products on the
    bf16 matrix cores (the fp32 matrix instruction is never issued), so the ceiling is
    the bf16 peak / 6; the fraction of the fp32 matrix peak is kept as a secondary
    field.  traffic: measured HBM bytes per launch, or None."""
    if not launches:
        return None
    per_launch = flops_per_step * steps / launches
    avg_ms = kernel_ms / launches
    achieved = per_launch / (avg_ms * 1e-3) / 1e12
    peak = PEAK_SPLIT_TFLOPS if dtype == "f32" else PEAK_TFLOPS[dtype]
    out = {"bound": "mfma", "achieved": round(achieved, 3), "peak": round(peak, 2), "unit": "TFLOP/s",
           "frac": round(achieved / peak, 4), "traffic": traffic,
           "kernel": kernel, "avg_launch_us": round(avg_ms * 1e3, 2),
           "flops_per_launch": per_launch}
    if traffic is not None:
        out["hbm_GBps"] = round(traffic / (avg_ms * 1e-3) / 1e9, 1)
        out["hbm_frac"] = round(traffic / (avg_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)
    if dtype == "f32":
        out["peak_note"] = "fp32-accurate products: bf16 peak 2500 TFLOP/s / 6 bf16 products each"
        out["fp32_mfma"] = {"peak": PEAK_TFLOPS["f32"], "frac": round(achieved / PEAK_TFLOPS["f32"], 4),
                            "note": "secondary: the fp32 matrix instruction is not issued"}
        out["executed"] = {"arith": "bf16 x3 split, 6 bf16 products per fp32 product",
                           "achieved_bf16_TFLOPs": round(6 * achieved, 2), "peak": PEAK_TFLOPS["bf16"],
                           "frac": round(6 * achieved / PEAK_TFLOPS["bf16"], 4)}
    elif dtype == "bf16":
        pad = 32.0 / 24.0   # d = 24 runs as K = 32 on the 32x32x16 bf16 instruction
        out["executed"] = {"arith": "d = 24 padded to K = 32 on the bf16 matrix cores",
                           "achieved_bf16_TFLOPs": round(pad * achieved, 2), "peak": PEAK_TFLOPS["bf16"],
                           "frac": round(pad * achieved / PEAK_TFLOPS["bf16"], 4)}
    return out


def roofline_alu(pairs_per_step, steps, kernel_ms, launches):
    """VALU-bound kernels (pointmaps): algorithmic lane-operations per launch over its
    average launch time, against the chip's VALU lane-operation rate."""
    if not launches:
        return None
    per_launch = pairs_per_step * POINT_OPS_PER_PAIR * steps / launches
    avg_ms = kernel_ms / launches
    achieved = per_launch / (avg_ms * 1e-3) / 1e12
    return {"bound": "alu", "achieved": round(achieved, 3), "peak": round(PEAK_VALU_TOPS, 2),
            "unit": "T VALU lane-ops/s", "frac": round(achieved / PEAK_VALU_TOPS, 4), "traffic": None,
            "kernel": "point_nn_kernel", "avg_launch_us": round(avg_ms * 1e3, 2),
            "ops_per_launch": per_launch, "ops_per_pair": POINT_OPS_PER_PAIR}


def roofline_lse(scores_per_step, d, steps, kernel_ms, launches):
    """The matching loss's log-sum-exp kernel: one exponential per score on the VALU's
    transcendental unit, next to 2*d flops per score on the bf16 matrix cores."""
    if not launches:
        return None
    per_launch = scores_per_step * steps / launches
    avg_ms = kernel_ms / launches
    exps = per_launch / (avg_ms * 1e-3) / 1e12
    flops = 2.0 * d * exps
    return {"bound": "alu", "achieved": round(exps, 3), "peak": round(PEAK_EXP_TOPS, 2),
            "unit": "T exp/s", "frac": round(exps / PEAK_EXP_TOPS, 4), "traffic": None,
            "kernel": "lse_partial_kernel", "avg_launch_us": round(avg_ms * 1e3, 2),
            "scores_per_launch": per_launch,
            "mfma": {"achieved_TFLOPs": round(flops, 2), "peak": PEAK_TFLOPS["bf16"],
                     "frac": round(flops / PEAK_TFLOPS["bf16"], 4)}}


def cpu_baseline(p, gpu=None):
    """The oracle timed on the host on this pair (and per core on it and the 64x48 pair);
    with `gpu` (the library's result on the same pair), also the pass/fail count of each
    parity rule of the fast scheme between the two."""
    import oracle
    import workloads
    threads = oracle.default_threads()
    t = time.perf_counter()
    r = oracle.fast(p.D1, p.H, p.W, p.D2, p.stride, p.offset, p.max_iters, nthreads=threads)
    dt = time.perf_counter() - t
    cpu, ncpu = oracle_host()
    out = {"value": round(1.0 / dt, 4), "unit": "pairs/s", "cores": threads, "kind": "oracle",
           "sample": "the whole 512x384 pair (3072 seeds, 10 iterations), binary64 C oracle, %d threads, "
                     "%.2f s, %d NN queries, CPU %s, nproc %d" % (threads, dt, r["nn_queries"], cpu, ncpu),
           "nn_queries_per_s": round(r["nn_queries"] / dt, 1), "matches": int(len(r["pairs"]))}
    # one core: the fast scheme on the 64x48 pair and on this 512x384 pair
    per_core = {}
    for name, q in (("pair-64x48-f32", workloads.config_pair(0)), ("pair-512x384-f32", p)):
        t = time.perf_counter()
        r1 = oracle.fast(q.D1, q.H, q.W, q.D2, q.stride, q.offset, q.max_iters, nthreads=1)
        dt1 = time.perf_counter() - t
        per_core[name] = {"pairs_per_s": round(1.0 / dt1, 4), "seconds": round(dt1, 3), "threads": 1,
                          "nn_queries_per_s": round(r1["nn_queries"] / dt1, 1)}
    out["per_core"] = per_core
    if gpu is not None:
        from tests.checks import fast_rule_counts
        t = time.perf_counter()
        rules, summary = fast_rule_counts(gpu["pairs0"], r, p.D1, p.D2, "f32", nthreads=threads,
                                          gpu_active=gpu["active"])
        for v in rules.values():
            if not v["failed"]:
                del v["examples"]
        out["parity_vs_gpu"] = {"workload": "pair-512x384-f32", "rules": rules, "summary": summary,
                                "all_passed": all(v["failed"] == 0 for v in rules.values()),
                                "seconds": round(time.perf_counter() - t, 2)}
    return out


def cpu_samples():
    """The oracle on bounded samples of two of the other workloads (brute-force bf16
    mutual NN, the matching loss), with the full-size time extrapolated from them."""
    import numpy as np
    import oracle
    import workloads
    threads = oracle.default_threads()
    out = {}
    p2 = workloads.config_pair(2)
    rows = np.sort(np.random.default_rng(2).choice(p2.N, 4096, replace=False)).astype(np.int32)
    t = time.perf_counter()
    oracle.nn_rows(p2.D1, rows, p2.D2, nthreads=threads)
    oracle.nn_rows(p2.D2, rows, p2.D1, nthreads=threads)
    dt = time.perf_counter() - t
    out["pair-512x384-bf16-bruteforce"] = {
        "sample": "4096 + 4096 query rows (both directions)", "seconds": round(dt, 3), "threads": threads,
        "nn_queries_per_s": round(8192 / dt, 1),
        "full_call_seconds_extrapolated": round(dt * p2.N / 4096, 1)}
    g = workloads.gt_pairs(p2)
    pick = np.sort(np.random.default_rng(3).choice(len(g), 1024, replace=False))
    t = time.perf_counter()
    oracle.infonce(p2.D1, p2.D2, g[pick], float(np.float32(0.1)), nthreads=threads)
    dt = time.perf_counter() - t
    out["infonce-512x384-bf16"] = {
        "sample": "1024 of the 137626 ground-truth terms", "seconds": round(dt, 3), "threads": threads,
        "terms_per_s": round(1024 / dt, 1), "full_loss_seconds_extrapolated": round(dt * len(g) / 1024, 1)}
    return out


def other_batch64(args, torch, dev):
    """64 independent 512x384 fp32 pairs in one call."""
    import workloads
    ps = [workloads.config_pair(3, b) for b in range(64)]
    A = torch.stack([dev_maps(q, torch, dev)[0][0] for q in ps])
    B = torch.stack([dev_maps(q, torch, dev)[1][0] for q in ps])
    del ps
    print("bench: batch data ready", file=sys.stderr, flush=True)
    rb = run_fast(workloads.config_pair(3, 0), (A, B), args, torch, dev)
    return {"pairs_per_s": round(64000.0 / rb["ms"], 2), "ms_per_call": round(rb["ms"], 3),
            "nn_queries_per_s": round(rb["nn_queries"] * 1000.0 / rb["ms"], 1),
            "roofline": roofline(rb["flops"], args.steps, rb["kernel_ms"], rb["launches"], "f32")}


def other_bf16_1024(args, torch, dev):
    """One 1024x768 bf16 pair, fast scheme, 15 iterations."""
    import workloads
    p4 = workloads.config_pair(4)
    r4 = run_fast(p4, None, args, torch, dev)
    return {"pairs_per_s": round(1000.0 / r4["ms"], 2), "ms_per_call": round(r4["ms"], 3),
            "nn_queries_per_s": round(r4["nn_queries"] * 1000.0 / r4["ms"], 1),
            "iter_active": r4["active"], "matches": r4["matches"][0],
            "roofline": roofline(r4["flops"], args.steps, r4["kernel_ms"], r4["launches"], "bf16")}


def other_bruteforce(args, torch, dev):
    """Brute-force mutual NN of the 512x384 pair in bf16 (both directions)."""
    import dense_grounded_image_amd as mr
    import workloads
    p2 = workloads.config_pair(2)
    A2, B2 = dev_maps(p2, torch, dev)
    ws = torch.empty(mr.workspace_bytes(mr.MR_OP_MUTUAL_NN, A2, B2), dtype=torch.uint8, device=dev)
    # about 2.5 ms per call: 10 warm-up calls (the first calls run at a lower clock),
    # then at least 10 timed calls
    steps = max(10, args.steps // 4)
    ms, kms, kn = time_steps(lambda: mr.mutual_nn(A2, B2, ws=ws), steps, 10, torch, 2 * steps)
    fl = 2.0 * p2.N * p2.N * p2.d   # the method's work: the similarity matrix once
    # the two-pass alternative: a row search in each direction (the maps' roles swapped),
    # i.e. the matrix computed twice; the mutual call above computes it once
    wn = torch.empty(mr.workspace_bytes(mr.MR_OP_NN_ARGMAX, A2, B2, p2.N), dtype=torch.uint8, device=dev)
    ms2, _, _ = time_steps(lambda: (mr.nn_argmax(A2, B2, ws=wn), mr.nn_argmax(B2, A2, ws=wn)), steps, 10, torch)
    out = {"pairs_per_s": round(1000.0 / ms, 2), "ms_per_call": round(ms, 3),
           "variant": "fused row + column pass (rowcol_argmax_kernel), then both recoveries",
           "two_pass_ms": round(ms2, 3),
           "two_pass_variant": "two row searches (nn_argmax_kernel, maps swapped), without the pair compaction",
           "nn_queries_per_s": round(2 * p2.N * 1000.0 / ms, 1),
           "mfma_frac_algorithmic": round(fl / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], 4),
           "similarity_launches_per_call": kn / steps if steps else None,
           "roofline": roofline(fl, steps, kms, kn, "bf16", kernel="rowcol_argmax_kernel")}
    return out


def point_maps(p, torch, dev):
    A = torch.from_numpy(p.D1.reshape(p.H, p.W, 3)).to(dev).unsqueeze(0)
    B = torch.from_numpy(p.D2.reshape(p.H, p.W, 3)).to(dev).unsqueeze(0)
    return A, B


def other_points_fast(args, torch, dev):
    """Fast reciprocal matching of one 512x384 pointmap pair (nearest 3D points)."""
    import workloads
    p = workloads.make_pointmaps(512, 384, seed=11)
    r = run_fast(p, point_maps(p, torch, dev), args, torch, dev, point=True)
    pairs_per_step = r["nn_queries"] * p.N            # each query against every point
    return {"pairs_per_s": round(1000.0 / r["ms"], 2), "ms_per_call": round(r["ms"], 3),
            "nn_queries_per_s": round(r["nn_queries"] * 1000.0 / r["ms"], 1),
            "iter_active": r["active"], "matches": r["matches"][0],
            "roofline": roofline_alu(pairs_per_step, args.steps, r["kernel_ms"], r["launches"])}


def other_points_bruteforce(args, torch, dev):
    """Brute-force reciprocal nearest points of one 512x384 pointmap pair."""
    import dense_grounded_image_amd as mr
    import workloads
    p = workloads.make_pointmaps(512, 384, seed=11)
    A, B = point_maps(p, torch, dev)
    ws = torch.empty(mr.workspace_bytes(mr.MR_OP_POINT_MUTUAL_NN, A, B), dtype=torch.uint8, device=dev)
    steps = max(3, args.steps // 4)
    ms, kms, kn = time_steps(lambda: mr.point_mutual_nn(A, B, ws=ws), steps, 2, torch, 2 * steps)
    return {"pairs_per_s": round(1000.0 / ms, 2), "ms_per_call": round(ms, 3),
            "nn_queries_per_s": round(2 * p.N * 1000.0 / ms, 1),
            "roofline": roofline_alu(2.0 * p.N * p.N, steps, kms, kn)}


def other_graph(args, torch, dev):
    """The complete pair graph of 50 images of 512x384 fp32 (1225 edges) in one call."""
    import dense_grounded_image_amd as mr
    import workloads
    n = 50
    maps, _, _ = workloads.make_collection(n, 512, 384, 24, seed=2000)
    imgs = torch.from_numpy(maps.reshape(n, 512, 384, 24)).to(dev)
    del maps
    edges = workloads.all_edges(n)
    print("bench: collection ready", file=sys.stderr, flush=True)
    g = mr.FastReciprocalGraph(imgs, edges, 8, 4, 10)
    steps, warm = max(2, args.steps // 10), 1
    queries = []
    ms, kms, kn = time_steps(lambda: g(imgs), steps, warm, torch, 20 * steps, queries=queries)
    _, npairs, active = g(imgs)
    torch.cuda.synchronize()
    q, flops = fast_work(searched_per_step(queries, steps), 512 * 384, 24)
    return {"pairs_per_s": round(len(edges) * 1000.0 / ms, 2), "ms_per_call": round(ms, 3),
            "edges": int(len(edges)), "images": n, "images_bytes": int(imgs.numel() * 4),
            "nn_queries_per_s": round(q * 1000.0 / ms, 1), "matches_total": int(npairs.sum()),
            "roofline": roofline(flops, steps, kms, kn, "f32")}


def other_infonce(args, torch, dev):
    """Matching loss (InfoNCE forward, tau = 0.1) of the 512x384 bf16 planted pair over its
    ground-truth correspondences (every non-occluded pixel of image 2: 137626 terms, each a
    log-sum-exp over all 196608 pixels of image 2)."""
    import dense_grounded_image_amd as mr
    import workloads
    p = workloads.config_pair(2)
    A, B = dev_maps(p, torch, dev)
    gt = torch.from_numpy(workloads.gt_pairs(p)).to(dev).unsqueeze(0)
    n_gt = int(gt.shape[1])
    f = mr.InfoNCE(A, B, n_gt, 0.1)
    steps = max(3, args.steps // 4)
    ms, kms, kn = time_steps(lambda: f(A, B, gt), steps, 2, torch, steps)
    scores = n_gt * p.N
    out = {"loss_evals_per_s": round(1000.0 / ms, 2), "ms_per_call": round(ms, 3), "n_gt": n_gt,
           "scores_per_s": round(scores * 1000.0 / ms, 1), "loss": float(f.loss[0].cpu()),
           "roofline": roofline_lse(scores, p.d, steps, kms, kn)}
    return out


def other_infonce_backward(args, torch, dev):
    """The matching loss and its gradient with respect to both maps, same pair and ground
    truth as infonce-512x384-bf16: the forward stage, then a row pass (softmax-weighted
    rows of image 2 per term) and a column pass (softmax-weighted ground-truth rows of
    image 1 per pixel of image 2), each recomputing every score."""
    import dense_grounded_image_amd as mr
    import workloads
    p = workloads.config_pair(2)
    A, B = dev_maps(p, torch, dev)
    gt = torch.from_numpy(workloads.gt_pairs(p)).to(dev).unsqueeze(0)
    n_gt = int(gt.shape[1])
    f = mr.InfoNCE(A, B, n_gt, 0.1, backward=True)
    steps = max(3, args.steps // 4)
    ms, kms, kn = time_steps(lambda: f(A, B, gt), steps, 2, torch, 2 * steps)
    scores = n_gt * p.N
    rl = roofline_lse(2 * scores, p.d, steps, kms, kn)
    if rl:
        rl["kernel"] = "nce_grad_kernel (row and column passes)"
        rl["mfma"]["note"] = "2*d flops per score for the scores; the p*X products add 4*32 executed flops per score"
    return {"loss_and_grad_per_s": round(1000.0 / ms, 2), "ms_per_call": round(ms, 3), "n_gt": n_gt,
            "scores_per_s": round(3 * scores * 1000.0 / ms, 1), "roofline": rl}


OTHER = {"batch64-512x384-f32": other_batch64, "pair-1024x768-bf16": other_bf16_1024,
         "graph-50x512x384-f32": other_graph,
         "pointmaps-512x384-f32": other_points_fast, "pointmaps-512x384-f32-bruteforce": other_points_bruteforce,
         "pair-512x384-bf16-bruteforce": other_bruteforce, "infonce-512x384-bf16": other_infonce,
         "infonce-backward-512x384-bf16": other_infonce_backward}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this matcher has no multi-GPU path "
              "(the 64-pair batch would shard by pairs; see the design notes).", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_mb:
        copy_calibration(args.copy_mb, torch)
        return
    import dense_grounded_image_amd as mr
    import workloads
    mr.load_library()
    dev = torch.device("cuda:0")
    if args.only:
        print(json.dumps({args.only: OTHER[args.only](args, torch, dev)}), flush=True)
        release_device(torch)
        return

    p = workloads.config_pair(1)
    print("bench: workload pair-512x384-f32 ready", file=sys.stderr, flush=True)
    r = run_fast(p, None, args, torch, dev)
    value = 1000.0 / r["ms"]
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "pairs/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "pair-512x384-f32: fast reciprocal matching, one 512x384 pair, d=24 fp32, "
                               "seed stride 8 offset 4 (3072 seeds), 10 iterations",
                   "H": 512, "W": 384, "d": 24, "batch": 1, "stride": 8, "offset": 4, "max_iters": 10},
        "nn_queries_per_s": round(r["nn_queries"] * 1000.0 / r["ms"], 1),
        "nn_queries_per_step": r["nn_queries"],
        "nn_answers_per_step": r["nn_answers"],
        "nn_queries_note": "queries searched per call: the forward NN of every live pixel and the backward "
                           "NN of each landing pixel once per call; nn_answers counts both NN of every live "
                           "pixel, backward ones found earlier in the call reused",
        "iter_active": r["active"], "matches": r["matches"][0],
        "roofline": roofline(r["flops"], args.steps, r["kernel_ms"], r["launches"], "f32",
                             measured_traffic("nn_argmax_pair512x384_f32_traffic.json")),
        "step_mfma_frac": round(r["flops"] / (r["ms"] * 1e-3) / 1e12 / PEAK_SPLIT_TFLOPS, 4),
        "binding_roof_by_round": rounds_roofline(r, p.N, p.d, 4, PEAK_SPLIT_TFLOPS),
    }
    f1 = mr.FastReciprocal(*dev_maps(p, torch, dev), p.stride, p.offset, p.max_iters)
    A1, B1 = dev_maps(p, torch, dev)
    out["step_ms_p10_p50_p90"] = step_percentiles(lambda: f1(A1, B1), max(args.steps, 20), torch)
    print("bench: fast pair %.4f ms/step" % r["ms"], file=sys.stderr, flush=True)

    if not args.main_only:
        out["other"] = {name: OTHER[name](args, torch, dev) for name in OTHER}

    if not args.no_cpu:
        print("bench: CPU oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(p, gpu=r)
        if not args.main_only:
            out["cpu_baseline"]["other_samples"] = cpu_samples()
    print(json.dumps(out), flush=True)
    # release the device objects while the runtime is fully up, so that nothing of this
    # process touches the GPU during interpreter teardown
    del f1, A1, B1
    release_device(torch)


def release_device(torch):
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
