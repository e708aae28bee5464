#!/usr/bin/env python3
"""Benchmark of the MoE routing hot path on one MI355X.

One step = one pass of the whole routing path over one batch of synthetic
router logits: softmax, top-k, expert histogram, f/P, aux loss, expert
offsets, stable capacity-limited dispatch permutation and the imbalance
statistics (plus the gate GEMM and/or the aux-loss backward for workloads
that include them).  Inputs are resident in HBM before timing starts and are
rotated over several copies (> 512 MB in total) so that the 256 MB Infinity
Cache cannot serve them.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload v3_shape]

Workloads: switch_top1, zipf_top2, gate_top2, v3_shape (default), v4_shape,
v3_select_bias; and the two planners, eplb_v4 and sinkhorn_r64, which print
their per-call latency instead.
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed tokens/sec at 1 GPU + achieved HBM GB/s vs peak (E=256 top-8, T=131072)"
HBM_PEAK_GBPS = 8000.0
ROTATE_BYTES = 600 * 1024 * 1024


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="v3_shape")
    ap.add_argument("--two-stream", action="store_true",
                    help="also time two streams taking alternate batches (forward-only workloads; "
                         "reported as detail.two_stream_ms_per_batch, never as value)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU work budget of the oracle baseline (0 disables it)")
    return ap.parse_args()


class HipEvents:
    """hipEvent_t handles from the HIP runtime PyTorch loaded (plumbing)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        h = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(h)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return h.value

    def record(self, ev, stream):
        if self.lib.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev):
        self.lib.hipEventDestroy(ctypes.c_void_p(ev))


def alg_bytes(w, T):
    """Algorithmic bytes of one step: only what the method must move (no
    workspace partials, no re-reads).  Per logit 4 B read; per assignment 8 B
    (index + weight) from the row pass and 5 B (perm + drop flag) from the
    scatter; per token 8 B of softmax statistics when the backward follows;
    gate path: X and Wg read, fp32 logits written; backward: logits and
    statistics read, gradient written."""
    k, E, d = w.k, w.E, w.d
    stats = 8 * T if w.backward else 0
    rows = 4 * T * E + 8 * T * k + stats
    gate = (2 * T * d + 2 * d * E + 4 * T * E) if d > 0 else 0
    scatter = 5 * T * k
    bwd = (8 * T * E + 8 * T) if w.backward else 0
    # gate backward: X read, dX (bf16) written, dlogits and Wg read, dWg written
    gate_bwd = (4 * T * d + 4 * T * E + 2 * d * E + 4 * d * E) if (d > 0 and w.backward) else 0
    forward = (gate + 8 * T * k + stats + scatter) if d > 0 else (rows + scatter)
    if w.select_bias_scale > 0:
        # selection bias read by the row pass; the update reads the counts
        # and reads and writes the bias
        forward += 4 * E + (4 * w.n_micro * E + 8 * E if w.bias_gamma > 0 else 0)
    return {"rows": rows, "gate": gate, "scatter": scatter, "backward": bwd + gate_bwd,
            "route_backward": bwd, "gate_backward": gate_bwd, "forward": forward}


def one_launch_path(w):
    """Whether moe_route routes this workload in one launch: E of 1, 2, 4 or
    8, k*E at most 16 and microbatches of at most 32768 logits, as the
    library decides in moe_route."""
    Tm = w.T // w.n_micro
    return (w.E in (1, 2, 4, 8) and w.k * w.E <= 16 and Tm * w.E <= 32768
            and w.n_micro <= 65535)


def kernel_source_hash():
    """Hash of the HIP sources, to tell whether stored counters still apply."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "load_balancing_statistics_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel_prefix):
    """HBM bytes per launch of a kernel from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary (already scaled by the copy-kernel calibration), or None
    when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_bytes_{workload}.txt")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        lines = fh.read().splitlines()
    h = [l.split(":")[-1].strip() for l in lines if l.startswith("# kernel sources sha256")]
    if not h or h[0] != kernel_source_hash():
        return None
    for l in lines:
        if l.startswith(kernel_prefix):
            parts = l.split()
            return int(round((float(parts[-2]) + float(parts[-1])) * 1e6))
    return None


def affinity_cores():
    """Cores the scheduler lets this process run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def host_cores():
    """Worker threads for the CPU leg: the affinity, capped at 16 -- the CPU
    share of a one-GPU slot on an 8-GPU host, however many cores the
    scheduler shows (a larger pool competes with the other slots' jobs)."""
    return max(1, min(16, affinity_cores()))


def cpu_baseline(w, inp, budget_s):
    """The serial C oracle on the host: first on one core, then on every core
    with one contiguous token chunk per core (a thread pool over the same
    unmodified library; ctypes releases the GIL during each call, so the
    chunks run in parallel).  Each chunk is routed as a microbatch of its own,
    as a data-parallel CPU router would; per-token outputs are those of the
    whole batch."""
    import concurrent.futures as cf
    import numpy as np
    import oracle
    L = inp["logits"] if "logits" in inp else None
    if L is None:
        X, Wg = inp["X"], inp["Wg"]
    T = w.T
    # rate on a small prefix, then a prefix sized for the budget
    n0 = min(T, max(w.n_micro, 2048 // max(1, w.n_micro) * w.n_micro))

    def work(a, b, whole):
        """Forward (+ backward, bias update) of tokens [a, b)."""
        m = w.n_micro if whole and b - a == T else 1
        lg = L[a:b] if L is not None else oracle.gate_logits(X[a:b], Wg)
        o = oracle.route(lg, w.k, n_micro=m, capacity_factor=w.capacity_factor, alpha=w.alpha,
                         renorm=w.renorm, select_bias=inp.get("select_bias"))
        if w.backward:
            dl = oracle.backward(lg, w.k, o["counts"], n_micro=m, alpha=w.alpha)
            if L is None:
                oracle.gate_backward(X[a:b], Wg, dl)
        if w.bias_gamma > 0:
            oracle.bias_update(o["counts"], T=b - a, k=w.k, gamma=w.bias_gamma,
                               bias=inp["select_bias"].copy())

    def run(n):
        t0 = time.perf_counter()
        work(0, n, True)
        return time.perf_counter() - t0

    def leg(run_once, half_budget):
        reps, elapsed = 0, 0.0
        while elapsed < half_budget or reps == 0:
            elapsed += run_once()
            reps += 1
            if reps >= 4096:
                break
        return reps, elapsed

    t_small = run(n0)
    n = int(min(T, max(n0, n0 * budget_s / max(t_small, 1e-6))))
    reps, elapsed = leg(lambda: run(n), budget_s * 0.5)
    serial = n * reps / elapsed

    cores = host_cores()
    chunk = max(1, n // cores)
    bounds = [(i * chunk, (i + 1) * chunk if i < cores - 1 else n) for i in range(cores)]
    bounds = [(a, b) for a, b in bounds if b > a]
    with cf.ThreadPoolExecutor(len(bounds)) as ex:
        def run_all():
            t0 = time.perf_counter()
            list(ex.map(lambda ab: work(ab[0], ab[1], False), bounds))
            return time.perf_counter() - t0
        reps_p, elapsed_p = leg(run_all, budget_s * 0.5)
    parallel = n * reps_p / elapsed_p

    what = (f"the first {n} tokens of the seed-0 {w.name} inputs: forward"
            + (" + backward" if w.backward else "")
            + (" incl. gate GEMM" if w.d > 0 else "")
            + (" and its backward" if w.d > 0 and w.backward else "")
            + (" with selection bias" if w.select_bias_scale > 0 else "")
            + (" + bias update" if w.bias_gamma > 0 else ""))
    legs = {"serial": {"value": serial, "cores": 1, "passes": reps, "seconds": round(elapsed, 2)},
            "all_cores": {"value": parallel, "cores": len(bounds), "passes": reps_p,
                          "seconds": round(elapsed_p, 2)}}
    # the faster leg is the baseline (tiny batches split over many threads
    # lose more to per-call overhead than they gain)
    best = "all_cores" if parallel >= serial else "serial"
    sample = (f"oracle (serial C, fp64) on {what}; " +
              (f"{len(bounds)} threads each routing one contiguous chunk of ~{chunk} tokens as "
               f"its own microbatch, x{reps_p} pass(es)" if best == "all_cores"
               else f"one thread, x{reps} pass(es) (faster than {len(bounds)} threads on chunks "
                    f"of ~{chunk} tokens)"))
    return {"value": legs[best]["value"], "unit": "tokens/s", "cores": legs[best]["cores"],
            "affinity_cores": affinity_cores(), "kind": "oracle", "sample": sample,
            "seconds": legs[best]["seconds"], **legs}


PLANNERS = ("eplb_v4", "sinkhorn_r64")


def planner_bench(args):
    """Latency of one planner call (EPLB placement over a v4_shape microbatch's
    counts: 384 experts, 64 extra replicas, 64 GPUs; or the Sinkhorn plan for
    64 ranks in nodes of 8, 50 rounds), GPU events around K back-to-back
    calls, with the oracle timed on the same input."""
    import numpy as np
    import torch
    import load_balancing_statistics_amd as lbs
    from load_balancing_statistics_amd.workloads import WORKLOADS, make_inputs
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    K = args.steps
    if args.workload == "eplb_v4":
        w = WORKLOADS["v4_shape"]
        inp = make_inputs(w, 0)
        p = lbs.make_params(w.T, w.E, w.k, n_micro=w.n_micro, capacity_factor=w.capacity_factor,
                            alpha=w.alpha, renorm=w.renorm)
        out = lbs.alloc_outputs(p, device=dev)
        ws = lbs.alloc_workspace(p, device=dev)
        lbs.moe_route(p, out, ws, logits=torch.from_numpy(inp["logits"]).to(dev))
        weight = out["counts"][0].contiguous()
        cfg = {"workload": "eplb_v4", "E": w.E, "num_phys": w.E + 64, "num_packs": 64}
        call = lambda: lbs.moe_eplb_plan(weight, w.E + 64, 64)
        host_w = weight.cpu().numpy()
        cpu_call = lambda: __import__("oracle").eplb(host_w, w.E + 64, 64)
    else:
        R, per_node, lam = 64, 8, 2.0
        rng = np.random.default_rng(0)
        load = rng.pareto(1.5, size=R) + 1.0
        a = np.maximum(load - load.mean(), 0.0)
        b = np.maximum(load.mean() - load, 0.0)
        b *= a.sum() / b.sum()
        node = np.arange(R) // per_node
        C = np.where(node[:, None] == node[None, :], 0.0, lam)
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float64)).to(dev)
        at, bt, Ct = t(a), t(b), t(C)
        cfg = {"workload": "sinkhorn_r64", "R": R, "ranks_per_node": per_node, "eps": lam, "iters": 50}
        call = lambda: lbs.moe_sinkhorn_plan(at, bt, Ct, lam, 50)
        cpu_call = lambda: __import__("oracle").sinkhorn(a, b, C, lam, 50)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / K
    cpu = None
    if args.cpu_seconds > 0:
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < min(args.cpu_seconds, 2.0) or n == 0:
            cpu_call()
            n += 1
        cpu_us = (time.perf_counter() - t0) / n * 1e6
        cpu = {"value": cpu_us, "unit": "us per call", "cores": 1, "kind": "oracle",
               "sample": f"the same call on the host, {n} repetitions"}
    print(json.dumps({"metric": "planner latency", "value": us, "unit": "us per call", "n_gpus": 1,
                      "steps": K, "warmup": args.warmup, "ms_per_step": us * 1e-3,
                      "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
                      "dtype": "int64/f64", "data": "synthetic", "config": cfg,
                      "roofline": {"bound": "latency", "achieved": None, "peak": None, "unit": None,
                                   "frac": None, "traffic": None},
                      "cpu_baseline": cpu}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    if args.workload in PLANNERS:
        planner_bench(args)
        return

    import numpy as np
    import torch
    import load_balancing_statistics_amd as lbs
    from load_balancing_statistics_amd.workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_inputs(w, 0)
    p = lbs.make_params(w.T, w.E, w.k, n_micro=w.n_micro, d=w.d,
                        capacity_factor=w.capacity_factor, alpha=w.alpha, renorm=w.renorm,
                        save_row_stats=w.backward, select_bias=w.select_bias_scale > 0)
    sbias = (torch.from_numpy(inp["select_bias"]).to(dev) if w.select_bias_scale > 0 else None)
    # input copies for cache rotation
    if w.d > 0:
        X0 = torch.from_numpy(inp["X"].view(np.int16)).to(dev)
        Wg = torch.from_numpy(inp["Wg"].view(np.int16)).to(dev)
        per_copy = X0.numel() * 2
        ncopy = max(1, math.ceil(ROTATE_BYTES / per_copy))
        srcs = [X0] + [X0.clone() for _ in range(ncopy - 1)]
    else:
        L0 = torch.from_numpy(inp["logits"]).to(dev)
        per_copy = L0.numel() * 4
        ncopy = max(1, math.ceil(ROTATE_BYTES / per_copy))
        srcs = [L0] + [L0.clone() for _ in range(ncopy - 1)]
    out = lbs.alloc_outputs(p, device=dev)
    ws = lbs.alloc_workspace(p, device=dev)
    dlogits = torch.empty((w.T, w.E), dtype=torch.float32, device=dev) if w.backward else None
    gate_bwd = w.d > 0 and w.backward
    if gate_bwd:  # gradients of the gate GEMM's inputs
        dX = torch.empty((w.T, w.d), dtype=torch.int16, device=dev)
        dWg = torch.empty((w.d, w.E), dtype=torch.float32, device=dev)
        ws_gb = torch.empty(max(256, lbs.moe_gate_backward_workspace_size(p)), dtype=torch.uint8,
                            device=dev)

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    hev = HipEvents()
    K = args.steps
    ev_rows = [(hev.create(), hev.create()) for _ in range(K)]
    ev_bwd = [(hev.create(), hev.create()) for _ in range(K)] if w.backward else None
    ev_gb = [(hev.create(), hev.create()) for _ in range(K)] if gate_bwd else None

    def step(i, timed):
        src = srcs[i % ncopy]
        kw = dict(X=src, Wg=Wg) if w.d > 0 else dict(logits=src)
        if w.bias_gamma > 0:  # one loss-free balancing step: the bias follows the loads
            lbs.moe_route_with_bias_update(p, out, ws, sbias, w.bias_gamma, stream=stream,
                                           row_pass_events=ev_rows[i] if timed else None, **kw)
        else:
            lbs.moe_route(p, out, ws, stream=stream, row_pass_events=ev_rows[i] if timed else None,
                          select_bias=sbias, **kw)
        if w.backward:
            L = out["logits"] if w.d > 0 else src
            if timed:
                hev.record(ev_bwd[i][0], sh)
            lbs.moe_route_backward(p, L, out["counts"], dlogits, row_stats=out["row_stats"],
                                   stream=stream)
            if timed:
                hev.record(ev_bwd[i][1], sh)
        if gate_bwd:
            if timed:
                hev.record(ev_gb[i][0], sh)
            lbs.moe_gate_backward(p, src, Wg, dlogits, dX=dX, dWg=dWg, workspace=ws_gb, stream=stream)
            if timed:
                hev.record(ev_gb[i][1], sh)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()

    # Let the host enqueue every timed step while the GPU is still busy, so
    # that the timed region measures the GPU and not the Python launch rate.
    def timed_loop(with_events):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(int(2e8))
        t0.record(stream)
        h0 = time.perf_counter()
        for i in range(K):
            step(i, with_events)
        hs = time.perf_counter() - h0
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1), hs

    # 1) the step as a whole, nothing recorded between kernels
    total_ms, host_s = timed_loop(False)
    ms_step = total_ms / K
    # 2) the same steps with events around the dominant kernels
    timed_loop(True)
    rows_ms = sum(hev.elapsed_ms(a, b) for a, b in ev_rows) / K
    bwd_ms = sum(hev.elapsed_ms(a, b) for a, b in ev_bwd) / K if w.backward else None
    gb_ms = sum(hev.elapsed_ms(a, b) for a, b in ev_gb) / K if gate_bwd else None
    status = int(out["status"].item())

    # 3) on request, forward-only workloads: two streams taking alternate
    # batches (each with its own outputs and workspace), as a caller routing a
    # stream of batches can run them; reported beside the one-stream step,
    # never as it (off by default, so that a profiled run times one stream)
    two_stream_ms = None
    if args.two_stream and w.d == 0 and not w.backward and w.bias_gamma == 0:
        s2 = torch.cuda.Stream()
        out2 = lbs.alloc_outputs(p, device=dev)
        ws2 = lbs.alloc_workspace(p, device=dev)
        pairs = [(stream, out, ws), (s2, out2, ws2)]

        def route_on(i):
            st, o, wsp = pairs[i % 2]
            lbs.moe_route(p, o, wsp, stream=st, logits=srcs[i % ncopy], select_bias=sbias)

        for i in range(args.warmup):
            route_on(i)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        joined = torch.cuda.Event()
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(int(2e8))
        t0.record(stream)
        s2.wait_event(t0)
        for i in range(K):
            route_on(i)
        joined.record(s2)
        stream.wait_event(joined)
        t1.record(stream)
        torch.cuda.synchronize()
        two_stream_ms = t0.elapsed_time(t1) / K

    # device-to-device copy ceiling (same rotation logic: 1 GiB buffers)
    cbuf = torch.empty(256 * 1024 * 1024, dtype=torch.float32, device=dev)
    cdst = torch.empty_like(cbuf)
    for _ in range(3):
        cdst.copy_(cbuf)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(10):
        cdst.copy_(cbuf)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * cbuf.numel() * 4 * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del cbuf, cdst

    ab = alg_bytes(w, w.T)
    if gate_bwd:
        # events around the call: the product kernel and the dWg slice reduction
        dom_name, dom_bytes, dom_ms = "gate_backward (product kernel + slice reduction)", ab["gate_backward"], gb_ms
    elif w.d > 0:
        dom_name, dom_bytes, dom_ms = "gate+route forward (no per-kernel split)", ab["forward"], ms_step
    elif w.backward and bwd_ms > rows_ms:
        dom_name, dom_bytes, dom_ms = "route_backward_kernel", ab["route_backward"], bwd_ms
    elif one_launch_path(w):
        # one kernel does the whole forward: the row-pass events time it
        dom_name, dom_bytes, dom_ms = "route_small_kernel", ab["forward"], rows_ms
    else:
        dom_name, dom_bytes, dom_ms = "route_rows_kernel", ab["rows"], rows_ms
    if gate_bwd:  # the kernel the gate backward launches for this E (its reduce step aside)
        traffic = measured_traffic(w.name, "moe::gate_backward_bf16_kernel" if w.E <= 8
                                   else "moe::gate_backward_mfma_kernel" if w.E <= 16
                                   else "moe::gate_backward_kernel<")
    elif one_launch_path(w):
        traffic = measured_traffic(w.name, "moe::route_small_kernel")
    else:
        traffic = measured_traffic(w.name, dom_name) if w.d == 0 else None
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    step_bytes = ab["forward"] + ab["backward"]

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, inp, args.cpu_seconds)

    res = {
        "metric": METRIC,
        "value": w.T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.d == 0 else "bf16-in/f32",
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "E": w.E, "k": w.k, "n_micro": w.n_micro,
                   "d": w.d, "capacity_factor": w.capacity_factor, "alpha": w.alpha,
                   "renorm": w.renorm, "backward": w.backward,
                   "select_bias": w.select_bias_scale > 0, "bias_gamma": w.bias_gamma},
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "alg_bytes_per_launch": dom_bytes,
                     "launch_ms": round(dom_ms, 5)},
        "cpu_baseline": cpu,
        "detail": {"step_alg_bytes": step_bytes,
                   "step_GBps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
                   "row_pass_ms": round(rows_ms, 5),
                   "backward_ms": None if bwd_ms is None else round(bwd_ms, 5),
                   "gate_backward_ms": None if gb_ms is None else round(gb_ms, 5),
                   "copy_ceiling_GBps": round(copy_gbps, 1),
                   # the dominant kernel against the copy ceiling measured here
                   "frac_of_copy_ceiling": round(achieved / copy_gbps, 4),
                   # the step without the backward kernels' event spans
                   "forward_ms": round(ms_step - (bwd_ms or 0.0) - (gb_ms or 0.0), 5),
                   "assignments_per_s": w.T * w.k / (ms_step * 1e-3),
                   "input_copies": ncopy, "host_enqueue_s": round(host_s, 4),
                   "status": status,
                   # per batch with two streams taking alternate batches
                   # (forward-only workloads); value is the one-stream step
                   "two_stream_ms_per_batch": None if two_stream_ms is None else round(two_stream_ms, 5)},
    }
    print(json.dumps(res), flush=True)
    for a, b in ev_rows:
        hev.destroy(a); hev.destroy(b)
    for evs in (ev_bwd, ev_gb):
        for a, b in (evs or []):
            hev.destroy(a); hev.destroy(b)


if __name__ == "__main__":
    main()
