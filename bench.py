#!/usr/bin/env python3
"""Benchmark of the row-wise norm hot path on one MI355X.

Headline workload: LayerNorm forward + backward, bf16 storage with fp32 arithmetic,
M = 16384 rows x N = 4096, X ~ N(0,1), dY ~ N(0,1), gamma ~ N(1,0.1), beta ~ N(0,0.1),
eps = 1e-5, synthetic seeded data. One step = norm_fwd on one buffer set, then the backward
(norm_bwd_fused + norm_bwd_reduce, which is exactly what norm_bwd runs) on another set. Sets
rotate over more than 1 GiB, so every pass starts with its inputs in HBM, not in the 256 MB
memory-side cache, and the backward never finds what the forward just touched.

Printed (rank 0, one JSON line): achieved HBM GB/s of forward + backward (algorithmic bytes /
measured time), with the forward and backward figures, a roofline entry for the dominant
kernel (the fused backward pass: on every launch inside the timed region, HIP events take the
kernel's own start and end timestamps) and the CPU oracle timed on this host as a reported
baseline.

--sweep also measures every workload shape (forward, backward, both) and writes the table to
stderr and to --sweep-out.

--projection instead measures the norm deferred into a following projection (norm_lazy_linear
after norm_fold_projection) on its two workloads, next to the unfused pair (norm_fwd, then
torch's 2-D product with the bias, which is hipBLASLt) and the bare hipBLASLt product, and
prints one JSON line per workload with a matrix-core roofline for the product kernel.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, published (no sparsity)
PROFILES = os.path.join(ROOT, "profiles")


def load_traffic(workload_name):
    """HBM bytes per launch of the fused backward from the committed rocprofv3 counter summary,
    or None if there is none or the kernels changed since it was taken."""
    path = os.path.join(PROFILES, "traffic_%s.json" % workload_name)
    if not os.path.exists(path):
        return None, "no counter summary"
    with open(path) as f:
        d = json.load(f)
    from deep_learning_normalization_amd.profiling import kernel_source_hash
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None, "kernels changed since the counters were taken"
    return d, None


class BufferSet:
    """One set of device tensors for a workload (inputs copied from host, outputs empty)."""

    def __init__(self, host, dev, torch):
        self.t = {k: (v.to(dev) if v is not None else None) for k, v in host.items()}
        X = self.t["X"]
        M = X.shape[0]
        self.Y = torch.empty_like(X)
        self.H = torch.empty_like(X) if self.t["R"] is not None else None
        self.mean = torch.empty(M, dtype=torch.float32, device=dev)
        self.rstd = torch.empty(M, dtype=torch.float32, device=dev)
        self.dX = torch.empty_like(X)


def set_bytes(host):
    n = sum(v.numel() * v.element_size() for v in host.values() if v is not None and v.dim() == 2)
    X = host["X"]
    outs = 2 if host["dY"] is not None else 1
    if host["R"] is not None:
        outs += 1
    return n + outs * X.numel() * X.element_size()


def timed_workload(w, steps, warmup, torch, nl, min_footprint=1 << 30, max_sets=64,
                   two_stage=True):
    """Cold-cache timing of one workload. Buffer sets rotate over more than min_footprint
    bytes; the backward of a step uses a different set than its forward. Three loops:
      step : forward, then the backward. two_stage: norm_bwd_fused (its kernels' own
             timestamps recorded into HIP events on every launch, norm_set_launch_events)
             followed by norm_bwd_reduce, which is what norm_bwd runs for the wave and block
             schemes; else norm_bwd, timed the same way as a whole;
      fwd  : forward only;   bwd : norm_bwd only.
    Each loop is bracketed by a synchronize and a pair of events on the launch stream."""
    from deep_learning_normalization_amd import inputs
    dev = torch.device("cuda:0")
    host = inputs.make(w)
    sb = set_bytes(host)
    S = max(2, min(max_sets, -(-min_footprint // sb)))
    if S % 2:
        S += 1
    sets = [BufferSet(host, dev, torch) for _ in range(S)]
    shared = sets[0].t
    W, B = shared["W"], shared["B"]
    M, N = w.M, w.N
    kind = w.kind
    eps = w.eps
    want_bwd = w.dy is not None
    wsf = nl.workspace(kind, host["X"].dtype, nl.PASS_FWD, M, N, w.r is not None)
    wsb = nl.workspace(kind, host["X"].dtype, nl.PASS_BWD, M, N) if want_bwd else None
    dW = torch.empty_like(W)
    dB = torch.empty_like(W) if kind == "layernorm" else None
    stream = torch.cuda.current_stream()

    def fwd(s):
        nl.norm_fwd(kind, s.t["X"], s.t["R"], W, B, eps, s.Y, s.H,
                    s.mean if kind == "layernorm" else None, s.rstd, wsf)

    def bwd_fused(s):
        Xin = s.H if s.H is not None else s.t["X"]
        nl.norm_bwd_fused(kind, Xin, s.t["dY"], None, W,
                          s.mean if kind == "layernorm" else None, s.rstd, eps, s.dX, None, wsb)

    def bwd_reduce():
        nl.norm_bwd_reduce(kind, M, N, dW, dB, wsb)

    def bwd_whole(s):
        Xin = s.H if s.H is not None else s.t["X"]
        nl.norm_bwd(kind, Xin, s.t["dY"], None, W, s.mean if kind == "layernorm" else None,
                    s.rstd, eps, s.dX, None, dW, dB, wsb)

    for s in sets:  # every set gets its statistics (and H) before the backward reads them
        fwd(s)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def run(body, n, timed_kernels=False):
        for i in range(warmup):
            body(i, None)
        torch.cuda.synchronize()
        marks = [nl.KernelTimer() for _ in range(n)] if timed_kernels else [None] * n
        start, end = ev(), ev()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        for i in range(n):
            body(i, marks[i])
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return start.elapsed_time(end) / n, wall, marks

    out = {"sets": S, "set_bytes": sb}

    def step(i, timer):
        fwd(sets[i % S])
        if want_bwd:
            if timer:
                timer.arm()  # the kernels' own start/end timestamps, no extra packets
            if two_stage:
                bwd_fused(sets[(i + S // 2) % S])
                bwd_reduce()
            else:
                bwd_whole(sets[(i + S // 2) % S])

    # the GPU clock settles within a few hundred ms of load: run steps for >= 0.3 s first
    t_end = time.perf_counter() + 0.3
    i = 0
    while time.perf_counter() < t_end or i < warmup:
        step(i, None)
        i += 1
        if i % 50 == 0:
            torch.cuda.synchronize()
    ms, wall, marks = run(step, steps, timed_kernels=want_bwd)
    out["ms_per_step"], out["wall_s"] = ms, wall
    if want_bwd:
        b = sorted(1e3 * m.elapsed_ms() for m in marks)
        out["bwd_timed_us_mean"] = sum(b) / len(b)
        out["bwd_timed_us_median"] = b[len(b) // 2]
        out["bwd_timed_us_p10"] = b[len(b) // 10]
        out["bwd_timed_us_p90"] = b[(9 * len(b)) // 10]
    ms, _, _ = run(lambda i, mk: fwd(sets[i % S]), steps)
    out["fwd_us"] = ms * 1e3
    if want_bwd:
        ms, _, _ = run(lambda i, mk: bwd_whole(sets[i % S]), steps)
        out["bwd_us"] = ms * 1e3
    del sets
    torch.cuda.empty_cache()
    return out


def stats_only(w, torch, nl, steps, warmup):
    """The statistics pass alone (norm_stats) on the workload's X: mean (LayerNorm) and rstd,
    no Y. X sets rotate over more than 1 GiB so every pass starts from HBM. Returns the mean
    loop time per call (launch gaps included) and its algorithmic bytes."""
    from deep_learning_normalization_amd import inputs
    X0 = inputs.make(w)["X"].cuda()
    M, N = w.M, w.N
    nsets = max(2, -(-(1 << 30) // (X0.numel() * X0.element_size())))
    xs = [X0] + [X0.clone() for _ in range(nsets - 1)]
    ln = w.kind == "layernorm"
    mean = torch.empty(M, device="cuda") if ln else None
    rstd = torch.empty(M, device="cuda")
    ws = nl.workspace(w.kind, X0.dtype, nl.PASS_FWD, M, N)
    for i in range(warmup):
        nl.norm_stats(w.kind, xs[i % nsets], None, w.eps, None, mean, rstd, ws)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        nl.norm_stats(w.kind, xs[i % nsets], None, w.eps, None, mean, rstd, ws)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / steps * 1e3
    nbytes = M * N * X0.element_size() + (8 if ln else 4) * M
    del xs
    torch.cuda.empty_cache()
    return us, nbytes


def graph_fwd_us(w, torch, nl, replays=10):
    """Forward calls replayed from a captured graph: one forward per buffer set, the sets
    rotating over more than 1 GiB so that every call starts from HBM as in the eager loops,
    replayed `replays` times; microseconds per forward. For shapes bound by the launch rather
    than by HBM."""
    from deep_learning_normalization_amd import inputs
    host = inputs.make(w)
    ln = w.kind == "layernorm"
    set_bytes = 2 * host["X"].numel() * host["X"].element_size()
    calls = max(20, -(-(1 << 30) // set_bytes))
    sets = []
    for _ in range(calls):
        X = host["X"].cuda()
        sets.append((X, torch.empty_like(X), torch.empty(w.M, device="cuda") if ln else None,
                     torch.empty(w.M, device="cuda")))
    W = host["W"].cuda()
    B = host["B"].cuda() if ln and host["B"] is not None else None
    ws = nl.workspace(w.kind, sets[0][0].dtype, nl.PASS_FWD, w.M, w.N)

    def body():
        for i in range(calls):
            X, Y, mean, rstd = sets[i]
            nl.norm_fwd(w.kind, X, None, W, B, w.eps, Y, None, mean, rstd, ws)
    body()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / (replays * calls)
    del g, sets
    torch.cuda.empty_cache()
    return us


def copy_ceiling(torch, nbytes=1 << 30, iters=20):
    """Achievable HBM bandwidth of a plain device copy (torch's copy kernel), GB/s moved
    (read + write). Two buffer pairs alternate so neither copy starts in cache."""
    n = nbytes // 2
    bufs = [(torch.empty(n, dtype=torch.bfloat16, device="cuda").normal_(),
             torch.empty(n, dtype=torch.bfloat16, device="cuda")) for _ in range(2)]
    for s, d in bufs:
        d.copy_(s)
    torch.cuda.synchronize()
    times = []
    for i in range(iters):
        s, d = bufs[i % 2]
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        d.copy_(s)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    del bufs
    torch.cuda.empty_cache()
    times.sort()
    med = times[len(times) // 2]
    return 2 * nbytes / (med * 1e-3) / 1e9, med * 1e3


def cpu_baseline(w, budget_s=10.0):
    """The CPU oracle (double precision, OpenMP over this host's cores): forward then backward
    of the whole workload, repeated for about budget_s seconds (at least 3 runs); the median
    run, as GB/s over the same algorithmic bytes as the GPU figure."""
    import oracle
    from deep_learning_normalization_amd import inputs, traffic
    host = inputs.make(w)
    bits = {k: inputs.host_bits(host[k]) for k in ("X", "W", "B", "dY")}
    kind = oracle.LAYERNORM if w.kind == "layernorm" else oracle.RMSNORM
    dt = oracle.BF16 if w.dtype == "bf16" else oracle.F32
    eps = float(w.eps)
    times = []
    t_start = time.perf_counter()
    while len(times) < 3 or time.perf_counter() - t_start < budget_s:
        t0 = time.perf_counter()
        oracle.fwd(kind, dt, bits["X"], bits["W"], bits["B"], eps=eps)
        oracle.bwd(kind, dt, bits["X"], bits["dY"], bits["W"], eps=eps)
        times.append(time.perf_counter() - t0)
    total = time.perf_counter() - t_start
    times.sort()
    t = times[len(times) // 2]
    nbytes = traffic.fwd_bytes(w.kind, w.dtype, w.M, w.N) + traffic.bwd_bytes(w.kind, w.dtype,
                                                                               w.M, w.N)
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(nbytes / t / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "whole workload (%d x %d), forward + backward incl. dW/dB, repeated %d "
                      "times in %.1f s; median run %.4f s; %s" % (w.M, w.N, len(times), total, t,
                                                                  cpu),
            "seconds": round(t, 4), "rows_per_s": round(w.M / t, 1),
            "single_thread": oracle_single_thread()}


def oracle_single_thread(runs=3):
    """The oracle on one host thread, median of `runs` runs each: the RMSNorm fp32 2048 x 1024
    forward and the RMSNorm bf16 32768 x 2048 forward + backward (the hidden-size workload),
    as GB/s over their algorithmic bytes."""
    import oracle
    from deep_learning_normalization_amd import inputs, traffic
    threads = oracle.num_threads()
    out = []
    try:
        oracle.set_num_threads(1)
        for w, both in ((inputs.RMS_F32_2048x1024, False), (inputs.rms_hidden(2048), True)):
            host = inputs.make(w)
            bits = {k: inputs.host_bits(host[k]) for k in ("X", "W", "dY")}
            dt = oracle.BF16 if w.dtype == "bf16" else oracle.F32
            times = []
            for _ in range(runs):
                t0 = time.perf_counter()
                oracle.fwd(oracle.RMSNORM, dt, bits["X"], bits["W"], eps=float(w.eps))
                if both:
                    oracle.bwd(oracle.RMSNORM, dt, bits["X"], bits["dY"], bits["W"],
                               eps=float(w.eps))
                times.append(time.perf_counter() - t0)
            t = sorted(times)[len(times) // 2]
            nbytes = traffic.fwd_bytes(w.kind, w.dtype, w.M, w.N)
            if both:
                nbytes += traffic.bwd_bytes(w.kind, w.dtype, w.M, w.N)
            out.append({"workload": w.name, "pass": "fwd+bwd" if both else "fwd",
                        "seconds": round(t, 4), "GBps": round(nbytes / t / 1e9, 3),
                        "rows_per_s": round(w.M / t, 1), "cores": 1})
    finally:
        oracle.set_num_threads(threads)
    return out


def sweep(torch, nl, steps, warmup, out_path, copy_gbps):
    from deep_learning_normalization_amd import inputs, traffic
    rows = []
    for w in inputs.all_workloads():
        r = timed_workload(w, steps, warmup, torch, nl, two_stage=False)
        res = w.r is not None
        fb = traffic.fwd_bytes(w.kind, w.dtype, w.M, w.N, residual=res, wdtype=w.wdtype)
        row = {"workload": w.name, "kind": w.kind, "dtype": w.dtype,
               "weight_dtype": w.wdtype or w.dtype, "M": w.M, "N": w.N,
               "residual": res, "sets": r["sets"], "fwd_us": round(r["fwd_us"], 2),
               "fwd_GBps": round(fb / (r["fwd_us"] * 1e-6) / 1e9, 1)}
        row["fwd_frac_peak"] = round(row["fwd_GBps"] / PEAK_HBM_GBPS, 4)
        if w.M * w.N <= (1 << 22):  # launch-bound sizes: the rate from a replayed graph
            gu = graph_fwd_us(w, torch, nl)
            row["fwd_graph_us"] = round(gu, 2)
            row["fwd_graph_GBps"] = round(fb / (gu * 1e-6) / 1e9, 1)
        row["fwd_rows_per_s"] = round(w.M / (r["fwd_us"] * 1e-6), 1)
        if w.dy is not None:
            bb = traffic.bwd_bytes(w.kind, w.dtype, w.M, w.N, wdtype=w.wdtype)
            step_us = r["ms_per_step"] * 1e3
            row.update({"bwd_us": round(r["bwd_us"], 2),
                        "bwd_GBps": round(bb / (r["bwd_us"] * 1e-6) / 1e9, 1),
                        "bwd_kernels_us": round(r["bwd_timed_us_mean"], 2),
                        "step_us": round(step_us, 2),
                        "fwd_bwd_GBps": round((fb + bb) / (step_us * 1e-6) / 1e9, 1)})
            row["fwd_bwd_frac_peak"] = round(row["fwd_bwd_GBps"] / PEAK_HBM_GBPS, 4)
        rows.append(row)
        sys.stderr.write(json.dumps(row) + "\n")
        sys.stderr.flush()
    if out_path:
        with open(out_path, "w") as f:
            json.dump({"copy_ceiling_GBps": copy_gbps, "rows": rows}, f, indent=1)
    return rows


def projection(p, torch, nl, steps, warmup):
    """One projection workload: the fused product (statistics formed from the X tiles), the
    statistics pass plus the product with given statistics, the unfused pair (norm_fwd to a
    bf16 Y, then torch's 2-D product with the bias in bf16, i.e. hipBLASLt) and that product
    alone. Two
    buffer sets alternate (X, Y: 2 x 256 MiB at 16384 x 4096, beyond the memory-side cache).
    Times are loop times per call over `steps` calls after `warmup`; the product kernel's own
    duration is taken from HIP events on every launch (norm_set_launch_events)."""
    from deep_learning_normalization_amd import inputs
    w = p.norm
    host = inputs.make(w)
    ph = inputs.make_projection(p)
    M, K, Nout = w.M, w.N, p.Nout
    ln = w.kind == "layernorm"
    Xs = [host["X"].cuda() for _ in range(2)]
    g = host["W"].cuda()
    b = host["B"].cuda() if host["B"] is not None else None
    L = ph["L"].cuda()
    c = ph["c"].cuda() if ph["c"] is not None else None
    cb = c.to(torch.bfloat16) if c is not None else None
    Lt = L.t()
    Ys = [torch.empty(M, Nout, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    Ns = [torch.empty_like(Xs[0]) for _ in range(2)]
    mean = torch.empty(M, device="cuda") if ln else None
    rstd = torch.empty(M, device="cuda")
    ws = nl.workspace(w.kind, torch.bfloat16, nl.PASS_FWD, M, K)
    G, sv, tv = nl.fold_projection(w.kind, L, g, b, c)

    def fold(i):
        nl.norm_fold_projection(w.kind, L, g, b, c, G, sv, tv)

    def fused(i):
        nl.norm_lazy_linear(w.kind, Xs[i % 2], w.eps, G, sv, tv, Ys[i % 2])

    def given(i):
        nl.norm_stats(w.kind, Xs[i % 2], None, w.eps, None, mean, rstd, ws)
        nl.norm_lazy_linear(w.kind, Xs[i % 2], w.eps, G, sv, tv, Ys[i % 2], mean_in=mean,
                            rstd_in=rstd)

    def stats(i):
        nl.norm_stats(w.kind, Xs[i % 2], None, w.eps, None, mean, rstd, ws)

    def norm(i):
        nl.norm_fwd(w.kind, Xs[i % 2], None, g, b, w.eps, Ns[i % 2], None, mean, rstd, ws)

    def product(A, Y):
        # hipBLASLt through torch: the 2-D product with L transposed, bias in its epilogue
        if cb is None:
            torch.mm(A, Lt, out=Y)
        else:
            torch.addmm(cb, A, Lt, out=Y)

    def unfused(i):
        norm(i)
        product(Ns[i % 2], Ys[i % 2])

    def linear(i):
        product(Xs[i % 2], Ys[i % 2])

    def loop(body, n, timers=None):
        for i in range(warmup):
            body(i)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(n):
            if timers is not None:
                timers[i].arm()
            body(i)
        e.record()
        torch.cuda.synchronize()
        return a.elapsed_time(e) / n * 1e3

    # settle the clock under load
    t_end = time.perf_counter() + 0.3
    while time.perf_counter() < t_end:
        fused(0)
        torch.cuda.synchronize()
    timers = [nl.KernelTimer() for _ in range(steps)]
    r = {"fused_us": loop(fused, steps, timers)}
    k_us = 1e3 * sum(t.elapsed_ms() for t in timers) / steps
    r["given_us"] = loop(given, steps)
    r["stats_us"] = loop(stats, steps)
    r["norm_fwd_us"] = loop(norm, steps)
    r["unfused_us"] = loop(unfused, steps)
    r["hipblaslt_linear_us"] = loop(linear, steps)
    r["fold_us"] = loop(fold, max(5, steps // 4))
    flops = 2.0 * M * K * Nout
    achieved = flops / (k_us * 1e-6) / 1e12
    out = {
        "workload": p.name, "kind": w.kind, "M": M, "K": K, "Nout": Nout, "dtype": "bf16",
        "what": "Norm(X) L^T + c: rstd * (X G^T - mean * s) + t on the matrix cores, G = "
                "bf16(L * gamma) from norm_fold_projection",
        "flops_per_call": flops,
    }
    out.update({k: round(v, 2) for k, v in r.items()})
    out["lazy_kernel_us"] = round(k_us, 2)
    out["roofline"] = {"bound": "mfma", "kernel": "lazy_linear_kernel", "achieved":
                       round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                       "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None}
    out["hipblaslt_TFLOPs"] = round(flops / (r["hipblaslt_linear_us"] * 1e-6) / 1e12, 1)
    # what the norm adds on top of the bare product, unfused and fused
    out["norm_cost_unfused_us"] = round(r["unfused_us"] - r["hipblaslt_linear_us"], 2)
    out["norm_cost_fused_us"] = round(r["fused_us"] - r["hipblaslt_linear_us"], 2)
    del Xs, Ys, Ns
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true", help="also time every workload shape")
    ap.add_argument("--sweep-out", default=None)
    ap.add_argument("--projection", action="store_true",
                    help="measure the norm deferred into a following projection instead")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures a single MI355X only (rows are independent: a multi-GPU run "
              "would shard rows and all-reduce dW/dB). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from deep_learning_normalization_amd import inputs, normlib as nl, traffic
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    nl.lib()  # fails loudly if libnorm.so is missing

    if args.projection:
        for p in (inputs.LN_LINEAR_BF16_16384x4096x4096, inputs.RMS_LINEAR_BF16_16384x4096x4096):
            print(json.dumps(projection(p, torch, nl, args.steps, args.warmup)), flush=True)
        return

    w = inputs.LN_BF16_16384x4096
    r = timed_workload(w, args.steps, args.warmup, torch, nl)
    copy_gbps, copy_us = copy_ceiling(torch)
    st_us, st_bytes = stats_only(w, torch, nl, args.steps, args.warmup)
    M, N = w.M, w.N
    fb = traffic.fwd_bytes(w.kind, w.dtype, M, N)
    bb = traffic.bwd_bytes(w.kind, w.dtype, M, N)
    bfb = traffic.bwd_fused_bytes(w.kind, w.dtype, M, N)
    ms = r["ms_per_step"]
    value = (fb + bb) / (ms * 1e-3) / 1e9
    # dominant kernel: the fused backward pass; mean launch duration over the timed steps
    bwd_us = r["bwd_timed_us_mean"]
    achieved = bfb / (bwd_us * 1e-6) / 1e9
    tr, why = load_traffic(w.name)
    traffic_bytes = None
    if tr is not None:
        traffic_bytes = tr["hbm_bytes_per_launch"]
    line = {
        "metric": "achieved HBM GB/s (% of peak) for norm fwd and fwd+bwd, bf16, per MxN shape",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; X~N(0,1), dY~N(0,1), gamma~N(1,0.1), beta~N(0,0.1))",
        "config": {"workload": "layernorm_fwd_bwd_bf16", "kind": "layernorm", "M": M, "N": N,
                   "eps": w.eps, "pass": "fwd+bwd", "buffer_sets": r["sets"],
                   "bytes_per_step": fb + bb},
        "roofline": {"bound": "hbm", "kernel": "team_bwd_kernel (fused dX + dW/dB partials)",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic_bytes,
                     "algorithmic_bytes": bfb, "avg_launch_us": round(bwd_us, 3),
                     "launch_us_p10_p50_p90": [round(r["bwd_timed_us_p10"], 3),
                                               round(r["bwd_timed_us_median"], 3),
                                               round(r["bwd_timed_us_p90"], 3)]},
        "fwd": {"us": round(r["fwd_us"], 3), "GBps": round(fb / (r["fwd_us"] * 1e-6) / 1e9, 1),
                "frac_peak": round(fb / (r["fwd_us"] * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                "bytes": fb},
        "bwd": {"us": round(r["bwd_us"], 3), "GBps": round(bb / (r["bwd_us"] * 1e-6) / 1e9, 1),
                "frac_peak": round(bb / (r["bwd_us"] * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                "bytes": bb},
        "fwd_bwd": {"GBps": round(value, 1), "frac_peak": round(value / PEAK_HBM_GBPS, 4),
                    "rows_per_s": round(M / (ms * 1e-3), 1)},
        "copy_ceiling": {"GBps": round(copy_gbps, 1), "us_per_GiB_copy": round(copy_us, 2),
                         "kernel": "HIP runtime device copy of 1 GiB, read + write counted"},
        "stats_only": {"us": round(st_us, 3), "GBps": round(st_bytes / (st_us * 1e-6) / 1e9, 1),
                       "bytes": st_bytes,
                       "what": "norm_stats: mean and rstd without Y (loop time per call)"},
    }
    if traffic_bytes is None:
        line["roofline"]["traffic_note"] = why
    if args.sweep:
        sweep(torch, nl, max(20, args.steps // 4), max(5, args.warmup // 4), args.sweep_out,
              copy_gbps)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
