#!/usr/bin/env python3
"""Benchmark of the row-wise norm hot path on one MI355X.

Headline workload: LayerNorm forward + backward, bf16 storage with fp32 arithmetic,
M = 16384 rows x N = 4096, X ~ N(0,1), dY ~ N(0,1), gamma ~ N(1,0.1), beta ~ N(0,0.1),
eps = 1e-5, synthetic seeded data. One step = norm_fwd on one buffer set, then the backward
(norm_bwd_fused + norm_bwd_reduce, which is exactly what norm_bwd runs) on another set.

Cache-cold protocol (deep_learning_normalization_amd/timing.py): every timed loop (step,
forward only, backward only) cycles through buffer sets sized from that loop's own bytes per
call, so that a set is used again only after at least 1 GiB (four times the 256 MB memory-side
cache) of the loop's traffic, and the step's forward never reads what the backward before it
touched.

Printed (one JSON line): achieved HBM GB/s of forward + backward (algorithmic bytes / measured
time) as `value`; the forward and backward figures; a roofline entry for the dominant kernel (the
fused backward pass: on every launch inside the timed region, HIP events take the kernel's own
start and end timestamps); `ceilings`, what hand-written streaming kernels (include/hbm_probe.h)
reach for each stream mix in the same run; `shapes`, the same figures for every other workload
the metric is quoted on (fractions of the 8 TB/s peak and of the measured ceiling of each pass's
stream mix); and the CPU oracle timed on this host as a reported baseline.

--sweep also times the registry's other workloads (ragged row, hidden 16384, fp16, fp32
weights) into `shapes`.

`attention`: attention over RMSNorm-normalised queries and keys (2 sequences x 4096 tokens, 32
query heads over 8 key/value heads of 128, causal) fused into one call (norm_attention_fwd),
against the same computation in two passes; --attention prints that for causal and full masks,
4096 and 1024 tokens, RMSNorm and LayerNorm, one JSON line each.

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


def stats_only(w, torch, nl, steps, warmup):
    """The statistics pass alone (norm_stats) on the workload's X: mean (LayerNorm) and rstd,
    no Y. X sets rotate over more than 1 GiB so every pass starts from HBM. Returns the mean
    loop time per call (launch gaps included) and its algorithmic bytes."""
    from deep_learning_normalization_amd import inputs
    X0 = inputs.make(w)["X"].cuda()
    M, N = w.M, w.N
    nsets = max(4, -(-(1 << 30) // (X0.numel() * X0.element_size())))
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


def ceiling_for(w, ceilings):
    """The measured ceilings (GB/s) for a workload's forward and backward stream mixes: the
    forward reads one [M, N] stream and writes one (two and two with the residual input), the
    backward reads two and writes one."""
    f = ceilings["2r2w" if w.r is not None else "copy"]
    return f, ceilings["triad"]


def shape_entry(w, r, ceilings):
    """One workload's figures from timing.timed_workload: loop time per call, achieved GB/s
    over the algorithmic bytes, its fraction of the 8 TB/s peak and of the measured ceiling for
    its stream mix, and the per-launch kernel durations."""
    fc, bc = ceiling_for(w, ceilings)
    fb, bb = r["fwd_bytes"], r["bwd_bytes"]
    e = {"workload": w.name, "kind": w.kind, "dtype": w.dtype, "M": w.M, "N": w.N,
         "residual": w.r is not None, "buffer_sets": r["sets"],
         "footprint_GiB": round(r["footprint_bytes"] / (1 << 30), 2)}
    fg = fb / (r["fwd_us"] * 1e-6) / 1e9
    e["fwd"] = {"us": round(r["fwd_us"], 2), "GBps": round(fg, 1),
                "frac_peak": round(fg / PEAK_HBM_GBPS, 4),
                "frac_ceiling": round(fg / fc["GBps"], 4), "ceiling": fc["streams"],
                "kernel_us_mean_p50": [round(r["fwd_kernels_us"]["mean"], 2),
                                       round(r["fwd_kernels_us"]["p50"], 2)],
                "rows_per_s": round(w.M / (r["fwd_us"] * 1e-6), 1), "bytes": fb}
    if bb:
        bg = bb / (r["bwd_us"] * 1e-6) / 1e9
        e["bwd"] = {"us": round(r["bwd_us"], 2), "GBps": round(bg, 1),
                    "frac_peak": round(bg / PEAK_HBM_GBPS, 4),
                    "frac_ceiling": round(bg / bc["GBps"], 4), "ceiling": bc["streams"],
                    "kernel_us_mean_p50": [round(r["bwd_kernels_us"]["mean"], 2),
                                           round(r["bwd_kernels_us"]["p50"], 2)],
                    "bytes": bb}
        step_us = r["ms_per_step"] * 1e3
        sg = (fb + bb) / (step_us * 1e-6) / 1e9
        # the ceiling of a step: each pass at its own mix's ceiling, back to back
        t_ceil = fb / (fc["GBps"] * 1e9) + bb / (bc["GBps"] * 1e9)
        e["fwd_bwd"] = {"us": round(step_us, 2), "GBps": round(sg, 1),
                        "frac_peak": round(sg / PEAK_HBM_GBPS, 4),
                        "frac_ceiling": round(sg * 1e9 * t_ceil / (fb + bb), 4),
                        "rows_per_s": round(w.M / (step_us * 1e-6), 1), "bytes": fb + bb}
    return e


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


def add_mfma_ceiling(roof, mfma):
    """The measured matrix-core ceiling (probes.mfma_ceiling) beside the published peak: these
    kernels issue 32x32x16 bf16 operations, so that shape's best rate is their ceiling."""
    if mfma is None:
        return
    c = mfma["32x32x16"]["TFLOPs"]
    roof["ceiling_TFLOPs"] = c
    roof["frac_ceiling"] = round(roof["achieved"] / c, 4)
    roof["ceiling"] = ("mfma_probe (libhbmprobe.so, include/hbm_probe.h): 32x32x16 bf16 "
                       "operations on register operands, no memory traffic")


def projection(p, torch, nl, steps, warmup, mfma=None):
    """One projection workload: the fused product (statistics formed from the X tiles), the
    statistics pass plus the product with given statistics, the unfused pair (norm_fwd to a
    bf16 Y, then torch's 2-D product with the bias in bf16, i.e. hipBLASLt) and that product
    alone. Two buffer sets alternate (X, Y: 2 x 256 MiB at 16384 x 4096, beyond the
    memory-side cache). The forms alternate call by call, each call bracketed by its own pair
    of HIP events, because the clock drifts by several percent over seconds of matrix-core
    load; the figures are medians over `steps` calls of each form. The product kernel's own
    duration is taken from HIP events on every fused launch (norm_set_launch_events)."""
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

    def product(A, Y):
        # hipBLASLt through torch: the 2-D product with L transposed, bias in its epilogue
        if cb is None:
            torch.mm(A, Lt, out=Y)
        else:
            torch.addmm(cb, A, Lt, out=Y)

    def norm(i):
        nl.norm_fwd(w.kind, Xs[i % 2], None, g, b, w.eps, Ns[i % 2], None, mean, rstd, ws)

    forms = {
        "fused": lambda i: nl.norm_lazy_linear(w.kind, Xs[i % 2], w.eps, G, sv, tv, Ys[i % 2]),
        "given": lambda i: (nl.norm_stats(w.kind, Xs[i % 2], None, w.eps, None, mean, rstd, ws),
                            nl.norm_lazy_linear(w.kind, Xs[i % 2], w.eps, G, sv, tv, Ys[i % 2],
                                                mean_in=mean, rstd_in=rstd)),
        "stats": lambda i: nl.norm_stats(w.kind, Xs[i % 2], None, w.eps, None, mean, rstd, ws),
        "norm_fwd": norm,
        "unfused": lambda i: (norm(i), product(Ns[i % 2], Ys[i % 2])),
        "hipblaslt_linear": lambda i: product(Xs[i % 2], Ys[i % 2]),
        "fold": lambda i: nl.norm_fold_projection(w.kind, L, g, b, c, G, sv, tv),
    }
    t_end = time.perf_counter() + 0.5  # the clock settles under load
    i = 0
    while time.perf_counter() < t_end or i < warmup:
        for f in forms.values():
            f(i)
        i += 1
        torch.cuda.synchronize()
    evs = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)] for k in forms}
    timers = [nl.KernelTimer() for _ in range(steps)]
    for j in range(steps):
        for k, f in forms.items():
            evs[k][j][0].record()
            if k == "fused":
                timers[j].arm()
            f(j)
            evs[k][j][1].record()
    torch.cuda.synchronize()
    r = {}
    for k in forms:
        d = sorted(a0.elapsed_time(a1) * 1e3 for a0, a1 in evs[k])
        r[k + "_us"] = d[len(d) // 2]
    kd = sorted(1e3 * t.elapsed_ms() for t in timers)
    k_us = kd[len(kd) // 2]
    flops = 2.0 * M * K * Nout
    achieved = flops / (k_us * 1e-6) / 1e12
    out = {
        "workload": p.name, "kind": w.kind, "M": M, "K": K, "Nout": Nout, "dtype": "bf16",
        "what": "Norm(X) L^T + c: rstd * (X G^T - mean * s) + t on the matrix cores, G = "
                "bf16(L * gamma) from norm_fold_projection; medians of alternating calls",
        "flops_per_call": flops,
    }
    out.update({k: round(v, 2) for k, v in r.items()})
    out["lazy_kernel_us"] = round(k_us, 2)
    out["roofline"] = {"bound": "mfma", "kernel": "lazy_linear_kernel", "achieved":
                       round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                       "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None}
    add_mfma_ceiling(out["roofline"], mfma)
    out["hipblaslt_TFLOPs"] = round(flops / (r["hipblaslt_linear_us"] * 1e-6) / 1e12, 1)
    # what the norm adds on top of the bare product, unfused and fused
    out["norm_cost_unfused_us"] = round(r["unfused_us"] - r["hipblaslt_linear_us"], 2)
    out["norm_cost_fused_us"] = round(r["fused_us"] - r["hipblaslt_linear_us"], 2)
    del Xs, Ys, Ns
    torch.cuda.empty_cache()
    return out


def attention_flops(a):
    """Matrix-product flops of one call: 2 * D per (query, visible key) pair for each of the two
    products, every query head of every sequence."""
    pairs = a.S * (a.S + 1) // 2 if a.causal else a.S * a.S
    return 4 * a.B * a.Hq * a.D * pairs


def attention_cpu_baseline(a, rows=None):
    """The oracle on `rows` queries at the end of one head (default: the whole head, every
    query of it), as matrix-product flops per second on the host's cores."""
    import oracle
    from deep_learning_normalization_amd import inputs
    t = inputs.make_attention(a)
    hb = inputs.host_bits
    kind = {"rmsnorm": oracle.RMSNORM, "layernorm": oracle.LAYERNORM, "none": oracle.NO_NORM}
    args = [hb(t[n]) for n in ("Q", "K", "V", "wq", "bq", "wk", "bk")]
    rows = a.S if rows is None else rows
    t0 = time.perf_counter()
    oracle.norm_attention(kind[a.kind], *args, eps=a.eps, scale=a.D ** -0.5, causal=a.causal,
                          b=0, h=0, rows=(a.S - rows, a.S))
    sec = time.perf_counter() - t0
    flops = 4 * a.D * sum((s + 1) if a.causal else a.S for s in range(a.S - rows, a.S))
    return {"value": round(flops / sec / 1e12, 6), "unit": "TFLOP/s", "kind": "oracle",
            "cores": oracle.num_threads(), "seconds": round(sec, 3),
            "sample": "the last %d queries of one head (each against %s keys), the norms of "
                      "that head's keys included" % (rows, "its preceding" if a.causal
                                                      else "all %d" % a.S)}


def attention_bench(a, torch, nl, steps, warmup, cpu=False, mfma=None):
    """Attention over normalised queries and keys (norm_attention_fwd with a workspace: the key
    pass, then the attention kernel with the queries normalised inside it) against the same
    computation in two passes (norm_fwd on the query vectors and on the key vectors, then the
    attention kernel without a norm), and that attention kernel alone on the normalised
    inputs. Inputs stay resident (Q, K, V: 100 MB at 2 x 4096 x (32 + 8 + 8) heads x 128). The
    forms alternate call by call, each call bracketed by its own pair of HIP events on the
    stream, because the clock drifts by several percent over seconds of matrix-core load; the
    figures are medians over `steps` calls of each form."""
    from deep_learning_normalization_amd.profiling import attention_forms
    forms = attention_forms(a, torch, nl)
    evs = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)] for k in forms}
    t_end = time.perf_counter() + 0.5  # the clock settles under load
    i = 0
    while time.perf_counter() < t_end or i < warmup:
        for f in forms.values():
            f()
        i += 1
        torch.cuda.synchronize()
    for j in range(steps):
        for k, f in forms.items():
            evs[k][j][0].record()
            f()
            evs[k][j][1].record()
    torch.cuda.synchronize()
    med = {}
    for k in forms:
        d = sorted(a0.elapsed_time(a1) * 1e3 for a0, a1 in evs[k])
        med[k] = d[len(d) // 2]
    flops = attention_flops(a)
    tf = flops / (med["fused"] * 1e-6) / 1e12
    out = {"workload": a.name, "kind": a.kind, "B": a.B, "S": a.S, "Hq": a.Hq, "Hk": a.Hk,
           "D": a.D, "causal": a.causal, "dtype": "bf16", "flops_per_call": flops,
           "fused_us": round(med["fused"], 2), "unfused_us": round(med["unfused"], 2),
           "attention_alone_us": round(med["attention_alone"], 2),
           "fused_speedup_vs_unfused": round(med["unfused"] / med["fused"], 4),
           "what": "norm_attention_fwd (key pass + attention with in-kernel query norm) vs "
                   "norm_fwd(Q) + norm_fwd(K) + attention; medians of alternating calls",
           "roofline": {"bound": "mfma", "kernel": "attn_fwd_kernel (whole fused call: key pass "
                        "included)", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                        "traffic": None}}
    add_mfma_ceiling(out["roofline"], mfma)
    out["attention_alone_TFLOPs"] = round(flops / (med["attention_alone"] * 1e-6) / 1e12, 1)
    if cpu:
        out["cpu_baseline"] = attention_cpu_baseline(a)
    del forms
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-shapes", action="store_true",
                    help="time only the headline workload (for profiling runs)")
    ap.add_argument("--sweep", action="store_true",
                    help="also time the other workloads of the registry (ragged, hidden 16384, "
                         "fp16, fp32 weights)")
    ap.add_argument("--projection", action="store_true",
                    help="measure the norm deferred into a following projection instead")
    ap.add_argument("--attention", action="store_true",
                    help="measure attention over normalised queries and keys instead (causal "
                         "and full, 4096 and 1024 tokens)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures a single MI355X only (rows are independent: a multi-GPU run "
              "would shard rows and all-reduce dW/dB). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from deep_learning_normalization_amd import inputs, normlib as nl, probes, timing
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    nl.lib()  # fails loudly if libnorm.so is missing
    probes.lib()

    if args.projection or args.attention:
        mfma = probes.mfma_ceiling()
        print(json.dumps({"mfma_ceiling_TFLOPs": mfma, "peak_TFLOPs": PEAK_BF16_TFLOPS,
                          "lds_read_bytes_per_clk_per_cu": probes.lds_read_rate()}),
              flush=True)
    if args.projection:
        for p in (inputs.LN_LINEAR_BF16_16384x4096x4096, inputs.RMS_LINEAR_BF16_16384x4096x4096):
            print(json.dumps(projection(p, torch, nl, args.steps, args.warmup, mfma)), flush=True)
        return
    if args.attention:
        from dataclasses import replace
        base = inputs.ATTN_QKNORM_B2_S4096
        for S in (4096, 1024):
            for causal in (True, False):
                for kind in ("rmsnorm", "layernorm"):
                    a = replace(base, S=S, causal=causal, kind=kind,
                                name="qknorm_attention_bf16_b2_s%d_hq32_hk8_d128_%s_%s" % (
                                    S, "causal" if causal else "full", kind))
                    print(json.dumps(attention_bench(a, torch, nl, min(args.steps, 50),
                                                     args.warmup, cpu=(S == 4096 and causal),
                                                     mfma=mfma)),
                          flush=True)
        return

    def say(msg):
        sys.stderr.write("[bench] %s\n" % msg)
        sys.stderr.flush()

    w = inputs.LN_BF16_16384x4096
    say("headline %s: %d steps" % (w.name, args.steps))
    r = timing.timed_workload(w, args.steps, args.warmup, torch, nl)
    say("ceilings: HBM probes")
    ceilings = probes.ceilings()
    st_us, st_bytes = stats_only(w, torch, nl, args.steps, args.warmup)
    M, N = w.M, w.N
    fb, bb, bfb = r["fwd_bytes"], r["bwd_bytes"], r["bwd_fused_bytes"]
    ms = r["ms_per_step"]
    value = (fb + bb) / (ms * 1e-3) / 1e9
    # dominant kernel: the fused backward pass; mean launch duration over the timed steps
    k = r["step_bwd_kernels_us"]
    achieved = bfb / (k["mean"] * 1e-6) / 1e9
    tr, why = load_traffic(w.name)
    traffic_bytes = tr["hbm_bytes_per_launch"] if tr is not None else None
    head = shape_entry(w, r, ceilings)
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
                   "footprint_GiB": head["footprint_GiB"], "bytes_per_step": fb + bb},
        "roofline": {"bound": "hbm", "kernel": "team_bwd_kernel (fused dX + dW/dB partials)",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic_bytes,
                     "algorithmic_bytes": bfb, "avg_launch_us": round(k["mean"], 3),
                     "launch_us_p10_p50_p90": [round(k["p10"], 3), round(k["p50"], 3),
                                               round(k["p90"], 3)],
                     "frac_ceiling": round(achieved / ceilings["triad"]["GBps"], 4),
                     "ceiling": "triad (2R1W)"},
        "fwd": head["fwd"],
        "bwd": head["bwd"],
        "fwd_bwd": head["fwd_bwd"],
        "ceilings": dict(ceilings, kernel="probe_kernel (libhbmprobe.so, include/hbm_probe.h): "
                         "16-byte accesses, nontemporal stores; best of 12 access shapes, "
                         "median of 12 launches each over a rotating 2 GiB pool"),
        "stats_only": {"us": round(st_us, 3), "GBps": round(st_bytes / (st_us * 1e-6) / 1e9, 1),
                       "bytes": st_bytes,
                       "what": "norm_stats: mean and rstd without Y (loop time per call)"},
    }
    if traffic_bytes is None:
        line["roofline"]["traffic_note"] = why
    if not args.no_shapes:
        shapes = []
        extra = [x for x in inputs.all_workloads() if x.name not in inputs.CONFIG_WORKLOADS]
        todo = [x for x in inputs.all_workloads() if x.name in inputs.CONFIG_WORKLOADS
                and x.name != w.name] + (extra if args.sweep else [])
        for x in todo:
            say("shape %s" % x.name)
            rx = timing.timed_workload(x, max(20, args.steps // 2), max(5, args.warmup // 2),
                                       torch, nl)
            e = shape_entry(x, rx, ceilings)
            if x.M * x.N <= (1 << 22):  # launch-bound sizes: the rate from a replayed graph
                gu = timing.graph_fwd_us(x, torch, nl)
                e["fwd"]["graph_us"] = round(gu, 2)
                e["fwd"]["graph_GBps"] = round(rx["fwd_bytes"] / (gu * 1e-6) / 1e9, 1)
            shapes.append(e)
            torch.cuda.empty_cache()
        line["shapes"] = shapes
        say("attention %s" % inputs.ATTN_QKNORM_B2_S4096.name)
        mfma = probes.mfma_ceiling()
        line["attention"] = attention_bench(inputs.ATTN_QKNORM_B2_S4096, torch, nl, 30,
                                            args.warmup, cpu=not args.no_cpu_baseline,
                                            mfma=mfma)
        line["attention"]["mfma_ceilings_TFLOPs"] = mfma
    if not args.no_cpu_baseline:
        say("cpu baseline")
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
