"""rocprofv3 support for the norm kernels: a workload driver and summaries of kernel durations
and HBM traffic.

    python -m deep_learning_normalization_amd.profiling drive --workload NAME [--steps K]
    python -m deep_learning_normalization_amd.profiling stats --trace DIR --out FILE --cmd "..."
    python -m deep_learning_normalization_amd.profiling traffic --fetch DIR --write DIR \\
        --workload NAME --kernel SUBSTR --algo-bytes N --out FILE --cmd "..."
    python -m deep_learning_normalization_amd.profiling workloads --root DIR --out FILE --cmd "..."
    python -m deep_learning_normalization_amd.profiling summarize --root DIR --out DIR
    python -m deep_learning_normalization_amd.profiling attention-drive [--steps K]
    python -m deep_learning_normalization_amd.profiling attention-stats --trace DIR --out FILE

`drive` runs one workload's step, forward and backward loops K times each with the benchmark's
cache-cold buffer rotation (run it under rocprofv3); it first runs the copy probes the counter
calibration uses.
`workloads` summarises, for every workload, the three runs <root>/<name>/{trace,fetch,write}
of `drive`: per kernel, its average duration, its calibrated HBM bytes and those bytes over
the pass's algorithmic bytes.

`stats` reads <DIR>/*_kernel_stats.csv and *_kernel_trace.csv (rocprofv3 --kernel-trace --stats
--output-format csv) and writes the per-kernel average durations plus the idle gaps between
consecutive norm kernels.

`traffic` reads the FETCH_SIZE and WRITE_SIZE counter collections of two rocprofv3 --pmc runs.
Each counter is calibrated on the copy probes the run makes (include/hbm_probe.h: a plain copy
kernel reading and writing 256 MiB per launch): factor = bytes the copy must read (write) /
what the counter reports for it. The result, per launch of the selected kernel, is written as JSON together with
a hash of the kernel sources, so a later change to the kernels invalidates it.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import shutil
import statistics
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
# Counter calibration: the in-tree copy probe (include/hbm_probe.h) reads and writes exactly
# CALIB_BYTES per launch.
CALIB_KERNEL = "probe_kernel<1, 1,"
CALIB_BYTES = 256 << 20


# Sources of the norm kernels and their dispatcher (launch shapes). The entry-point layer and
# the projection product (norm_lazy.hip, measured on its own) are not part of it.
NORM_KERNEL_SOURCES = ("norm_device.hpp", "norm_internal.hpp", "norm_team_kernels.hpp",
                       "norm_team_menu.hpp", "norm_team.hip", "norm_team_f32.hip",
                       "norm_team_bf16.hip", "norm_team_bf16w.hip", "norm_team_f16.hip",
                       "norm_team_f16w.hip", "norm_looped.hip", "norm_split.hip",
                       "norm_xsplit.hip",
                       "norm_plan.cpp", "norm_plan.hpp")


def kernel_source_hash():
    """Hash of the norm kernels' HIP sources and the dispatcher."""
    h = hashlib.sha256()
    for name in sorted(NORM_KERNEL_SOURCES):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _one(directory, suffix):
    hits = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError("no *%s under %s" % (suffix, directory))
    return hits[0]


_demangled = {}


def _name(raw):
    """A kernel name as rocprofv3 reports it, demangled where it left it mangled (it does not
    demangle _Float16 template arguments, DF16_; they are shown as 'half')."""
    if not raw.startswith("_Z"):
        return raw
    if raw not in _demangled:
        tool = shutil.which("c++filt")
        out = raw
        if tool:
            r = subprocess.run([tool], input=raw.replace("DF16_", "Dh"), capture_output=True,
                               text=True)
            out = r.stdout.strip() or raw
        _demangled[raw] = out if out != raw.replace("DF16_", "Dh") else raw
    return _demangled[raw]


def _short(name):
    """Kernel name without the argument list or namespaces' anonymous part; torch kernels cut to
    their first words."""
    name = name.replace("(anonymous namespace)::", "")
    base = name.split("(")[0] if "dln::" in name else name[:60]
    return base.replace("void dln::", "").strip()


def stats(trace_dir, out, cmd, algo=None):
    """algo: {pass label: (kernel name substring, grid threads or None, algorithmic bytes per
    launch)} for the rate table."""
    rows = list(csv.DictReader(open(_one(trace_dir, "_kernel_stats.csv"))))
    trace = list(csv.DictReader(open(_one(trace_dir, "_kernel_trace.csv"))))
    for r in rows:
        r["Name"] = _name(r["Name"])
    for r in trace:
        r["Kernel_Name"] = _name(r["Kernel_Name"])
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    ours = [r for r in trace if "dln::" in r["Kernel_Name"]]
    gaps = {}
    for prev, cur in zip(ours, ours[1:]):
        g = (int(cur["Start_Timestamp"]) - int(prev["End_Timestamp"])) / 1000.0
        if 0 <= g < 1000:
            gaps.setdefault(_short(cur["Kernel_Name"]), []).append(g)
    lines = ["# rocprofv3 kernel statistics", "", "command: %s" % cmd, "",
             "| kernel | calls | average us | min us | max us | share of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append("| %s | %s | %.2f | %.2f | %.2f | %.1f%% |" % (
            _short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    lines += ["", "Idle time before each norm kernel (end of the previous norm kernel to its "
              "start), median over the run:", "", "| kernel | median gap us | launches |",
              "|---|---|---|"]
    for k, v in sorted(gaps.items()):
        lines.append("| %s | %.2f | %d |" % (k, statistics.median(v), len(v)))
    if algo:
        lines += ["", "Algorithmic bytes per launch over the launch's duration: the average, and "
                  "at the fastest launch (above 8000 GB/s would mean a launch found its data "
                  "in a cache). Launches are told apart by kernel and grid (threads), since the "
                  "statistics pass runs the forward's kernel on a grid of its own:", "",
                  "| pass | kernel | grid threads | algorithmic bytes | launches | average us | "
                  "GB/s at average | fastest us | GB/s at fastest |",
                  "|---|---|---|---|---|---|---|---|---|"]
        for label, (sub, grid, nbytes) in algo.items():
            d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
                 for r in trace if sub in r["Kernel_Name"] and
                 (grid is None or int(r.get("Grid_Size_X", -1)) == grid)]
            if not d:
                continue
            avg, fast = statistics.mean(d), min(d)
            lines.append("| %s | %s | %s | %d | %d | %.2f | %.0f | %.2f | %.0f |" % (
                label, sub, grid if grid is not None else "any", nbytes, len(d), avg,
                nbytes / (avg * 1e3), fast, nbytes / (fast * 1e3)))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    return rows


def _counter(directory, counter):
    path = _one(directory, "_counter_collection.csv")
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return per


def _calibration(fetch, write):
    """Bytes per counter KiB for FETCH_SIZE and WRITE_SIZE, from the copy probes of the run."""
    cf = [v for n, vs in fetch.items() if CALIB_KERNEL in n for v in vs]
    cw = [v for n, vs in write.items() if CALIB_KERNEL in n for v in vs]
    if not cf or not cw:
        raise RuntimeError("no calibration copies (%s) in the counter runs" % CALIB_KERNEL)
    return (CALIB_BYTES / (statistics.median(cf) * 1024.0),
            CALIB_BYTES / (statistics.median(cw) * 1024.0))


def traffic(fetch_dir, write_dir, workload, kernel, algo_bytes, out, cmd):
    fetch = _counter(fetch_dir, "FETCH_SIZE")
    write = _counter(write_dir, "WRITE_SIZE")
    f_factor, w_factor = _calibration(fetch, write)
    names = [n for n in fetch if kernel in n]
    if len(names) != 1:
        raise RuntimeError("kernel filter %r matches %d kernels: %s" % (kernel, len(names), names))
    name = names[0]
    fk = statistics.median(fetch[name]) * 1024.0 * f_factor
    wk = statistics.median(write.get(name, [0.0])) * 1024.0 * w_factor
    d = {"workload": workload, "kernel": _short(name), "launches_fetch": len(fetch[name]),
         "launches_write": len(write.get(name, [])),
         "fetch_kib_raw_median": statistics.median(fetch[name]),
         "write_kib_raw_median": statistics.median(write.get(name, [0.0])),
         "fetch_calibration": f_factor, "write_calibration": w_factor,
         "hbm_read_bytes_per_launch": round(fk), "hbm_write_bytes_per_launch": round(wk),
         "hbm_bytes_per_launch": round(fk + wk), "algorithmic_bytes_per_launch": algo_bytes,
         "traffic_over_algorithmic": round((fk + wk) / algo_bytes, 4),
         "kernel_source_hash": kernel_source_hash(), "command": cmd}
    with open(out, "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")
    return d


# ---- workload driver -------------------------------------------------------------------------

def calibration_copies(torch, probes, n=4):
    """n launches of the copy probe on fresh CALIB_BYTES buffers (the counter calibration)."""
    a = torch.empty(CALIB_BYTES // 4, dtype=torch.int32, device="cuda").random_()
    b = torch.empty_like(a)
    for _ in range(n):
        probes.probe(1, 1, [a], [b], CALIB_BYTES)
    torch.cuda.synchronize()
    del a, b
    torch.cuda.empty_cache()


def drive(name, steps):
    """One workload's step, forward and backward loops (timing.timed_workload: the benchmark's
    cache-cold buffer rotation), `steps` calls each, after the copy probes the counter
    calibration uses."""
    import torch
    from deep_learning_normalization_amd import inputs, normlib as nl, probes, timing
    w = {x.name: x for x in inputs.all_workloads()}[name]
    nl.lib()
    calibration_copies(torch, probes)
    timing.timed_workload(w, steps, 2, torch, nl, settle_s=0.1)
    torch.cuda.synchronize()


# Counter passes for what bounds the streaming kernels (one rocprofv3 --pmc run each; a pass
# stays within the per-block counter limits: 8 SQ, 4 TCC, 4 TCP, 2 TA, 2 GRBM).
COUNTER_PASSES = {
    "sq": ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_LEVEL_WAVES",
           "SQ_INST_LEVEL_VMEM", "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR", "SQ_WAIT_INST_ANY",
           "GRBM_GUI_ACTIVE"],
    "tcc": ["TCC_EA0_RDREQ_LEVEL_sum", "TCC_EA0_RDREQ_sum", "TCC_EA0_WRREQ_LEVEL_sum",
            "TCC_EA0_WRREQ_sum", "GRBM_GUI_ACTIVE"],
    "tcp": ["TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum", "TCP_PENDING_STALL_CYCLES_sum",
            "TA_BUSY_avr", "TA_ADDR_STALLED_BY_TC_CYCLES_sum", "GRBM_GUI_ACTIVE"],
}


def counters_drive(launches=20):
    """The kernels the counter summary compares, `launches` times each with the cache-cold
    rotation: the LayerNorm 16384 x 4096 fused backward and forward, the RMSNorm 32768 x 4096
    fused backward, and the copy and triad probes."""
    import torch
    from deep_learning_normalization_amd import inputs, normlib as nl, probes, timing
    nl.lib()
    for w in (inputs.LN_BF16_16384x4096, inputs.rms_hidden(4096)):
        rot = timing.Rotation(w, torch, nl)
        for i in range(launches):
            rot.bwd_fused(rot.sets[(i + rot.S // 2) % rot.S])
            if w.kind == "layernorm":
                rot.fwd(rot.sets[i % rot.S])
        torch.cuda.synchronize()
        rot.free()
    nbytes = 256 << 20
    bufs = [torch.empty(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(8)]
    for i in range(launches):
        probes.probe(2, 1, [bufs[(3 * i) % 8], bufs[(3 * i + 1) % 8]], [bufs[(3 * i + 2) % 8]],
                     nbytes, 4, 1, 0)
        probes.probe(1, 1, [bufs[(2 * i + 3) % 8]], [bufs[(2 * i + 4) % 8]], nbytes, 2, 1, 0)
    torch.cuda.synchronize()


def _pmc_rows(directory):
    """{(kernel name, grid threads): {counter: [values per dispatch]}} of one --pmc run."""
    path = _one(directory, "_counter_collection.csv")
    per = {}
    for r in csv.DictReader(open(path)):
        key = (_name(r["Kernel_Name"]), int(r.get("Grid_Size", r.get("Grid_Size_X", 0)) or 0),
               r.get("Dispatch_Id"))
        per.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
    out = {}
    for (name, grid, _), cs in per.items():
        d = out.setdefault((name, grid), {})
        for c, v in cs.items():
            d.setdefault(c, []).append(v)
    return out


def counters(root, out, cmd):
    """Markdown summary of the counter passes under root/<pass>/ for the kernels of
    counters_drive: occupancy, memory instructions in flight, DRAM requests in flight and their
    latency."""
    runs = {p: _pmc_rows(os.path.join(root, p)) for p in COUNTER_PASSES}

    kernels = [("LayerNorm 16384x4096 fused backward", "team_bwd_kernel", "true, false"),
               ("LayerNorm 16384x4096 forward", "team_fwd_kernel", None),
               ("RMSNorm 32768x4096 fused backward", "team_bwd_kernel", "false, true"),
               ("triad probe (2R1W)", "probe_kernel<2, 1", None),
               ("copy probe (1R1W)", "probe_kernel<1, 1", None)]

    def pick(run, sub, tail):
        vals = {}
        for (name, grid), cs in run.items():
            if sub in name and (tail is None or tail in name):
                for c, v in cs.items():
                    vals.setdefault(c, []).extend(v)
        return {c: statistics.median(v) for c, v in vals.items()}
    lines = ["# What bounds the streaming kernels: rocprofv3 counters", "",
             "command: %s" % cmd, "",
             "Medians over the dispatches of each kernel. Derived columns: DRAM reads in "
             "flight = TCC_EA0_RDREQ_LEVEL (summed over the L2 channels) / GRBM_GUI_ACTIVE "
             "(summed over the 8 XCDs): a relative measure of the read requests outstanding "
             "to memory; DRAM read latency = RDREQ_LEVEL / RDREQ in cycles; their ratio is "
             "proportional to the read bandwidth; writes likewise; L2 read latency seen by the "
             "vector caches = TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ. The SQ pass's "
             "level counters (SQ_LEVEL_WAVES, SQ_INST_LEVEL_VMEM) read 0 or implausibly low on "
             "this part and are listed raw only.", "",
             "| kernel | GPU cycles (8 XCDs) | DRAM reads in flight | DRAM read latency | "
             "reads in flight / latency | DRAM writes in flight | L2 read latency (TCP) | "
             "TA busy (avg) | TCP pending-stall cycles |",
             "|---|---|---|---|---|---|---|---|---|"]
    for label, sub, tail in kernels:
        sq, tcc, tcp = (pick(runs[p], sub, tail) for p in ("sq", "tcc", "tcp"))
        if not sq or not tcc:
            continue
        g = tcc.get("GRBM_GUI_ACTIVE") or sq.get("GRBM_GUI_ACTIVE") or float("nan")
        f = lambda a, b: a / b if b else float("nan")  # noqa: E731
        rin = f(tcc.get("TCC_EA0_RDREQ_LEVEL_sum", 0), g)
        rlat = f(tcc.get("TCC_EA0_RDREQ_LEVEL_sum", 0), tcc.get("TCC_EA0_RDREQ_sum", 0))
        lines.append("| %s | %.0f | %.0f | %.0f | %.2f | %.0f | %.0f | %.0f | %.3g |"
                     % (label, g, rin, rlat, f(rin, rlat),
                        f(tcc.get("TCC_EA0_WRREQ_LEVEL_sum", 0), g),
                        f(tcp.get("TCP_TCC_READ_REQ_LATENCY_sum", 0),
                          tcp.get("TCP_TCC_READ_REQ_sum", 0)),
                        tcp.get("TA_BUSY_avr", float("nan")),
                        tcp.get("TCP_PENDING_STALL_CYCLES_sum", float("nan"))))
    lines += ["", "Raw medians:", ""]
    for label, sub, tail in kernels:
        for p in COUNTER_PASSES:
            d = pick(runs[p], sub, tail)
            if d:
                lines.append("- %s, %s pass: %s" % (label, p, ", ".join(
                    "%s %.6g" % (k, v) for k, v in sorted(d.items()))))
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def _kernel_rows(trace_dir):
    rows = list(csv.DictReader(open(_one(trace_dir, "_kernel_trace.csv"))))
    per = {}
    for r in rows:
        name = _name(r["Kernel_Name"])
        if "dln::" not in name:
            continue
        per.setdefault(_short(name), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    return per


def workloads(root, out, cmd):
    """Markdown table over every workload directory under root."""
    from deep_learning_normalization_amd import inputs, traffic
    lines = ["# Norm kernels per workload: duration and HBM traffic (rocprofv3)", "",
             "command (per workload NAME): %s" % cmd, "",
             "HBM bytes = FETCH_SIZE x fetch calibration + WRITE_SIZE x write calibration, the "
             "factors taken from the copy probes (256 MiB read and written) in the same run. "
             "'algorithmic' is the "
             "pass's minimum traffic; the backward's dW/dB partials are extra by design.", "",
             "| workload | kernel | launches | avg us | fastest us | HBM MB/launch | pass | "
             "algorithmic MB | HBM / algorithmic | GB/s (HBM) | pass GB/s at fastest launch |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for w in inputs.all_workloads():
        d = os.path.join(root, w.name)
        if not os.path.isdir(d):
            continue
        dur = _kernel_rows(os.path.join(d, "trace"))
        fetch = _counter(os.path.join(d, "fetch"), "FETCH_SIZE")
        write = _counter(os.path.join(d, "write"), "WRITE_SIZE")
        f_factor, w_factor = _calibration(fetch, write)
        res = w.r is not None
        fwd_alg = traffic.fwd_bytes(w.kind, w.dtype, w.M, w.N, residual=res, wdtype=w.wdtype)
        bwd_alg = traffic.bwd_bytes(w.kind, w.dtype, w.M, w.N, wdtype=w.wdtype) \
            if w.dy is not None else 0
        names = {_short(n): n for n in fetch if "dln::" in n}
        for short in sorted(names, key=lambda k: (("bwd" in k or "colsum" in k or "dx" in k
                                                   or "partial" in k), k)):
            full = names[short]
            fb = statistics.median(fetch[full]) * 1024.0 * f_factor
            wb = statistics.median(write.get(full, [0.0])) * 1024.0 * w_factor
            us = statistics.mean(dur.get(short, [float("nan")]))
            fast = min(dur.get(short, [float("nan")]))
            bwd_kernel = any(t in short for t in ("bwd", "colsum", "partial", "dx_kernel"))
            alg = bwd_alg if bwd_kernel else fwd_alg
            # the pass's bytes over the fastest launch, for the kernel that moves the pass's
            # data (its HBM traffic at least half the pass's algorithmic bytes)
            main = (fb + wb) >= 0.5 * alg
            lines.append("| %s | %s | %d | %.2f | %.2f | %.1f | %s | %.1f | | %.0f | %s |" % (
                w.name, short, len(dur.get(short, [])), us, fast, (fb + wb) / 1e6,
                "bwd" if bwd_kernel else "fwd", alg / 1e6, (fb + wb) / (us * 1e-6) / 1e9,
                "%.0f" % (alg / (fast * 1e-6) / 1e9) if main else ""))
        # per pass totals: all kernels of the pass
        for pname, alg, sel in (("fwd", fwd_alg, False), ("bwd", bwd_alg, True)):
            if not alg:
                continue
            tot_b = tot_us = 0.0
            for short, full in names.items():
                bk = any(t in short for t in ("bwd", "colsum", "partial", "dx_kernel"))
                if bk != sel:
                    continue
                tot_b += (statistics.median(fetch[full]) * f_factor +
                          statistics.median(write.get(full, [0.0])) * w_factor) * 1024.0
                tot_us += statistics.mean(dur.get(short, [0.0]))
            lines.append("| %s | **%s pass, all kernels** | | %.2f | | %.1f | %s | %.1f | %.3f | "
                         "%.0f | |" % (w.name, pname, tot_us, tot_b / 1e6, pname, alg / 1e6,
                                       tot_b / alg, alg / (tot_us * 1e-6) / 1e9))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


HEADLINE_TRACE_CMD = ("cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats -d $REPO/gpurun_out/prof_trace "
                      "-o trace --output-format csv -- python3 $REPO/bench.py --steps 50 --warmup 10 "
                      "--no-cpu-baseline --no-shapes")
HEADLINE_PMC_CMD = ("cd /tmp && TMPDIR=/tmp rocprofv3 --pmc FETCH_SIZE -d $REPO/gpurun_out/prof_fetch -o fetch "
                    "--output-format csv -- python3 $REPO/bench.py --steps 20 --warmup 5 "
                    "--no-cpu-baseline --no-shapes; the same with --pmc WRITE_SIZE -d "
                    "$REPO/gpurun_out/prof_write -o write")
WORKLOAD_CMD = ("cd /tmp && PYTHONPATH=$REPO rocprofv3 {--kernel-trace | --pmc FETCH_SIZE | --pmc "
                "WRITE_SIZE} -d $REPO/gpurun_out/wl/NAME/{trace|fetch|write} -o run --output-format csv "
                "-- python3 -m deep_learning_normalization_amd.profiling drive --workload NAME")


ATTENTION_CMD = ("cd /tmp && PYTHONPATH=$REPO rocprofv3 --kernel-trace --stats -d "
                 "$REPO/gpurun_out/attn_trace -o run --output-format csv -- python3 -m "
                 "deep_learning_normalization_amd.profiling attention-drive --steps 20")


def attention_forms(a, torch, nl):
    """The three forms the benchmark compares for attention workload a, on resident inputs:
    the fused call (key pass into a workspace, then the attention kernel with the query norm
    inside), the two-pass form (norm_fwd on the query vectors and on the key vectors, then the
    attention kernel without a norm) and that attention kernel alone."""
    from deep_learning_normalization_amd import inputs
    t = {k: (v.to("cuda") if v is not None else None)
         for k, v in inputs.make_attention(a).items()}
    Q, K, V = t["Q"], t["K"], t["V"]
    O = torch.empty_like(Q)
    ws = torch.empty(nl.attention_workspace_bytes(a.B, a.S, a.Hk, a.D), dtype=torch.uint8,
                     device="cuda")
    Qn, Kn = torch.empty_like(Q), torch.empty_like(K)
    rq = torch.empty(Q.numel() // a.D, device="cuda")
    rk = torch.empty(K.numel() // a.D, device="cuda")
    scale = a.D ** -0.5

    def fused():
        nl.norm_attention_fwd(a.kind, Q, K, V, t["wq"], t["bq"], t["wk"], t["bk"], a.eps, scale,
                              O, None, a.causal, workspace=ws)

    def alone():
        nl.norm_attention_fwd("none", Qn, Kn, V, None, None, None, None, a.eps, scale, O, None,
                              a.causal)

    def unfused():
        nl.norm_fwd(a.kind, Q.view(-1, a.D), None, t["wq"], t["bq"], a.eps, Qn.view(-1, a.D),
                    None, None, rq)
        nl.norm_fwd(a.kind, K.view(-1, a.D), None, t["wk"], t["bk"], a.eps, Kn.view(-1, a.D),
                    None, None, rk)
        alone()
    return {"fused": fused, "unfused": unfused, "attention_alone": alone}


def attention_drive(steps):
    """The attention workload's three forms, alternating, `steps` calls each (run it under
    rocprofv3)."""
    import torch
    from deep_learning_normalization_amd import inputs, normlib as nl
    nl.lib()
    forms = attention_forms(inputs.ATTN_QKNORM_B2_S4096, torch, nl)
    for _ in range(steps):
        for f in forms.values():
            f()
    torch.cuda.synchronize()


def attention_stats(trace_dir, out, cmd):
    """Kernel statistics of the attention capture, plus each attention kernel's matrix-core
    rate at its average duration."""
    from deep_learning_normalization_amd import inputs
    a = inputs.ATTN_QKNORM_B2_S4096
    stats(trace_dir, out, cmd)
    trace = list(csv.DictReader(open(_one(trace_dir, "_kernel_trace.csv"))))
    pairs = a.S * (a.S + 1) // 2 if a.causal else a.S * a.S
    flops = 4 * a.B * a.Hq * a.D * pairs
    by = {}
    for r in trace:
        n = _name(r["Kernel_Name"])
        if "attn_fwd_kernel" in n:
            key = n.replace("(anonymous namespace)::", "").split("(")[0].replace("void dln::", "")
            by.setdefault(key, []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    lines = ["", "Workload %s: B %d, S %d, Hq %d, Hk %d, D %d, %s, %s; %d matrix-product flops "
             "per call (2 D per visible (query, key) pair and product). Template arguments: "
             "<norm (0 LayerNorm, 1 RMSNorm, 2 none), keys normalised by the key pass, causal>."
             % (a.name, a.B, a.S, a.Hq, a.Hk, a.D, a.kind, "causal" if a.causal else "full",
                flops), "",
             "| attention kernel | launches | average us | TFLOP/s at average | of 2500 |",
             "|---|---|---|---|---|"]
    for k, d in sorted(by.items()):
        avg = statistics.mean(d)
        tf = flops / (avg * 1e-6) / 1e12
        lines.append("| %s | %d | %.2f | %.1f | %.3f |" % (k, len(d), avg, tf, tf / 2500.0))
    with open(out, "a") as f:
        f.write("\n".join(lines) + "\n")


def summarize(root, out):
    """Every committed summary from one capture: the headline command's kernel statistics and
    its fused backward's and forward's traffic (under root/prof_{trace,fetch,write}), and the
    per-workload table (under root/wl)."""
    from deep_learning_normalization_amd import inputs, traffic as model
    w = inputs.LN_BF16_16384x4096
    from deep_learning_normalization_amd import normlib as nl

    def grid_threads(pass_):
        p = nl.norm_plan(w.kind, nl.BF16, pass_, w.M, w.N, cu_count=256)
        return p["grid"] * p["threads"]
    stats_bytes = w.M * w.N * 2 + 8 * w.M
    stats(os.path.join(root, "prof_trace"), os.path.join(out, "kernel_stats_%s.md" % w.name),
          HEADLINE_TRACE_CMD,
          {"fused backward": ("team_bwd_kernel", grid_threads(nl.PASS_BWD),
                              model.bwd_fused_bytes(w.kind, w.dtype, w.M, w.N)),
           "forward": ("team_fwd_kernel", grid_threads(nl.PASS_FWD),
                       model.fwd_bytes(w.kind, w.dtype, w.M, w.N)),
           "statistics alone": ("team_fwd_kernel", grid_threads(nl.PASS_STATS), stats_bytes),
           "copy probe": ("probe_kernel<1, 1", None, 2 * (256 << 20)),
           "triad probe": ("probe_kernel<2, 1", None, 3 * (256 << 20))})
    fetch, write = os.path.join(root, "prof_fetch"), os.path.join(root, "prof_write")
    traffic(fetch, write, w.name, "team_bwd_kernel",
            model.bwd_fused_bytes(w.kind, w.dtype, w.M, w.N),
            os.path.join(out, "traffic_%s.json" % w.name), HEADLINE_PMC_CMD)
    traffic(fetch, write, w.name, "team_fwd_kernel",
            model.fwd_bytes(w.kind, w.dtype, w.M, w.N),
            os.path.join(out, "traffic_%s_fwd.json" % w.name),
            "the same two runs as traffic_%s.json" % w.name)
    workloads(os.path.join(root, "wl"), os.path.join(out, "kernels_all_workloads.md"),
              WORKLOAD_CMD)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--trace", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--algo-bytes", type=int, required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--cmd", required=True)
    d = sub.add_parser("drive")
    d.add_argument("--workload", required=True)
    d.add_argument("--steps", type=int, default=20)
    wk = sub.add_parser("workloads")
    wk.add_argument("--root", required=True)
    wk.add_argument("--out", required=True)
    wk.add_argument("--cmd", required=True)
    sub.add_parser("counters-drive")
    cn = sub.add_parser("counters")
    cn.add_argument("--root", required=True)
    cn.add_argument("--out", required=True)
    cn.add_argument("--cmd", required=True)
    ad = sub.add_parser("attention-drive")
    ad.add_argument("--steps", type=int, default=20)
    ast = sub.add_parser("attention-stats")
    ast.add_argument("--trace", required=True)
    ast.add_argument("--out", required=True)
    sm = sub.add_parser("summarize")
    sm.add_argument("--root", required=True, help="the capture's output folder")
    sm.add_argument("--out", required=True, help="where the summaries go")
    a = ap.parse_args()
    if a.what == "summarize":
        summarize(a.root, a.out)
    elif a.what == "attention-drive":
        attention_drive(a.steps)
    elif a.what == "attention-stats":
        attention_stats(a.trace, a.out, ATTENTION_CMD)
    elif a.what == "counters-drive":
        counters_drive()
    elif a.what == "counters":
        counters(a.root, a.out, a.cmd)
    elif a.what == "drive":
        drive(a.workload, a.steps)
    elif a.what == "workloads":
        workloads(a.root, a.out, a.cmd)
    elif a.what == "stats":
        stats(a.trace, a.out, a.cmd)
    else:
        print(json.dumps(traffic(a.fetch, a.write, a.workload, a.kernel, a.algo_bytes, a.out,
                                 a.cmd), indent=1))


if __name__ == "__main__":
    main()
