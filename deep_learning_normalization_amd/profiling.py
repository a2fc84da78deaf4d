"""rocprofv3 support for the norm kernels: a workload driver and summaries of kernel durations
and HBM traffic.

    python -m deep_learning_normalization_amd.profiling drive --workload NAME [--steps K]
    python -m deep_learning_normalization_amd.profiling stats --trace DIR --out FILE --cmd "..."
    python -m deep_learning_normalization_amd.profiling traffic --fetch DIR --write DIR \\
        --workload NAME --kernel SUBSTR --algo-bytes N --out FILE --cmd "..."
    python -m deep_learning_normalization_amd.profiling workloads --root DIR --out FILE --cmd "..."
    python -m deep_learning_normalization_amd.profiling summarize --root DIR --out DIR

`drive` runs one workload's forward and backward K times on two rotating buffer sets (run it
under rocprofv3); it first makes the 1 GiB device copies the counter calibration uses.
`workloads` summarises, for every workload, the three runs <root>/<name>/{trace,fetch,write}
of `drive`: per kernel, its average duration, its calibrated HBM bytes and those bytes over
the pass's algorithmic bytes.

`stats` reads <DIR>/*_kernel_stats.csv and *_kernel_trace.csv (rocprofv3 --kernel-trace --stats
--output-format csv) and writes the per-kernel average durations plus the idle gaps between
consecutive norm kernels.

`traffic` reads the FETCH_SIZE and WRITE_SIZE counter collections of two rocprofv3 --pmc runs.
Each counter is calibrated on the 1 GiB device-to-device copies the benchmark makes (a plain
copy kernel of known size): factor = bytes the copy must read (write) / what the counter
reports for it. The result, per launch of the selected kernel, is written as JSON together with
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
COPY_BYTES = 1 << 30
COPY_KERNEL = "__amd_rocclr_copyBuffer"


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


def stats(trace_dir, out, cmd):
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


def traffic(fetch_dir, write_dir, workload, kernel, algo_bytes, out, cmd):
    fetch = _counter(fetch_dir, "FETCH_SIZE")
    write = _counter(write_dir, "WRITE_SIZE")
    # calibration: the 1 GiB copies are the largest copy dispatches
    cf = sorted(fetch.get(COPY_KERNEL, []))[-8:]
    cw = sorted(write.get(COPY_KERNEL, []))[-8:]
    if not cf or not cw:
        raise RuntimeError("no calibration copies in the counter runs")
    f_factor = COPY_BYTES / (statistics.median(cf) * 1024.0)
    w_factor = COPY_BYTES / (statistics.median(cw) * 1024.0)
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

def drive(name, steps):
    """Forward then backward of one workload, `steps` times over two buffer sets."""
    import torch
    from deep_learning_normalization_amd import inputs, normlib as nl
    w = {x.name: x for x in inputs.all_workloads()}[name]
    nl.lib()
    # calibration: 1 GiB device-to-device copies of known size
    a = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    for _ in range(4):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    torch.cuda.empty_cache()
    host = inputs.make(w)
    dev = [{k: (v.cuda() if v is not None else None) for k, v in host.items()} for _ in range(2)]
    ln = w.kind == "layernorm"
    M, N = w.M, w.N
    outs = []
    for d in dev:
        X = d["X"]
        outs.append({"Y": torch.empty_like(X),
                     "H": torch.empty_like(X) if d["R"] is not None else None,
                     "mean": torch.empty(M, device="cuda") if ln else None,
                     "rstd": torch.empty(M, device="cuda"), "dX": torch.empty_like(X)})
    W, B = dev[0]["W"], dev[0]["B"]
    dW = torch.empty_like(W)
    dB = torch.empty_like(W) if ln else None
    wsf = nl.workspace(w.kind, host["X"].dtype, nl.PASS_FWD, M, N, w.r is not None)
    wsb = nl.workspace(w.kind, host["X"].dtype, nl.PASS_BWD, M, N)
    for i in range(steps):
        d, o = dev[i % 2], outs[i % 2]
        nl.norm_fwd(w.kind, d["X"], d["R"], W, B, w.eps, o["Y"], o["H"], o["mean"], o["rstd"],
                    wsf)
        if w.dy is not None:
            Xin = o["H"] if o["H"] is not None else d["X"]
            nl.norm_bwd(w.kind, Xin, d["dY"], None, W, o["mean"], o["rstd"], w.eps, o["dX"],
                        None, dW, dB, wsb)
    torch.cuda.synchronize()


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
             "factors taken from 1 GiB device copies in the same run. 'algorithmic' is the "
             "pass's minimum traffic; the backward's dW/dB partials are extra by design.", "",
             "| workload | kernel | launches | avg us | HBM MB/launch | pass | algorithmic MB | "
             "HBM / algorithmic | GB/s (HBM) |", "|---|---|---|---|---|---|---|---|---|"]
    for w in inputs.all_workloads():
        d = os.path.join(root, w.name)
        if not os.path.isdir(d):
            continue
        dur = _kernel_rows(os.path.join(d, "trace"))
        fetch = _counter(os.path.join(d, "fetch"), "FETCH_SIZE")
        write = _counter(os.path.join(d, "write"), "WRITE_SIZE")
        cf = sorted(fetch.get(COPY_KERNEL, []))[-4:]
        cw = sorted(write.get(COPY_KERNEL, []))[-4:]
        f_factor = COPY_BYTES / (statistics.median(cf) * 1024.0)
        w_factor = COPY_BYTES / (statistics.median(cw) * 1024.0)
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
            bwd_kernel = any(t in short for t in ("bwd", "colsum", "partial", "dx_kernel"))
            alg = bwd_alg if bwd_kernel else fwd_alg
            lines.append("| %s | %s | %d | %.2f | %.1f | %s | %.1f | | %.0f |" % (
                w.name, short, len(dur.get(short, [])), us, (fb + wb) / 1e6,
                "bwd" if bwd_kernel else "fwd", alg / 1e6, (fb + wb) / (us * 1e-6) / 1e9))
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
            lines.append("| %s | **%s pass, all kernels** | | %.2f | %.1f | %s | %.1f | %.3f | "
                         "%.0f |" % (w.name, pname, tot_us, tot_b / 1e6, pname, alg / 1e6,
                                     tot_b / alg, alg / (tot_us * 1e-6) / 1e9))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


HEADLINE_TRACE_CMD = ("cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats -d $REPO/gpurun_out/prof_trace "
                      "-o trace --output-format csv -- python3 $REPO/bench.py --steps 50 --warmup 10 "
                      "--no-cpu-baseline")
HEADLINE_PMC_CMD = ("cd /tmp && TMPDIR=/tmp rocprofv3 --pmc FETCH_SIZE -d $REPO/gpurun_out/prof_fetch -o fetch "
                    "--output-format csv -- python3 $REPO/bench.py --steps 20 --warmup 5 "
                    "--no-cpu-baseline; the same with --pmc WRITE_SIZE -d $REPO/gpurun_out/prof_write "
                    "-o write")
WORKLOAD_CMD = ("cd /tmp && PYTHONPATH=$REPO rocprofv3 {--kernel-trace | --pmc FETCH_SIZE | --pmc "
                "WRITE_SIZE} -d $REPO/gpurun_out/wl/NAME/{trace|fetch|write} -o run --output-format csv "
                "-- python3 -m deep_learning_normalization_amd.profiling drive --workload NAME")


def summarize(root, out):
    """Every committed summary from one capture: the headline command's kernel statistics and
    its fused backward's and forward's traffic (under root/prof_{trace,fetch,write}), and the
    per-workload table (under root/wl)."""
    from deep_learning_normalization_amd import inputs, traffic as model
    w = inputs.LN_BF16_16384x4096
    stats(os.path.join(root, "prof_trace"), os.path.join(out, "kernel_stats_%s.md" % w.name),
          HEADLINE_TRACE_CMD)
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
    sm = sub.add_parser("summarize")
    sm.add_argument("--root", required=True, help="the capture's output folder")
    sm.add_argument("--out", required=True, help="where the summaries go")
    a = ap.parse_args()
    if a.what == "summarize":
        summarize(a.root, a.out)
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
