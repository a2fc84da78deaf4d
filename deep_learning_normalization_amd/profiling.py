"""Summaries of rocprofv3 output for the norm kernels (kernel durations and HBM traffic).

    python -m deep_learning_normalization_amd.profiling stats --trace DIR --out FILE --cmd "..."
    python -m deep_learning_normalization_amd.profiling traffic --fetch DIR --write DIR \\
        --workload NAME --kernel SUBSTR --algo-bytes N --out FILE --cmd "..."

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
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
COPY_BYTES = 1 << 30
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def kernel_source_hash():
    """Hash of the HIP sources and the dispatcher."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _one(directory, suffix):
    hits = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError("no *%s under %s" % (suffix, directory))
    return hits[0]


def _short(name):
    """Kernel name without the argument list; torch kernels cut to their first words."""
    base = name.split("(")[0] if "dln::" in name else name[:60]
    return base.replace("void dln::", "").strip()


def stats(trace_dir, out, cmd):
    rows = list(csv.DictReader(open(_one(trace_dir, "_kernel_stats.csv"))))
    trace = list(csv.DictReader(open(_one(trace_dir, "_kernel_trace.csv"))))
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
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
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
    a = ap.parse_args()
    if a.what == "stats":
        stats(a.trace, a.out, a.cmd)
    else:
        print(json.dumps(traffic(a.fetch, a.write, a.workload, a.kernel, a.algo_bytes, a.out,
                                 a.cmd), indent=1))


if __name__ == "__main__":
    main()
