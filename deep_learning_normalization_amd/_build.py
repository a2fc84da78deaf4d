"""Build libnorm.so (the HIP kernels and the C ABI) and libhbmprobe.so (the HBM bandwidth
probes the benchmark compares against) in-tree for gfx950 with hipcc.

Each source compiles to an object under _build/ in parallel, then one link step per library
writes it next to this file.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libnorm.so")
PROBE_LIB = os.path.join(PKG, "libhbmprobe.so")
PROBE_SOURCES = ["hbm_probe.hip"]

ARCH = os.environ.get("DLN_OFFLOAD_ARCH", "gfx950")
SOURCES = [
    "norm_team.hip", "norm_team_f32.hip", "norm_team_bf16.hip", "norm_team_bf16w.hip",
    "norm_team_f16.hip", "norm_team_f16w.hip", "norm_looped.hip", "norm_split.hip",
    "norm_xsplit.hip", "norm_noalloc.hip",
    "norm_lazy.hip", "norm_lazy_check.cpp", "norm_attn.hip",
    "norm_abi.cpp", "norm_plan.cpp",
]

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops (v_pk_*_f32).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found")
    return exe


def _compile(src, extra):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-x", "hip", "-c", path, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = DEVICE_FLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is expected.
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)


def build(extra_flags=(), jobs=None):
    """Compile every source and link libnorm.so and libhbmprobe.so. Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    jobs = jobs or min(len(srcs), os.cpu_count() or 1, 16)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(sys.argv[1:]))
