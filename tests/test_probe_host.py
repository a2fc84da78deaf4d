"""The HBM probe library on the host (no GPU): it loads, exports what include/hbm_probe.h
declares, and refuses bad arguments before touching a device; the benchmark's buffer rotation
moves at least 1 GiB between two uses of a set in every loop."""
import os
import re
import subprocess

import pytest

from deep_learning_normalization_amd import _build, probes, timing, traffic, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hbm_probe.h")


@pytest.fixture(scope="module", autouse=True)
def _lib_built():
    if not os.path.exists(probes.LIB_PATH):
        _build.build()
    probes.lib()


def test_exports_what_the_header_declares():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    declared = set(re.findall(r"\b((?:hbm|mfma|lds)_[a-z_]+)\s*\(", text))
    out = subprocess.run(["nm", "-D", "--defined-only", probes.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    assert declared == {"hbm_probe", "mfma_probe", "lds_probe"}
    assert declared <= set(re.findall(r"\bT ((?:hbm|mfma|lds)_[a-z_]+)\b", out))


def test_header_compiles_as_c():
    r = subprocess.run(["gcc", "-x", "c", "-std=c99", "-Wall", "-Werror", "-I",
                        os.path.dirname(HEADER), "-fsyntax-only", "-"],
                       input='#include "hbm_probe.h"\nint main(void){ return 0; }\n', text=True,
                       capture_output=True)
    assert r.returncode == 0, r.stderr


A, B, C, D = (1 << 40) * 1, (1 << 40) * 2, (1 << 40) * 3, (1 << 40) * 4  # never dereferenced


@pytest.mark.parametrize("args", [
    (1, 1, A, None, C, None, 0, 4, 0, 0),        # no bytes
    (1, 1, A, None, C, None, 24, 4, 0, 0),       # not a multiple of 16
    (1, 1, A, None, C, None, 4096, 3, 0, 0),     # unroll not in {1, 2, 4, 8}
    (1, 1, A, None, C, None, 4096, 4, 2, 0),     # nt_loads not 0 / 1
    (1, 1, A, None, C, None, 4096, 4, 0, -1),    # negative grid
    (0, 0, A, None, C, None, 4096, 4, 0, 0),     # no streams
    (2, 0, A, B, C, None, 4096, 4, 0, 0),        # no such mix
    (1, 2, A, None, C, D, 4096, 4, 0, 0),        # no such mix
    (1, 1, None, None, C, None, 4096, 4, 0, 0),  # missing input
    (2, 1, A, None, C, None, 4096, 4, 0, 0),     # missing second input
    (1, 1, A, None, None, None, 4096, 4, 0, 0),  # missing output
    (2, 2, A, B, C, None, 4096, 4, 0, 0),        # missing second output
    (1, 1, A + 8, None, C, None, 4096, 4, 0, 0),  # unaligned
])
def test_probe_rejects(args):
    nin, nout, i0, i1, o0, o1, nbytes, unroll, nt, grid = args
    assert probes.lib().hbm_probe(nin, nout, i0, i1, o0, o1, nbytes, unroll, nt, grid, 0, None,
                                  None, None) == -1
    # one event without the other
    assert probes.lib().hbm_probe(1, 1, A, None, C, None, 4096, 4, 0, 0, 0, A, None, None) == -1


@pytest.mark.parametrize("args", [
    (8, 1, 256, 16, A),        # no such shape
    (32, 3, 256, 16, A),       # one or two wavefronts per SIMD only
    (32, 1, 0, 16, A),         # no workgroups
    (16, 2, 1 << 30, 16, A),   # grid past 32-bit thread counts
    (32, 1, 256, 0, A),        # no iterations
    (16, 1, 256, 16, None),    # no output
])
def test_mfma_probe_rejects(args):
    shape, waves, grid, iters, out = args
    assert probes.lib().mfma_probe(shape, waves, grid, iters, out, None, None, None) == -1
    assert probes.lib().mfma_probe(32, 1, 256, 16, A, A, None, None) == -1


@pytest.mark.parametrize("args", [
    (3, 256, 16, A),           # 1, 2 or 4 wavefronts per SIMD only
    (1, 0, 16, A),             # no workgroups
    (4, 1 << 30, 16, A),       # grid past 32-bit thread counts
    (2, 256, 0, A),            # no iterations
    (2, 256, 16, None),        # no output
])
def test_lds_probe_rejects(args):
    waves, grid, iters, out = args
    assert probes.lib().lds_probe(waves, grid, iters, out, None, None, None) == -1
    assert probes.lib().lds_probe(1, 256, 16, A, None, A, None) == -1


@pytest.mark.parametrize("w", inputs.all_workloads(), ids=lambda w: w.name)
def test_rotation_moves_a_gib_between_reuses(w):
    """Every timed loop moves at least 1 GiB of its own bytes between two uses of one buffer set,
    and the step loop's forward and backward are S/2 >= 2 sets apart."""
    res = w.r is not None
    fb = traffic.fwd_bytes(w.kind, w.dtype, w.M, w.N, residual=res, wdtype=w.wdtype)
    bb = traffic.bwd_bytes(w.kind, w.dtype, w.M, w.N, wdtype=w.wdtype) if w.dy is not None else 0
    S = timing.set_count(fb, bb)
    assert S >= 4 and S % 2 == 0
    assert S * fb >= 1 << 30
    if bb:
        assert S * bb >= 1 << 30
        assert (S // 2) * (fb + bb) >= 1 << 30
