"""The C ABI library on the host (no GPU): it loads, exports every symbol the header declares,
rejects bad arguments before touching a device, and its dispatcher picks the documented
schemes and workspace layouts."""
import ctypes
import math
import os
import re
import subprocess

import pytest
import torch

from deep_learning_normalization_amd import _build, normlib as nl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "norm.h")


@pytest.fixture(scope="module", autouse=True)
def _lib_built():
    if not os.path.exists(nl.LIB_PATH):
        _build.build()
    nl.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(norm_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert set(_declared_functions()) == set(nl.SYMBOLS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", nl.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (norm_[a-z_]+)\b", out))
    missing = set(_declared_functions()) - exported
    assert not missing, missing
    lib = ctypes.CDLL(nl.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name)


def test_header_compiles_as_c():
    src = '#include "norm.h"\nint main(void){ norm_plan_t p; (void)p; return NORM_OK; }\n'
    r = subprocess.run(["gcc", "-x", "c", "-std=c99", "-Wall", "-Werror", "-I",
                        os.path.dirname(HEADER), "-fsyntax-only", "-"], input=src, text=True,
                       capture_output=True)
    assert r.returncode == 0, r.stderr


def test_status_strings():
    for s in range(6):
        assert nl.status_string(s).startswith("NORM_")
    assert "unknown" in nl.status_string(99)
    assert nl.norm_version() >= 100


# ---- argument checks (fail before any device access) -------------------------------------

L = None
FAKE = 1 << 20  # never dereferenced: every call below fails its checks first


def _fwd(**kw):
    a = dict(kind=0, X=FAKE, R=None, W=FAKE * 2, B=None, eps=1e-5, M=4, N=8, dtype=1,
             Y=FAKE * 3, H=None, mean=None, rstd=None, ws=None, wsb=0, stream=None)
    a.update(kw)
    return nl.lib().norm_fwd(a["kind"], a["X"], a["R"], a["W"], a["B"], a["eps"], a["M"], a["N"],
                             a["dtype"], a["Y"], a["H"], a["mean"], a["rstd"], a["ws"], a["wsb"],
                             a["stream"])


def _bwd(**kw):
    a = dict(kind=0, X=FAKE, dY=FAKE * 2, dH=None, W=FAKE * 3, mean=None, rstd=None, eps=1e-5,
             M=4, N=8, dtype=1, dX=FAKE * 4, dR=None, dW=FAKE * 5, dB=None, ws=None, wsb=0,
             stream=None)
    a.update(kw)
    return nl.lib().norm_bwd(a["kind"], a["X"], a["dY"], a["dH"], a["W"], a["mean"], a["rstd"],
                             a["eps"], a["M"], a["N"], a["dtype"], a["dX"], a["dR"], a["dW"],
                             a["dB"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(kind=2), dict(kind=-1), dict(dtype=5), dict(M=-1), dict(N=0), dict(N=-5),
    dict(N=1 << 31), dict(eps=-1e-5), dict(eps=float("nan")), dict(eps=float("inf")),
    dict(X=None), dict(W=None), dict(Y=None),
    dict(kind=1, B=FAKE * 9), dict(kind=1, mean=FAKE * 9),
    dict(R=FAKE * 9), dict(H=FAKE * 9),                  # R and H go together
    dict(Y=FAKE),                                        # in place
    dict(Y=FAKE + 16),                                   # overlapping the input
    dict(mean=FAKE * 3 + 8),                             # output overlapping an output
    dict(M=1 << 40, N=1 << 30),                          # size overflow
], ids=lambda kw: ",".join("%s=%s" % i for i in kw.items()))
def test_fwd_rejects(kw):
    assert _fwd(**kw) == nl.ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [
    dict(kind=3), dict(dtype=7), dict(M=-2), dict(N=0), dict(eps=-1.0),
    dict(X=None), dict(dY=None), dict(W=None), dict(dX=None), dict(dW=None),
    dict(kind=1, dB=FAKE * 9), dict(kind=1, mean=FAKE * 9, rstd=FAKE * 10),
    dict(mean=FAKE * 9),                                 # LayerNorm: mean and rstd together
    dict(rstd=FAKE * 9),
    dict(dX=FAKE * 2),                                   # dX over dY
    dict(dR=FAKE * 2 + 4),                               # dR over dY
    dict(dW=FAKE * 3),                                   # dW over W
    dict(ws=FAKE * 4, wsb=64),                           # workspace over dX
], ids=lambda kw: ",".join("%s=%s" % i for i in kw.items()))
def test_bwd_rejects(kw):
    assert _bwd(**kw) == nl.ERR_INVALID_ARG


def _strides(**kw):
    ld = nl.RowStrides()
    for k, v in kw.items():
        setattr(ld, k, v)
    return ctypes.byref(ld)


def _fwd_ex(ld, **kw):
    a = dict(kind=0, X=FAKE, R=None, W=FAKE * 2, B=None, eps=1e-5, M=4, N=8, dtype=1,
             Y=FAKE * 3, H=None, mean=None, rstd=None, ws=None, wsb=0, stream=None)
    a.update(kw)
    return nl.lib().norm_fwd_ex(a["kind"], a["X"], a["R"], a["W"], a["B"], a["eps"], a["M"],
                                a["N"], a["dtype"], a["Y"], a["H"], a["mean"], a["rstd"], a["ws"],
                                a["wsb"], ld, a["stream"])


def _bwd_ex(ld, **kw):
    a = dict(kind=0, X=FAKE, dY=FAKE * 2, dH=None, W=FAKE * 3, mean=None, rstd=None, eps=1e-5,
             M=4, N=8, dtype=1, dX=FAKE * 4, dR=None, dW=FAKE * 5, dB=None, ws=None, wsb=0,
             stream=None)
    a.update(kw)
    return nl.lib().norm_bwd_ex(a["kind"], a["X"], a["dY"], a["dH"], a["W"], a["mean"],
                                a["rstd"], a["eps"], a["M"], a["N"], a["dtype"], a["dX"], a["dR"],
                                a["dW"], a["dB"], a["ws"], a["wsb"], ld, a["stream"])


def test_row_strides_on_the_host():
    # a NULL struct and all-zero strides are the contiguous call
    assert _fwd_ex(None) == _fwd() == nl.ERR_HIP
    assert _fwd_ex(_strides()) == nl.ERR_HIP
    # a stride below N is rejected; N or more is accepted (then no device)
    assert _fwd_ex(_strides(x=7)) == nl.ERR_INVALID_ARG
    assert _fwd_ex(_strides(y=-8)) == nl.ERR_INVALID_ARG
    assert _fwd_ex(_strides(x=24, y=9)) == nl.ERR_HIP
    # spans grow with the stride: X rows 3 x 64 elements apart (bf16) now reach Y at FAKE * 3
    # only if (M - 1) * ld + N elements cover 2 MiB: M = 4, ld = 2^19 does
    assert _fwd_ex(_strides(x=1 << 19)) == nl.ERR_INVALID_ARG
    assert _fwd_ex(_strides(x=1 << 17)) == nl.ERR_HIP
    # a residual stride is checked only with R
    assert _fwd_ex(_strides(r=3)) == nl.ERR_HIP
    assert _fwd_ex(_strides(r=3), R=FAKE * 5, H=FAKE * 6) == nl.ERR_INVALID_ARG
    # backward: dR may alias dX only with the same stride
    assert _bwd_ex(_strides(dx=16, dr=16), dR=FAKE * 4) == nl.ERR_HIP
    assert _bwd_ex(_strides(dx=16, dr=8), dR=FAKE * 4) == nl.ERR_INVALID_ARG
    assert _bwd_ex(_strides(dy=5)) == nl.ERR_INVALID_ARG
    # a stride overflowing the addressable span
    assert _fwd_ex(_strides(x=1 << 60)) == nl.ERR_INVALID_ARG


def _stats(**kw):
    a = dict(kind=0, X=FAKE, R=None, eps=1e-5, M=4, N=8, dtype=1, H=None, mean=FAKE * 3,
             rstd=FAKE * 4, ws=None, wsb=0, ld=None, stream=None)
    a.update(kw)
    return nl.lib().norm_stats(a["kind"], a["X"], a["R"], a["eps"], a["M"], a["N"], a["dtype"],
                               a["H"], a["mean"], a["rstd"], a["ws"], a["wsb"], a["ld"],
                               a["stream"])


def test_stats_only_on_the_host():
    assert _stats() == nl.ERR_HIP                              # valid: then no device
    assert _stats(mean=None) == nl.ERR_HIP                     # rstd alone
    assert _stats(mean=None, rstd=None) == nl.ERR_INVALID_ARG  # nothing to compute
    assert _stats(mean=None, rstd=None, R=FAKE * 5, H=FAKE * 6) == nl.ERR_HIP  # H alone
    assert _stats(kind=1) == nl.ERR_INVALID_ARG                # RMSNorm has no mean
    assert _stats(kind=1, mean=None) == nl.ERR_HIP
    assert _stats(R=FAKE * 5) == nl.ERR_INVALID_ARG            # R without H
    assert _stats(X=None) == nl.ERR_INVALID_ARG
    assert _stats(mean=FAKE + 8) == nl.ERR_INVALID_ARG         # an output inside X
    assert _stats(eps=-1.0) == nl.ERR_INVALID_ARG
    assert _stats(M=0, X=None) == nl.OK
    # its plan: the forward's shapes on a persistent grid (8 workgroups per CU), the forward's
    # workspace
    for N in (512, 4096, 8192, 262144):
        f = nl.norm_plan(0, BF, nl.PASS_FWD, 16384, N, cu_count=256)
        st = nl.norm_plan(0, BF, nl.PASS_STATS, 16384, N, cu_count=256)
        for k in ("scheme", "team_threads", "accesses_per_thread", "workspace_bytes"):
            assert f[k] == st[k], (N, k)
        if st["scheme"] == nl.SCHEME_BLOCK:
            assert st["grid"] == min(16384, 256 * 8)


def test_dr_may_alias_dx_and_zero_rows_need_no_pointers():
    # dR == dX passes the checks; with no device the call then fails at the device query
    assert _bwd(dR=FAKE * 4) == nl.ERR_HIP
    # M == 0: the forward is a no-op that needs no row pointers and no device
    assert _fwd(M=0, X=None, Y=None) == nl.OK


def test_tuning_rejects_bad_values():
    lib = nl.lib()
    assert lib.norm_set_tuning(nl.TUNE_SCHEME, 7) == nl.ERR_INVALID_ARG
    assert lib.norm_set_tuning(nl.TUNE_ROWS_PER_ITER, 3) == nl.ERR_INVALID_ARG
    assert lib.norm_set_tuning(nl.TUNE_TEAM_THREADS, 100) == nl.ERR_INVALID_ARG
    assert lib.norm_set_tuning(99, 1) == nl.ERR_INVALID_ARG
    assert lib.norm_set_tuning(nl.TUNE_ROW_ORDER, 2) == nl.ERR_INVALID_ARG
    assert lib.norm_set_tuning(nl.TUNE_SCHEME, -1) == nl.OK


# ---- the dispatcher --------------------------------------------------------------------------

BF, F = torch.bfloat16, torch.float32
BF32W = nl.BF16_F32W


def test_scheme_boundaries():
    # one row per wavefront up to N = 1024, a team of wavefronts above, split for long rows
    for dt in (BF, F):
        assert nl.norm_plan(0, dt, 0, 4096, 1024)["scheme"] == nl.SCHEME_WAVE
        assert nl.norm_plan(0, dt, 0, 4096, 1025)["scheme"] == nl.SCHEME_BLOCK
        assert nl.norm_plan(1, dt, 1, 4096, 1024)["scheme"] == nl.SCHEME_WAVE
        assert nl.norm_plan(1, dt, 1, 4096, 1032)["scheme"] == nl.SCHEME_BLOCK
    assert nl.norm_plan(0, BF, 0, 256, 262144)["scheme"] == nl.SCHEME_SPLIT
    assert nl.norm_plan(1, BF, 1, 4, 4194304)["scheme"] == nl.SCHEME_SPLIT
    assert nl.norm_plan(0, BF, 0, 16384, 16384)["scheme"] == nl.SCHEME_BLOCK
    assert nl.norm_plan(0, BF, 0, 16384, 16392)["scheme"] == nl.SCHEME_SPLIT
    # the backward holds twice the state per element: its block rows end at 8192 bf16; the
    # looped backward (two sweeps, the second from the L2) takes rows up to 16384 bf16 / 8192
    # fp32 with 16- or 8-byte accesses, and the split scheme what is longer
    assert nl.norm_plan(0, BF, 1, 16384, 8192)["scheme"] == nl.SCHEME_BLOCK
    assert nl.norm_plan(0, BF, 1, 16384, 8200)["scheme"] == nl.SCHEME_LOOP
    assert nl.norm_plan(0, BF, 1, 16384, 16384)["scheme"] == nl.SCHEME_LOOP
    assert nl.norm_plan(0, BF, 1, 16384, 16380)["scheme"] == nl.SCHEME_LOOP   # 8-byte
    assert nl.norm_plan(0, BF, 1, 16384, 16382)["scheme"] == nl.SCHEME_SPLIT  # 4-byte
    assert nl.norm_plan(0, BF, 1, 16384, 16392)["scheme"] == nl.SCHEME_SPLIT
    assert nl.norm_plan(0, F, 1, 16384, 8192)["scheme"] == nl.SCHEME_LOOP
    assert nl.norm_plan(0, F, 1, 16384, 8196)["scheme"] == nl.SCHEME_SPLIT
    # odd rows: 16-byte accesses over row phase classes in the block scheme while the class
    # whose rows start 7 elements past a boundary needs at most 1024 accesses (N <= 8185 bf16),
    # element-wise in the split scheme beyond
    assert nl.norm_plan(0, BF, 1, 16384, 4095)["scheme"] == nl.SCHEME_BLOCK
    assert nl.norm_plan(0, BF, 1, 16384, 4097)["scheme"] == nl.SCHEME_BLOCK
    assert nl.norm_plan(0, BF, 1, 16384, 8185)["scheme"] == nl.SCHEME_BLOCK
    assert nl.norm_plan(0, BF, 1, 16384, 8187)["scheme"] == nl.SCHEME_SPLIT   # element-wise
    assert nl.norm_plan(0, BF, 0, 16384, 16377)["scheme"] == nl.SCHEME_BLOCK
    assert nl.norm_plan(0, BF, 0, 16384, 16379)["scheme"] == nl.SCHEME_SPLIT   # element-wise
    try:
        nl.norm_set_tuning(nl.TUNE_UNALIGNED, 0)
        assert nl.norm_plan(0, BF, 1, 16384, 4095)["scheme"] == nl.SCHEME_BLOCK   # element-wise
        assert nl.norm_plan(0, BF, 1, 16384, 4097)["scheme"] == nl.SCHEME_SPLIT   # element-wise
    finally:
        nl.norm_set_tuning(nl.TUNE_UNALIGNED, -1)
    # forcing the looped scheme leaves the forward to the dispatcher
    try:
        nl.norm_set_tuning(nl.TUNE_SCHEME, nl.SCHEME_LOOP)
        assert nl.norm_plan(0, BF, 0, 64, 4096)["scheme"] == nl.SCHEME_BLOCK
        assert nl.norm_plan(0, BF, 1, 64, 4096)["scheme"] == nl.SCHEME_LOOP
        with pytest.raises(nl.NormError):
            nl.norm_plan(0, BF, 1, 64, 4098)    # 4-byte accesses: no looped kernel
    finally:
        nl.norm_set_tuning(nl.TUNE_SCHEME, -1)


def test_wide_row_grids():
    """Grids of the wide-row plans, with 256 CUs."""
    F16 = torch.float16
    g = lambda *a, **k: nl.norm_plan(*a, cu_count=256, **k)
    # forwards of 16-bit rows on 320-512-thread teams with four accesses: two persistent
    # workgroups per CU (RMSNorm and the residual form up to 384 threads), short-lived otherwise
    for kind, dt, N, res in [(0, BF, 8200, False), (0, BF, 16384, False), (0, F16, 10240, False),
                             (1, BF, 12288, False), (1, BF, 10240, True), (0, F16, 12288, True),
                             (0, BF32W, 16384, False), (1, BF32W, 10240, False),
                             (0, F, 4100, False), (0, F, 5120, False)]:
        p = g(kind, dt, 0, 16384, N, residual=res)
        assert p["threads"] > 256 and p["accesses_per_thread"] == 4 and p["grid"] == 512, (kind, N)
    # (short-lived: two row groups a workgroup, one in the residual form)
    for kind, dt, N, res in [(1, BF, 14336, False), (1, BF, 16384, False), (0, BF, 16384, True),
                             (1, BF, 7168, True), (0, F, 6144, False), (0, BF, 8192, False),
                             (1, F, 4100, False), (0, F, 4100, True), (1, BF32W, 16384, False)]:
        assert g(kind, dt, 0, 16384, N, residual=res)["grid"] == (16384 if res else 8192), (kind, N)
    # looped backward: two workgroups per CU for rows of at most 1792 16-byte accesses whose
    # kernel fits two 512-thread teams (RMSNorm on 16-bit rows, fp32 rows, and 16-bit LayerNorm
    # rows of at most 1536 accesses through its three-segment kernel), for every 16-bit
    # LayerNorm row (its four-segment kernel keeps dB in LDS), one otherwise
    for kind, dt, N, seg in [(1, BF, 8200, 4), (1, BF, 14336, 4), (0, F, 4100, 4), (1, F, 7168, 4),
                             (0, BF, 8200, 3), (0, BF, 12288, 3), (0, F16, 10240, 3),
                             (0, BF32W, 10240, 3), (0, BF, 12296, 4), (0, BF, 16384, 4),
                             (0, BF32W, 14336, 4), (0, F16, 12296, 4), (0, F16, 16384, 4)]:
        p = g(kind, dt, 1, 16384, N)
        assert (p["scheme"], p["accesses_per_thread"], p["grid"]) == (nl.SCHEME_LOOP, seg, 512), \
            (kind, N)
    for kind, dt, N, seg in [(1, BF, 16384, 4), (1, F16, 16384, 4), (0, F, 8192, 4),
                             (1, BF, 16380, 8), (0, BF, 16380, 8)]:
        p = g(kind, dt, 1, 16384, N)
        assert (p["scheme"], p["accesses_per_thread"], p["grid"]) == (nl.SCHEME_LOOP, seg, 256), \
            (kind, N)
    # backward over phase classes: four rows at a time on 320-384-thread teams with one access
    for kind, dt, N, rows in [(0, BF, 2049, 4), (1, BF, 2049, 4), (0, F, 1025, 4), (0, BF, 2561, 4),
                              (0, BF, 1537, 2), (0, BF, 3073, 2), (0, BF, 4097, 2),
                              (0, BF32W, 2049, 2)]:
        p = g(kind, dt, 1, 16384, N)
        assert p["phase_classes"] > 1 and p["rows_per_iter"] == rows, (kind, N)
    assert g(0, BF, 1, 16384, 2049, residual=True)["rows_per_iter"] == 2
    # fewer rows than workgroups: one workgroup a row
    assert g(0, BF, 1, 300, 10240)["grid"] == 300
    # a grid override applies to the looped backward as given
    try:
        nl.norm_set_tuning(nl.TUNE_GRID_PER_CU, 1)
        assert g(1, BF, 1, 16384, 10240)["grid"] == 256
        assert g(0, BF, 1, 16384, 10240)["accesses_per_thread"] == 3
    finally:
        nl.norm_set_tuning(nl.TUNE_GRID_PER_CU, -1)


def test_backward_team_rules():
    """Backward plans of 16-bit rows up to 3584 elements, with 256 CUs: (threads, accesses per
    thread, rows at a time, grid)."""
    F16 = torch.float16
    cases = [
        ((1, BF, 65536, 256), (256, 1, 4, 512)),    # wave, one access: RMSNorm four rows
        ((1, F16, 65536, 512), (256, 1, 4, 512)),
        ((0, BF, 65536, 512), (256, 1, 2, 512)),    # LayerNorm two
        ((1, BF, 65536, 768), (256, 2, 1, 512)),    # two accesses: one row
        ((0, F, 65536, 512), (256, 2, 1, 512)),     # fp32 unchanged
        ((1, BF, 65536, 1280), (192, 1, 2, 768)),   # 192-thread two-row teams: three per CU
        ((0, BF, 65536, 1536), (192, 1, 2, 768)),
        ((1, BF, 65536, 2560), (320, 1, 2, 512)),   # RMSNorm 320-384 threads: two per CU
        ((1, F16, 65536, 3072), (384, 1, 2, 512)),
        ((1, BF, 65536, 3584), (448, 1, 2, 256)),   # 448 threads: one
        ((0, BF, 65536, 2304), (256, 2, 1, 512)),   # LayerNorm 257-384 accesses: 256 x 2
        ((0, F16, 65536, 3072), (256, 2, 1, 512)),
        ((0, BF, 65536, 3584), (448, 1, 2, 256)),
        ((0, BF, 16384, 4096), (512, 1, 2, 256)),   # the 4096-element plan is unchanged
        ((0, F, 65536, 1536), (384, 1, 2, 256)),   # fp32 LayerNorm on 384 threads: one per CU
        ((1, F, 65536, 256), (256, 1, 4, 512)),     # fp32 wave, one access
        ((0, F, 65536, 256), (256, 1, 2, 512)),
        ((1, F, 65536, 1536), (384, 1, 2, 512)),    # fp32 RMSNorm 320-384 threads: two per CU
        ((0, F, 65536, 1280), (320, 1, 2, 512)),    # fp32 LayerNorm 320 threads: two per CU
        ((1, BF32W, 65536, 512), (256, 1, 4, 512)),  # fp32 weights follow the 16-bit rows
        ((0, BF32W, 65536, 1536), (192, 1, 2, 768)),
        ((1, BF32W, 65536, 2560), (320, 1, 2, 512)),
        ((0, BF32W, 65536, 2560), (256, 2, 1, 512)),
    ]
    for (kind, dt, M, N), want in cases:
        p = nl.norm_plan(kind, dt, 1, M, N, cu_count=256)
        got = (p["threads"], p["accesses_per_thread"], p["rows_per_iter"], p["grid"])
        assert got == want, (kind, dt, N, got)
    # the residual form keeps the earlier plans
    p = nl.norm_plan(1, BF, 1, 65536, 2560, residual=True, cu_count=256)
    assert p["grid"] == 256
    p = nl.norm_plan(0, BF, 1, 65536, 2560, residual=True, cu_count=256)
    assert p["threads"] == 320
    # overrides win over the rules
    try:
        nl.norm_set_tuning(nl.TUNE_ROWS_PER_ITER, 1)
        assert nl.norm_plan(1, BF, 1, 65536, 512, cu_count=256)["rows_per_iter"] == 1
        assert nl.norm_plan(0, BF, 1, 65536, 2560, cu_count=256)["threads"] == 320
    finally:
        nl.norm_set_tuning(nl.TUNE_ROWS_PER_ITER, -1)


def test_access_width_follows_row_length_and_alignment():
    def width(dt, N, align=16, pass_=0):
        p = nl.norm_plan(0, dt, pass_, 64, N, align=align)
        assert p["access_bytes"] == p["elems_per_access"] * (4 if dt == F else 2)
        return p["access_bytes"]
    # 16 bytes when N is a multiple of the 16-byte access, else 16 bytes over row phase classes:
    # row r of contiguous rows starts at phase r * N mod 8 (bf16), so N % 8 = 4, 2 or odd gives
    # 2, 4 or 8 classes (fp32: N % 4 = 2 or odd gives 2 or 4)
    assert [width(BF, N) for N in (4096, 4100, 4098, 4097)] == [16, 16, 16, 16]
    assert [nl.norm_plan(0, BF, 0, 64, N)["phase_classes"] for N in (4096, 4100, 4098, 4097)] \
        == [0, 2, 4, 8]
    assert [width(F, N) for N in (4096, 4098, 4097)] == [16, 16, 16]
    assert [nl.norm_plan(0, F, 0, 64, N)["phase_classes"] for N in (4096, 4098, 4097)] \
        == [0, 2, 4]
    for dt, N, classes in ((BF, 4097, 8), (BF, 4103, 8), (F, 4093, 4), (F, 1027, 4),
                           (BF, 1001, 8), (BF, 9, 8), (F, 5, 4)):
        p = nl.norm_plan(0, dt, 1, 64, N)
        assert p["phase_classes"] == classes and p["elems_per_access"] == (8 if dt == BF else 4)
        assert p["grid"] % classes == 0
    assert nl.norm_plan(0, BF, 1, 64, 4096)["phase_classes"] == 0
    # pointers whose phase is unknown (align below 16), and rows shorter than one 16-byte
    # access: the widest aligned access, element-wise for odd rows
    assert width(BF, 4097, 8) == 2 and width(F, 4097, 8) == 4 and width(BF, 4100, 8) == 8
    assert width(BF, 7) == 2 and width(F, 3) == 4
    try:
        # without phase classes: 8 bytes (N % 4 == 0), 4 (N even) or one element
        nl.norm_set_tuning(nl.TUNE_UNALIGNED, 0)
        assert [width(BF, N) for N in (4100, 4098, 4097)] == [8, 4, 2]
        assert [width(F, N) for N in (4098, 4097)] == [8, 4]
        # fp32 weights beside bf16 activations: 4 bf16 need 16-byte weight loads, 2 need 8
        assert [width(BF32W, N) for N in (4096, 4100, 4098)] == [16, 8, 4]
        assert [width(BF32W, 4100, a) for a in (16, 8, 4)] == [8, 4, 2]
        nl.norm_set_tuning(nl.TUNE_UNALIGNED, 1)     # the same as the default
        assert [width(BF, N) for N in (4100, 4098, 4097)] == [16, 16, 16]
    finally:
        nl.norm_set_tuning(nl.TUNE_UNALIGNED, -1)
    # the pointers' common alignment caps the width
    assert [width(BF, 4096, a) for a in (16, 8, 4, 2, 1, 0)] == [16, 8, 4, 2, 2, 2]
    assert [width(F, 4096, a) for a in (16, 8, 4)] == [16, 8, 4]
    # fp32 weights: the phase classes gather them at any alignment
    assert [width(BF32W, N) for N in (4096, 4100, 4098)] == [16, 16, 16]
    assert [width(BF32W, 4100, a) for a in (16, 8, 4)] == [16, 4, 2]
    # the narrow paths size their teams like the 16-byte path: same scheme, same threads
    for pass_ in (0, 1):
        full = nl.norm_plan(0, BF, pass_, 16384, 4096)
        for N in (4100, 4098):
            narrow = nl.norm_plan(0, BF, pass_, 16384, N)
            assert narrow["scheme"] == full["scheme"] == nl.SCHEME_BLOCK
            assert narrow["team_threads"] * narrow["accesses_per_thread"] * \
                narrow["elems_per_access"] >= N


@pytest.mark.parametrize("dt", [BF, F])
@pytest.mark.parametrize("N", [1, 7, 64, 1000, 1024, 1025, 2048, 4096, 5120, 7168, 8192, 16384,
                               65535, 262144, 4194304])
@pytest.mark.parametrize("M", [1, 3, 4, 256, 16384, 65536])
@pytest.mark.parametrize("pass_", [0, 1])
def test_plan_covers_every_row_and_column(dt, N, M, pass_):
    for align in (16, 8, 4, 2, 1):
        p = nl.norm_plan(0, dt, pass_, M, N, align=align)
        epv = p["elems_per_access"]
        P = p["phase_classes"]
        if P:
            # 16-byte accesses over row phase classes (contiguous rows of N elements from a
            # 16-byte aligned start: row r at phase r * N mod epv), a team scheme
            assert align == 16 and p["access_bytes"] == 16 and N % epv and N >= epv
            assert p["scheme"] in (nl.SCHEME_WAVE, nl.SCHEME_BLOCK)
            assert P == epv // math.gcd(N % epv, epv) and p["grid"] % P == 0
            nacc = max(-(-(N + (c * N) % epv) // epv) for c in range(P))
        else:
            assert N % epv == 0 and p["access_bytes"] <= max(align, 4 if dt == F else 2)
            nacc = N // epv
        assert p["threads"] % 64 == 0 and 64 <= p["threads"] <= 1024
        assert p["grid"] >= 1
        if p["scheme"] == nl.SCHEME_SPLIT:
            assert p["chunks"] * p["chunk_elems"] >= N
            assert (p["chunks"] - 1) * p["chunk_elems"] < N
            if pass_ == 1:
                assert p["grid"] == p["chunks"] * p["row_groups"]
                assert p["partials"] == max(p["row_groups"], p["exchange_row_groups"])
                assert p["partials"] <= M
        else:
            # a team's registers cover the whole row
            assert p["team_threads"] * p["accesses_per_thread"] >= nacc
            if pass_ == 1:
                assert p["partials"] == p["grid"]
        if pass_ == 1:
            assert p["workspace_bytes"] >= 256 + 2 * p["partials"] * N * 4


def test_plan_tuning_overrides():
    try:
        nl.norm_set_tuning(nl.TUNE_SCHEME, nl.SCHEME_SPLIT)
        assert nl.norm_plan(0, BF, 0, 64, 512)["scheme"] == nl.SCHEME_SPLIT
        nl.norm_set_tuning(nl.TUNE_SCHEME, nl.SCHEME_BLOCK)
        assert nl.norm_plan(0, BF, 0, 64, 512)["scheme"] == nl.SCHEME_BLOCK
        nl.norm_set_tuning(nl.TUNE_SCHEME, nl.SCHEME_WAVE)
        with pytest.raises(nl.NormError):
            nl.norm_plan(0, BF, 0, 64, 65536)      # a wavefront cannot hold this row
        nl.norm_set_tuning(nl.TUNE_SCHEME, -1)
        nl.norm_set_tuning(nl.TUNE_GRID_PER_CU, 1)
        assert nl.norm_plan(0, BF, 1, 65536, 4096, cu_count=256)["partials"] == 256
        nl.norm_set_tuning(nl.TUNE_ROWS_PER_ITER, 2)
        assert nl.norm_plan(0, BF, 0, 65536, 512)["rows_per_iter"] == 2
        assert nl.norm_plan(0, BF, 0, 65536, 4096)["row_order"] == 0
        nl.norm_set_tuning(nl.TUNE_ROW_ORDER, 1)
        assert nl.norm_plan(0, BF, 0, 65536, 4096)["row_order"] == 1
        assert nl.norm_plan(0, BF, 1, 65536, 512)["row_order"] == 1
    finally:
        for k in range(nl.N_TUNE_KEYS):
            nl.norm_set_tuning(k, -1)


def test_split_exchange_partial_limit():
    """By default the single-pass split form needs a row to gather at most 512 chunk partials
    forward and 640 backward: LayerNorm (three per chunk) keeps it up to 170 / 213 chunks of
    8192, RMSNorm (one) up to the form's 512."""
    try:
        for kind, nq in ((0, 3), (1, 1)):
            for pass_, limit in ((0, 512), (1, 640)):
                for C in (64, 128, 170, 171, 192, 213, 214, 256, 512):
                    M = 4 if C > 256 else 8
                    p = nl.norm_plan(kind, BF, pass_, M, 8192 * C, cu_count=256)
                    assert (p["exchange_row_groups"] > 0) == (C * nq <= limit), (kind, pass_, C)
                    nl.norm_set_tuning(nl.TUNE_SPLIT_EXCHANGE, 1)
                    assert nl.norm_plan(kind, BF, pass_, M, 8192 * C,
                                        cu_count=256)["exchange_row_groups"] > 0
                    nl.norm_set_tuning(nl.TUNE_SPLIT_EXCHANGE, -1)
    finally:
        nl.norm_set_tuning(nl.TUNE_SPLIT_EXCHANGE, -1)


def test_split_exchange_plan():
    """The single-pass split form: 16-byte accesses, the default chunk, no residual input, at
    most 512 chunks, and a grid (row groups x chunks) the device keeps resident: 4 workgroups
    per CU forward (3 with fp32 weights beside 16-bit activations), with room for two row
    groups, and 2 backward."""
    cu = 256
    try:
        mixed = nl.norm_plan(0, nl.BF16_F32W, 0, 256, 262144, cu_count=cu)
        assert mixed["exchange_row_groups"] == min(256, cu * 3 // 32)
        for kind, pass_, per_cu in ((0, 0, 4), (1, 0, 4), (0, 1, 2), (1, 1, 2)):
            for M, N in ((256, 262144), (4, 4194304), (3, 20000), (1000, 65536)):
                # more chunks than the device holds at once (forward: twice over)
                if N // 8192 * (2 if pass_ == 0 else 1) > cu * per_cu:
                    assert nl.norm_plan(kind, BF, pass_, M, N,
                                        cu_count=cu)["exchange_row_groups"] == 0
                    continue
                # by default a row gathers at most 512 chunk partials forward and 640
                # backward (LayerNorm three per chunk, RMSNorm one); the knob at 1 lifts that
                partials = -(-N // 8192) * (3 if kind == 0 else 1)
                if partials > (512 if pass_ == 0 else 640):
                    assert nl.norm_plan(kind, BF, pass_, M, N,
                                        cu_count=cu)["exchange_row_groups"] == 0
                    nl.norm_set_tuning(nl.TUNE_SPLIT_EXCHANGE, 1)
                p = nl.norm_plan(kind, BF, pass_, M, N, cu_count=cu)
                nl.norm_set_tuning(nl.TUNE_SPLIT_EXCHANGE, -1)
                assert p["scheme"] == nl.SCHEME_SPLIT and p["chunk_elems"] == 8192
                G = p["exchange_row_groups"]
                assert G == min(M, cu * per_cu // p["chunks"]) >= 1
                assert G * p["chunks"] <= cu * per_cu
                if pass_ == 1:
                    assert p["partials"] >= G
            # residual input, narrower accesses, the statistics pass, or a tuned chunk: two passes
            assert nl.norm_plan(1, BF, pass_, 64, 262144, residual=1,
                                cu_count=cu)["exchange_row_groups"] == 0
            assert nl.norm_plan(0, BF, pass_, 64, 262148, cu_count=cu)["exchange_row_groups"] == 0
            nl.norm_set_tuning(nl.TUNE_SPLIT_CHUNK, 4096)
            assert nl.norm_plan(0, BF, pass_, 64, 262144, cu_count=cu)["exchange_row_groups"] == 0
            nl.norm_set_tuning(nl.TUNE_SPLIT_CHUNK, -1)
            nl.norm_set_tuning(nl.TUNE_SPLIT_EXCHANGE, 0)
            assert nl.norm_plan(0, BF, pass_, 64, 262144, cu_count=cu)["exchange_row_groups"] == 0
            nl.norm_set_tuning(nl.TUNE_SPLIT_EXCHANGE, -1)
        # the statistics pass shares the forward's plan and workspace (it runs two passes)
        assert (nl.norm_plan(0, BF, 2, 64, 262144, cu_count=cu)["workspace_bytes"] ==
                nl.norm_plan(0, BF, 0, 64, 262144, cu_count=cu)["workspace_bytes"])
        # more chunks than 512, or than the device holds at once
        assert nl.norm_plan(0, BF, 0, 2, 8192 * 513, cu_count=cu)["exchange_row_groups"] == 0
        assert nl.norm_plan(0, BF, 1, 4, 4194304, cu_count=128)["exchange_row_groups"] == 0
        # the backward's row-group knob lowers its row groups
        nl.norm_set_tuning(nl.TUNE_ROW_GROUPS, 5)
        assert nl.norm_plan(0, BF, 1, 256, 262144, cu_count=cu)["exchange_row_groups"] == 5
        assert nl.lib().norm_set_tuning(nl.TUNE_SPLIT_EXCHANGE, 2) == nl.ERR_INVALID_ARG
        for bad in (0, (1 << 24) + 1):
            assert nl.lib().norm_set_tuning(nl.TUNE_EXCHANGE_POLLS, bad) == nl.ERR_INVALID_ARG
        assert nl.lib().norm_set_tuning(nl.TUNE_EXCHANGE_POLLS, 1) == nl.OK
        assert nl.lib().norm_set_tuning(nl.TUNE_EXCHANGE_WITHHOLD, 2) == nl.ERR_INVALID_ARG
    finally:
        for k in range(nl.N_TUNE_KEYS):
            nl.norm_set_tuning(k, -1)


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("pass_", [0, 1, 2])
@pytest.mark.parametrize("M,N", [(1, 1), (3, 1000), (2048, 1024), (16384, 4096), (16384, 4100),
                                 (32768, 8192), (65536, 7168), (16384, 16384), (256, 262144),
                                 (4, 4194304), (2, 8192 * 513), (1000, 65536), (16384, 10240),
                                 (16384, 12288), (16384, 2049), (16384, 4100 * 2 + 1)])
def test_workspace_bytes_on_the_host(kind, pass_, M, N):
    """norm_workspace_bytes needs no device and covers the plan of every compute-unit count
    (1 .. 256) and every pointer alignment."""
    for dt in (BF, F, nl.BF16_F32W):
        for res in ((0, 1) if (kind == 1 and pass_ != 1) else (0,)):
            code = nl.dtype_code(dt) if isinstance(dt, torch.dtype) else dt
            b = nl.lib().norm_workspace_bytes(kind, pass_, M, N, code, res)
            assert b == nl.norm_workspace_bytes(kind, pass_, M, N, dt, bool(res))
            assert b != nl.SIZE_MAX
            most = 0
            for cu in (1, 2, 3, 7, 32, 64, 80, 128, 200, 255, 256):
                for align in (16, 8, 4, 2, 1):
                    p = nl.norm_plan(kind, dt, pass_, M, N, residual=bool(res), align=align,
                                     cu_count=cu)
                    most = max(most, p["workspace_bytes"])
            assert b >= most
            # a workspace is either none at all or starts with the 256-byte header
            assert b == 0 or b >= 256
            if pass_ == 1:
                assert b >= 256 + 2 * N * 4
            assert b % 256 == 0


def test_workspace_bytes_rejects():
    L = nl.lib()
    B16 = nl.BF16
    for args in ((0, 0, -1, 16, B16, 0), (0, 0, 4, 0, B16, 0), (0, 0, 4, -5, B16, 0),
                 (7, 0, 4, 16, B16, 0), (0, 7, 4, 16, B16, 0), (0, 0, 4, 16, 9, 0),
                 (0, 1, 4, 1 << 31, B16, 0)):
        assert L.norm_workspace_bytes(*args) == nl.SIZE_MAX, args
    # M == 0 is a valid (empty) call
    assert L.norm_workspace_bytes(0, 1, 0, 4096, B16, 0) != nl.SIZE_MAX


def test_workspace_status_host_checks():
    """Arguments the status query rejects (or answers) without touching a device."""
    L = nl.lib()
    assert L.norm_workspace_status(None, 0, None) == nl.OK      # no workspace: nothing waited
    assert L.norm_workspace_status(None, 255, None) == nl.OK
    assert L.norm_workspace_status(None, 256, None) == nl.ERR_WORKSPACE
    assert L.norm_workspace_status(FAKE + 4, 4096, None) == nl.ERR_WORKSPACE  # unaligned


def test_workspace_needs_a_device_here():
    with pytest.raises(nl.NormError) as e:
        nl.norm_workspace_size(0, BF, 1, 16, 4096)
    assert e.value.status == nl.ERR_HIP


def test_launch_events_arm_and_disarm():
    lib = nl.lib()
    assert lib.norm_set_launch_events(None, None) == nl.OK
    assert lib.norm_set_launch_events(FAKE, None) == nl.ERR_INVALID_ARG
    assert lib.norm_set_launch_events(None, FAKE) == nl.ERR_INVALID_ARG
    # armed with handles that are never used: the call fails its checks and disarms them
    assert lib.norm_set_launch_events(FAKE, FAKE * 2) == nl.OK
    assert _fwd(kind=9) == nl.ERR_INVALID_ARG
    assert lib.norm_set_launch_events(None, None) == nl.OK


def test_mixed_weight_dtype_on_the_host():
    # bf16 activations with fp32 weights plan like bf16 and size spans with 4-byte weights
    for pass_ in (0, 1):
        a = nl.norm_plan(0, nl.BF16_F32W, pass_, 4096, 4096)
        b = nl.norm_plan(0, BF, pass_, 4096, 4096)
        assert a == b
    assert nl.lib().norm_set_tuning(nl.TUNE_SCHEME, -1) == nl.OK
    with pytest.raises(nl.NormError):
        nl.norm_plan(0, 5, 0, 16, 16)                      # no such dtype
    # W holds N fp32 values: an output placed inside them overlaps
    assert _fwd(dtype=2, W=FAKE * 2, Y=FAKE * 2 + 16) == nl.ERR_INVALID_ARG
    assert _fwd(dtype=2, W=FAKE * 2, mean=FAKE * 2 + 16, M=4, N=8) == nl.ERR_INVALID_ARG
    # with bf16 weights the same output starts after W's 16 bytes: accepted (then no device)
    assert _fwd(dtype=1, W=FAKE * 2, mean=FAKE * 2 + 16, M=4, N=8) == nl.ERR_HIP
    assert nl.dtype_code(torch.bfloat16, torch.float32) == nl.BF16_F32W
    with pytest.raises(ValueError):
        nl.dtype_code(torch.float32, torch.bfloat16)


def test_fp16_dtypes_on_the_host():
    # fp16 plans like bf16 (two-byte elements); fp16 activations with fp32 weights like the
    # bf16 mixed layout, and their weight spans are 4 bytes per element
    HF = torch.float16
    for pass_ in (0, 1):
        for N in (1000, 4096, 4100, 4098, 12288, 262144):
            assert nl.norm_plan(0, HF, pass_, 4096, N) == nl.norm_plan(0, BF, pass_, 4096, N)
            assert nl.norm_plan(0, nl.F16_F32W, pass_, 4096, N) == \
                nl.norm_plan(0, nl.BF16_F32W, pass_, 4096, N)
    assert nl.dtype_code(HF) == nl.F16 == 3
    assert nl.dtype_code(HF, torch.float32) == nl.F16_F32W == 4
    with pytest.raises(ValueError):
        nl.dtype_code(HF, torch.bfloat16)
    assert _fwd(dtype=4, W=FAKE * 2, Y=FAKE * 2 + 16) == nl.ERR_INVALID_ARG
    assert _fwd(dtype=3, W=FAKE * 2, mean=FAKE * 2 + 16, M=4, N=8) == nl.ERR_HIP


# ---- the norm deferred into a projection: argument checks --------------------------------

def _fold(**kw):
    a = dict(kind=0, dtype=1, L=FAKE, ldl=64, gamma=FAKE * 2, beta=FAKE * 3, c=None, Nout=32,
             K=64, G=FAKE * 4, ldg=64, s=FAKE * 5, t=FAKE * 6, stream=None)
    a.update(kw)
    return nl.lib().norm_fold_projection(*a.values())


def _lazy(**kw):
    a = dict(kind=0, X=FAKE, ldx=64, M=16, K=64, eps=1e-5, G=FAKE * 2, ldg=64, Nout=32,
             s=FAKE * 3, t=FAKE * 4, mean_in=None, rstd_in=None, mean_out=None, rstd_out=None,
             Y=FAKE * 5, ldy=32, stream=None)
    a.update(kw)
    return nl.lib().norm_lazy_linear(*a.values())


def test_fold_projection_checks():
    assert _fold() == nl.ERR_HIP                           # valid: reaches the launch
    assert _fold(dtype=2, kind=1, beta=None, s=None, t=None) == nl.ERR_HIP
    for kw in (dict(dtype=0), dict(dtype=3), dict(kind=2), dict(L=None), dict(G=None),
               dict(gamma=None), dict(Nout=0), dict(K=0), dict(ldl=63), dict(ldg=8),
               dict(s=None),                               # LayerNorm needs s
               dict(t=None),                               # beta given: t needed
               dict(kind=1, s=None),                       # RMSNorm has no beta
               dict(G=FAKE + 64),                          # G over L
               dict(s=FAKE * 2),                           # s over gamma
               dict(t=FAKE * 5 + 4),                       # t over s
               dict(L=FAKE + 1)):                          # misaligned bf16
        assert _fold(**kw) == nl.ERR_INVALID_ARG, kw


# fake operands far apart, for strides whose spans would overlap the packed fakes above
FAR = dict(X=1 << 40, G=2 << 40, s=3 << 40, t=4 << 40, Y=5 << 40)


def test_lazy_linear_checks():
    assert _lazy() == nl.ERR_HIP                           # statistics formed in the product
    assert _lazy(mean_out=FAKE * 6, rstd_out=FAKE * 7) == nl.ERR_HIP
    assert _lazy(mean_in=FAKE * 6, rstd_in=FAKE * 7) == nl.ERR_HIP
    assert _lazy(kind=1, s=None, t=None, rstd_in=FAKE * 7) == nl.ERR_HIP
    assert _lazy(M=0) == nl.OK                             # nothing to launch
    assert _lazy(M=0, X=None, Y=None) == nl.OK
    assert _lazy(M=0, K=0) == nl.ERR_INVALID_ARG
    for kw in (dict(kind=2), dict(X=None), dict(G=None), dict(Y=None), dict(M=-1), dict(K=0),
               dict(Nout=0), dict(eps=-1.0), dict(eps=float("nan")), dict(ldx=32),
               dict(ldy=16), dict(s=None),
               dict(rstd_in=FAKE * 7),                     # LayerNorm: mean_in too
               dict(mean_in=FAKE * 6),                     # mean without rstd
               dict(mean_in=FAKE * 6, rstd_in=FAKE * 7, rstd_out=FAKE * 8),
               dict(kind=1, mean_out=FAKE * 6),            # RMSNorm has no mean
               dict(kind=1, rstd_in=FAKE * 7, mean_in=FAKE * 6),
               dict(Y=FAKE + 64),                          # Y over X
               dict(rstd_out=FAKE * 5),                    # statistics over Y
               dict(Y=FAKE * 5 + 1)):                      # misaligned bf16
        assert _lazy(**kw) == nl.ERR_INVALID_ARG, kw
    for kw in (dict(K=60, ldx=64, ldg=64),                 # K not a multiple of 8
               dict(ldx=68), dict(ldg=72 + 4),             # row strides not multiples of 8
               dict(X=FAKE + 8), dict(G=FAKE * 2 + 2),     # not 16-byte aligned
               dict(FAR, M=2, ldx=1 << 23),                # tile rows past 32-bit offsets
               dict(FAR, Nout=2, ldg=1 << 23, ldy=32)):
        assert _lazy(**kw) == nl.ERR_UNSUPPORTED, kw
    assert _lazy(**dict(FAR, M=2, ldx=(1 << 23) - 8)) == nl.ERR_HIP


# ---- attention over normalised queries and keys: argument checks ------------------------------

def _attn(**kw):
    # B=2, S=300, Hq=4, Hk=2, D=128 over one packed QKV buffer: token stride (4 + 2 + 2) * 128
    ld = 8 * 128
    a = dict(kind=1, flags=0, B=2, S=300, Hq=4, Hk=2, D=128, Q=FAKE, ldq=ld, K=FAKE + 1024,
             ldk=ld, V=FAKE + 1536, ldv=ld, wq=FAKE * 2, bq=None, wk=FAKE * 2 + 256, bk=None,
             eps=1e-6, scale=128 ** -0.5, O=FAKE * 3, ldo=512, lse=FAKE * 4, workspace=None,
             workspace_bytes=0, stream=None)
    a.update(kw)
    return nl.lib().norm_attention_fwd(*a.values())


def test_attention_checks():
    assert _attn() == nl.ERR_HIP                           # valid: reaches the launch
    assert _attn(kind=0, bq=FAKE * 2 + 512, bk=FAKE * 2 + 768) == nl.ERR_HIP
    assert _attn(kind=0) == nl.ERR_HIP                     # LayerNorm without betas
    assert _attn(flags=3, wq=None, wk=None) == nl.ERR_HIP  # causal, no norm
    assert _attn(lse=None) == nl.ERR_HIP
    assert _attn(Hk=4, ldq=1536, ldk=1536, ldv=1536) == nl.ERR_HIP
    assert _attn(B=0) == nl.OK and _attn(S=0, Q=None, O=None) == nl.OK
    ws = nl.attention_workspace_bytes(2, 300, 2, 128)
    assert ws == 2 * 300 * 2 * 128 * 2
    assert _attn(workspace=FAKE * 5, workspace_bytes=ws) == nl.ERR_HIP
    assert _attn(workspace=FAKE * 5, workspace_bytes=16) == nl.ERR_HIP   # too small: not used
    assert nl.attention_workspace_bytes(0, 300, 2, 128) == 0
    assert nl.attention_workspace_bytes(1 << 31, 1 << 31, 2, 128) == 0
    for kw in (dict(kind=2), dict(flags=4), dict(Hk=3), dict(Hq=0), dict(D=0), dict(B=-1),
               dict(Q=None), dict(K=None), dict(V=None), dict(O=None), dict(wq=None),
               dict(wk=None), dict(bq=FAKE * 2 + 512),    # RMSNorm has no beta
               dict(flags=2),                             # no norm, but gammas given
               dict(eps=-1.0), dict(eps=float("inf")), dict(scale=0.0), dict(scale=-0.1),
               dict(scale=float("nan")),
               dict(ldq=511), dict(ldk=255), dict(ldo=256),  # strides below the heads
               dict(O=FAKE + 64),                         # O over Q
               dict(lse=FAKE * 3 + 8),                    # lse over O
               dict(lse=FAKE * 4 + 2),                    # misaligned lse
               dict(workspace=FAKE * 5),                  # workspace without its size
               dict(workspace_bytes=64),                  # a size without a workspace
               dict(workspace=FAKE * 3 + 256, workspace_bytes=1024)):  # workspace over O
        assert _attn(**kw) == nl.ERR_INVALID_ARG, kw
    for kw in (dict(D=64, ldq=512, ldk=512, ldv=512, ldo=256),   # head size
               dict(ldq=8 * 128 + 4), dict(ldo=516),            # strides not multiples of 8
               dict(Q=FAKE + 8), dict(wk=FAKE * 2 + 264),       # not 16-byte aligned
               dict(workspace=FAKE * 5 + 8, workspace_bytes=1024),
               dict(B=1 << 16, S=1 << 16, Hq=128, Hk=1,          # grid past 2^31 - 1
                    Q=1 << 48, ldq=1 << 14, K=2 << 48, ldk=128, V=3 << 48, ldv=128,
                    O=4 << 48, ldo=1 << 14, lse=5 << 48)):
        assert _attn(**kw) == nl.ERR_UNSUPPORTED, kw
