"""Rows off 16-byte boundaries against the CPU oracle, through the C ABI (needs a gfx950 GPU).

A row whose length is not a multiple of the 16-byte access (an odd N in bf16 or fp16, N % 4 != 0
in fp32), or whose start is not 16-byte aligned (odd row strides, shifted pointers), keeps
aligned 16-byte accesses in the wave and block schemes when all its [M, N] tensors share one
phase: rows fall into phase classes, each workgroup takes the rows of one class, and a row's
first and last accesses are partial. Covers: odd row lengths across the wave and block schemes
and their boundaries, every storage type, the residual variant with dR and dH, the backward
recomputing its statistics, the tuning knobs (rows per team, teams per workgroup, grid, forced
schemes), classes with no row at all (M below the class count), row strides and pointer shifts
(shared phases, and mixed ones that fall back to narrower accesses), the same path in place of
8- and 4-byte accesses, and guard bands around every buffer.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from deep_learning_normalization_amd import inputs, normlib as nl
from tests.parity import check_colsums, check_values, run_and_check, tuned

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[gpu] " + msg, flush=True)


def _small(kind, dtype, M, N, seed=0, wdtype=None, **kw):
    base = dict(x=inputs.normal(0.3, 1.5), w=inputs.normal(1, 0.1), dy=inputs.normal(0, 1),
                b=inputs.normal(0, 0.1) if kind == "layernorm" else None)
    base.update(kw)
    eps = 1e-5 if kind == "layernorm" else 1e-6
    w = inputs.Workload("%s_%s_%dx%d" % (kind, dtype, M, N), kind, dtype, M, N, eps, seed=seed,
                        **base)
    return dataclasses.replace(w, wdtype=wdtype) if wdtype else w


def _code(dt, wdt):
    return nl.BF16_F32W if (wdt == "f32" and dt == "bf16") else \
        nl.F16_F32W if (wdt == "f32" and dt == "f16") else inputs.TORCH_DTYPES[dt]


def _plan(kind, dt, wdt, pass_, M, N, residual=False):
    return nl.norm_plan(kind, _code(dt, wdt), pass_, M, N, residual)


def _classes(N, epv):
    """Row phase classes of contiguous rows of N elements from an aligned start, and the most
    accesses any class's rows need."""
    P = epv // math.gcd(N % epv, epv)
    return P, max(-(-(N + (c * N) % epv) // epv) for c in range(P))


# Odd row lengths: the wave scheme (up to 1024), the block scheme, the backward's block limit
# (8185 bf16: at most 1024 accesses in every class; 8187 goes element-wise to the split scheme)
# and the forward's (16377 bf16), rows shorter than one access.
ODD_N = [1, 3, 7, 9, 15, 63, 127, 1001, 1023, 1025, 2047, 2049, 4097, 4103, 5121, 8185, 8187,
         12289, 16377, 16383]
TYPES = [("bf16", None), ("bf16", "f32"), ("f16", None), ("f32", None)]


def _odd_cases():
    out = []
    for N in ODD_N:
        for kind in ("layernorm", "rmsnorm"):
            for dt, wdt in TYPES:
                out.append((kind, dt, wdt, 129 if N <= 4103 else 41, N))
    return out


@pytest.mark.parametrize("kind,dt,wdt,M,N", _odd_cases(), ids=lambda v: str(v))
def test_odd_rows(kind, dt, wdt, M, N):
    epv = 4 if dt == "f32" else 8
    P, nal = _classes(N, epv)
    for pass_, limit in ((nl.PASS_FWD, 2048), (nl.PASS_BWD, 1024)):
        p = _plan(kind, dt, wdt, pass_, M, N)
        # (the wave scheme takes rows up to 1024; its backward with phase classes up to 256
        # accesses)
        wave_limit = 256 if pass_ == nl.PASS_BWD else 512
        expect = N % epv != 0 and N >= epv and nal <= (wave_limit if N <= 1024 else limit)
        assert p["phase_classes"] == (P if expect else 0), (pass_, p)
        if expect:
            assert p["access_bytes"] == 16 and p["grid"] % P == 0
            assert p["scheme"] in (nl.SCHEME_WAVE, nl.SCHEME_BLOCK)
    _say("odd rows %s %s w=%s %dx%d" % (kind, dt, wdt, M, N))
    w = _small(kind, dt, M, N, seed=M + N, wdtype=wdt)
    run_and_check(w)


@pytest.mark.parametrize("N", [1001, 4097, 7169])
@pytest.mark.parametrize("kind", ["rmsnorm", "layernorm"])
def test_odd_rows_residual(kind, N):
    assert _plan(kind, "bf16", None, nl.PASS_FWD, 65, N, residual=True)["phase_classes"] == 8
    _say("odd rows residual %s N=%d" % (kind, N))
    w = _small(kind, "bf16", 65, N, seed=N, x=inputs.normal(0, 0.5), r=inputs.normal(0, 1))
    run_and_check(w, dr="alias", dh=True)
    run_and_check(dataclasses.replace(w, seed=N + 1), dr="separate")
    run_and_check(dataclasses.replace(w, seed=N + 2), dr="separate", dh=True)


@pytest.mark.parametrize("N", [63, 1001, 4097])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("kind", ["layernorm", "rmsnorm"])
def test_odd_rows_recomputed_statistics(kind, dt, N):
    """The backward without saved statistics forms them again from the partial last access."""
    _say("odd rows, backward recomputing statistics, %s %s N=%d" % (kind, dt, N))
    w = _small(kind, dt, 77, N, seed=N + 5, x=inputs.normal(40.0, 0.5))
    run_and_check(w, stats=False)


KNOBS = [dict(rows=2), dict(rows=4), dict(grid_per_cu=1), dict(teams=4), dict(teams=2),
         dict(row_order=1), dict(team_threads=1024), dict(scheme=nl.SCHEME_BLOCK),
         dict(scheme=nl.SCHEME_WAVE)]


@pytest.mark.parametrize("knob", KNOBS, ids=lambda k: ",".join("%s=%s" % i for i in k.items()))
@pytest.mark.parametrize("kind,dt,M,N", [("layernorm", "bf16", 300, 2047),
                                         ("rmsnorm", "bf16", 300, 1001),
                                         ("layernorm", "f32", 300, 1021),
                                         ("rmsnorm", "f16", 131, 4095)], ids=lambda v: str(v))
def test_odd_rows_tuning_knobs(knob, kind, dt, M, N):
    P, nal = _classes(N, 4 if dt == "f32" else 8)
    with tuned(**knob):
        if knob.get("scheme") == nl.SCHEME_WAVE and nal > 256:
            # the wave backward takes phase classes up to 4 accesses per thread (256 per row);
            # element-wise, a wavefront holds 1024 elements: no wave plan for this row
            with pytest.raises(nl.NormError):
                _plan(kind, dt, None, nl.PASS_BWD, M, N)
            return
        p = _plan(kind, dt, None, nl.PASS_BWD, M, N)
        assert p["phase_classes"] == P
        _say("odd rows %s %s %dx%d knob %s: scheme %d, %d threads, %d rows" % (
            kind, dt, M, N, knob, p["scheme"], p["threads"], p["rows_per_iter"]))
        run_and_check(_small(kind, dt, M, N, seed=M + N + 3))


@pytest.mark.parametrize("N", [1002, 1004, 4098, 4100, 7170, 8196])
@pytest.mark.parametrize("kind,dt,wdt", [("layernorm", "bf16", None), ("rmsnorm", "bf16", "f32"),
                                         ("layernorm", "f32", None)], ids=lambda v: str(v))
def test_in_place_of_narrow_accesses(kind, dt, wdt, N):
    """NORM_TUNE_UNALIGNED = 1: 16-byte accesses from each row's start also where 8- or 4-byte
    ones would be aligned."""
    if dt == "f32" and N % 4 == 0:
        pytest.skip("16-byte aligned")
    with tuned(unaligned=1):
        epv = 4 if dt == "f32" else 8
        P, nal = _classes(N, epv)
        for pass_, limit in ((nl.PASS_FWD, 2048), (nl.PASS_BWD, 1024)):
            p = _plan(kind, dt, wdt, pass_, 97, N)
            wave_limit = 256 if pass_ == nl.PASS_BWD else 512
            assert p["phase_classes"] == (P if nal <= (wave_limit if N <= 1024 else limit) else 0)
        _say("unaligned in place of narrow %s %s w=%s N=%d" % (kind, dt, wdt, N))
        run_and_check(_small(kind, dt, 97, N, seed=N, wdtype=wdt))
        w = _small(kind, dt, 33, N, seed=N + 9, wdtype=wdt, x=inputs.normal(0, 0.5),
                   r=inputs.normal(0, 1))
        if dt == "bf16" and wdt is None:
            run_and_check(w, dr="separate", dh=True)


def _strided_like(src, ld, col0, fill):
    M, N = src.shape
    buf = torch.full((M, ld), fill, dtype=src.dtype, device="cuda")
    v = buf[:, col0:col0 + N]
    v.copy_(src.to("cuda"))
    return buf, v


# (kind, N, input stride, input column offset, output stride): whole 16-byte accesses at rows
# that start 2, 4 or 6 bytes past a 16-byte boundary (odd strides), and odd rows in odd strides
STRIDED = [("layernorm", 4096, 4097, 0, 4099), ("rmsnorm", 2048, 6145, 1, 2051),
           ("layernorm", 1024, 1025, 1, 1027), ("rmsnorm", 4097, 4097, 0, 4099),
           ("layernorm", 1001, 3003, 1001, 1003)]


@pytest.mark.parametrize("kind,N,ldi,col0,ldo", STRIDED, ids=lambda v: str(v))
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_odd_row_strides(kind, N, ldi, col0, ldo, dt):
    """Row-strided views with odd strides: the results match the oracle, and the columns
    between the rows of every output keep their fill (a partial access writes nothing past the
    row's end)."""
    M = 37
    w = _small(kind, dt, M, N, seed=N + ldi)
    t = inputs.make(w)
    sentinel = -7.0
    _, X = _strided_like(t["X"], ldi, col0, 0.0)
    _, dY = _strided_like(t["dY"], ldi, col0, 0.0)
    W = t["W"].cuda()
    B = t["B"].cuda() if t["B"] is not None else None
    ybuf, Y = _strided_like(torch.zeros(M, N, dtype=X.dtype), ldo, ldo - N, sentinel)
    xbuf, dX = _strided_like(torch.zeros(M, N, dtype=X.dtype), ldo, 0, sentinel)
    mean = torch.empty(M, dtype=torch.float32, device="cuda") if kind == "layernorm" else None
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    _say("odd strides %s %s N=%d in ld %d (+%d) out ld %d" % (kind, dt, N, ldi, col0, ldo))
    nl.norm_fwd(kind, X, None, W, B, w.eps, Y, None, mean, rstd,
                nl.workspace(kind, X.dtype, nl.PASS_FWD, M, N))
    dW = torch.empty_like(W)
    dB = torch.empty_like(W) if kind == "layernorm" else None
    nl.norm_bwd(kind, X, dY, None, W, mean, rstd, w.eps, dX, None, dW, dB,
                nl.workspace(kind, X.dtype, nl.PASS_BWD, M, N))
    torch.cuda.synchronize()
    bits = {k: inputs.host_bits(t[k]) for k in ("X", "W", "B", "dY")}
    code = oracle.F32 if dt == "f32" else oracle.BF16
    k = oracle.LAYERNORM if kind == "layernorm" else oracle.RMSNORM
    eps = float(np.float32(w.eps))
    f = oracle.fwd(k, code, bits["X"], bits["W"], bits["B"], eps=eps)
    g = oracle.bwd(k, code, bits["X"], bits["dY"], bits["W"], eps=eps)
    check_values("Y", Y.double().cpu().numpy(), f["y"], dt)
    check_values("dX", dX.double().cpu().numpy(), g["dx"], dt)
    check_colsums("dW", dW.double().cpu().numpy(), g["dw"], dt)
    if dB is not None:
        check_colsums("dB", dB.double().cpu().numpy(), g["db"], dt)
    for buf, c0 in ((ybuf, ldo - N), (xbuf, 0)):
        gap = torch.ones(ldo, dtype=torch.bool, device="cuda")
        gap[c0:c0 + N] = False
        assert (buf[:, gap] == sentinel).all()


@pytest.mark.parametrize("N", [1000, 4096, 4097, 5120])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_shifted_activations_aligned_weights(dt, N):
    """X, Y, dY and dX one element past a 16-byte boundary, W, B, dW and dB aligned: 16-byte
    accesses at unaligned addresses (whole ones when N is a multiple of the width)."""
    kind = "layernorm"
    M = 61
    w = _small(kind, dt, M, N, seed=N + 1)
    t = inputs.make(w)

    def shifted(src):
        buf = torch.empty(src.numel() + 16, dtype=src.dtype, device="cuda")
        v = buf[1:1 + src.numel()].view(src.shape)
        v.copy_(src.to("cuda"))
        return v

    X, dY = shifted(t["X"]), shifted(t["dY"])
    W, B = t["W"].cuda(), t["B"].cuda()
    Y = shifted(torch.zeros(M, N, dtype=X.dtype))
    dX = shifted(torch.zeros(M, N, dtype=X.dtype))
    mean = torch.empty(M, dtype=torch.float32, device="cuda")
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    _say("shifted activations %s N=%d" % (dt, N))
    nl.norm_fwd(kind, X, None, W, B, w.eps, Y, None, mean, rstd,
                nl.workspace(kind, X.dtype, nl.PASS_FWD, M, N))
    dW, dB = torch.empty_like(W), torch.empty_like(W)
    nl.norm_bwd(kind, X, dY, None, W, mean, rstd, w.eps, dX, None, dW, dB,
                nl.workspace(kind, X.dtype, nl.PASS_BWD, M, N))
    torch.cuda.synchronize()
    bits = {k: inputs.host_bits(t[k]) for k in ("X", "W", "B", "dY")}
    code = oracle.F32 if dt == "f32" else oracle.BF16
    eps = float(np.float32(w.eps))
    f = oracle.fwd(oracle.LAYERNORM, code, bits["X"], bits["W"], bits["B"], eps=eps)
    g = oracle.bwd(oracle.LAYERNORM, code, bits["X"], bits["dY"], bits["W"], eps=eps)
    check_values("Y", Y.double().cpu().numpy(), f["y"], dt)
    check_values("dX", dX.double().cpu().numpy(), g["dx"], dt)
    check_colsums("dW", dW.double().cpu().numpy(), g["dw"], dt)
    check_colsums("dB", dB.double().cpu().numpy(), g["db"], dt)


@pytest.mark.parametrize("scheme", [nl.SCHEME_AUTO, nl.SCHEME_WAVE, nl.SCHEME_BLOCK])
@pytest.mark.parametrize("N", [1001, 2049, 4097])
def test_odd_rows_guard_bands(scheme, N):
    """Every buffer between 4 KiB guard regions filled with a pattern: no partial access writes
    past its buffer."""
    if scheme == nl.SCHEME_WAVE and _classes(N, 8)[1] > 256:
        pytest.skip("no wave backward over phase classes beyond 4 accesses per thread")
    M, G = 300, 4096
    kind = "layernorm"
    dt = torch.bfloat16

    def guarded(n, dtype):
        es = torch.tensor([], dtype=dtype).element_size()
        g = G // es
        buf = torch.full((n + 2 * g,), 0, dtype=dtype, device="cuda")
        buf.view(torch.uint8).fill_(0xA5)
        return buf, buf[g:g + n]

    w = _small(kind, "bf16", M, N, seed=N)
    t = inputs.make(w)
    bufs = []

    def put(src, shape, dtype):
        b, v = guarded(int(np.prod(shape)), dtype)
        bufs.append(b)
        v = v.view(*shape)
        if src is not None:
            v.copy_(src.cuda())
        return v

    X = put(t["X"], (M, N), dt)
    W = put(t["W"], (N,), dt)
    B = put(t["B"], (N,), dt)
    dY = put(t["dY"], (M, N), dt)
    Y, dX = put(None, (M, N), dt), put(None, (M, N), dt)
    dW, dB = put(None, (N,), dt), put(None, (N,), dt)
    mean, rstd = put(None, (M,), torch.float32), put(None, (M,), torch.float32)
    with tuned(scheme=scheme):
        assert nl.norm_plan(kind, dt, nl.PASS_BWD, M, N)["phase_classes"] == 8
        _say("odd rows guard bands scheme %d N=%d" % (scheme, N))
        nfw = nl.norm_workspace_size(kind, dt, nl.PASS_FWD, M, N)
        nbw = nl.norm_workspace_size(kind, dt, nl.PASS_BWD, M, N)
        wsf = put(None, (max(nfw, 16),), torch.uint8)
        wsb = put(None, (max(nbw, 16),), torch.uint8)
        nl.norm_fwd(kind, X, None, W, B, w.eps, Y, None, mean, rstd, wsf)
        nl.norm_bwd(kind, X, dY, None, W, mean, rstd, w.eps, dX, None, dW, dB, wsb)
    torch.cuda.synchronize()
    for b in bufs:
        u = b.view(torch.uint8)
        assert (u[:G] == 0xA5).all() and (u[-G:] == 0xA5).all(), "guard band overwritten"
    bits = {k: inputs.host_bits(t[k]) for k in ("X", "W", "B", "dY")}
    f = oracle.fwd(oracle.LAYERNORM, oracle.BF16, bits["X"], bits["W"], bits["B"],
                   eps=float(np.float32(w.eps)))
    check_values("Y", Y.double().cpu().numpy(), f["y"], "bf16")


def test_odd_full_size_layernorm():
    """LayerNorm bf16 16384 x 4097 (every row compared), forward and backward."""
    w = _small("layernorm", "bf16", 16384, 4097, seed=4097)
    _say("odd full size layernorm 16384x4097")
    out = run_and_check(w)
    assert out["rows_compared"] == 16384
