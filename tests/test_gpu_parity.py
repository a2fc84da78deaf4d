"""HIP library vs the CPU oracle, element by element, through the C ABI (needs a gfx950 GPU).

Covers: every full-size workload in the launch configuration the benchmark uses; a sweep of
row lengths and row counts around every tile and scheme boundary with ragged tails; each scheme
forced outside its natural range; the tuning knobs; the residual variant with dR aliasing and an
incoming gradient; statistics recomputed in the backward; the element-wise path for unaligned
rows; large-mean rows; exact cases; empty inputs; bitwise run-to-run determinism; guard bands
around every buffer; workspace errors and the two-stage backward.
"""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

import oracle
from deep_learning_normalization_amd import inputs, normlib as nl
from tests.parity import (check_colsums, check_h, check_values, dx_floor, run_and_check,
                          tuned)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "exact_cases.json")


def _say(msg):
    print("[gpu] " + msg, flush=True)


def _small(kind, dtype, M, N, seed=0, **kw):
    base = dict(x=inputs.normal(0.3, 1.5), w=inputs.normal(1, 0.1), dy=inputs.normal(0, 1),
                b=inputs.normal(0, 0.1) if kind == "layernorm" else None)
    base.update(kw)
    eps = 1e-5 if kind == "layernorm" else 1e-6
    return inputs.Workload("%s_%s_%dx%d" % (kind, dtype, M, N), kind, dtype, M, N, eps, seed=seed,
                           **base)


# ---- full-size workloads ----------------------------------------------------------------------

@pytest.mark.parametrize("w", inputs.all_workloads(), ids=lambda w: w.name)
def test_full_size_workload(w):
    _say("full size %s (%d x %d, %s %s)" % (w.name, w.M, w.N, w.kind, w.dtype))
    out = run_and_check(w)
    torch.cuda.synchronize()
    assert out["rows_compared"] == w.M
    _say("full size %s: rows compared %d of %d (100%%), every column of dW/dB"
         % (w.name, out["rows_compared"], w.M))


# ---- sweep around tile and scheme boundaries ----------------------------------------------------

SWEEP_N = [1, 2, 7, 8, 63, 64, 65, 1000, 1023, 1024, 1025, 2048, 5120, 7168, 8200, 16384, 65535,
           65536, 262144]


def _sweep_cases():
    out = []
    for N in SWEEP_N:
        Ms = [1, 3, 257] if N <= 16384 else [1, 3, 17]
        for M in Ms:
            for kind in ("layernorm", "rmsnorm"):
                for dt in ("bf16", "f32"):
                    out.append((kind, dt, M, N))
    return out


@pytest.mark.parametrize("kind,dt,M,N", _sweep_cases(), ids=lambda v: str(v))
def test_sweep(kind, dt, M, N):
    _say("sweep %s %s %dx%d" % (kind, dt, M, N))
    run_and_check(_small(kind, dt, M, N, seed=M + N))


# ---- each scheme forced, outside its natural range -------------------------------------------

FORCED = [
    ("wave", nl.SCHEME_WAVE, [8, 200, 512, 1024, 2048, 4096]),
    ("block", nl.SCHEME_BLOCK, [8, 64, 200, 1000, 1024, 4104, 16384]),
    ("split", nl.SCHEME_SPLIT, [8, 200, 1024, 4096, 8200, 20000]),
    ("loop", nl.SCHEME_LOOP, [8, 200, 1000, 4100, 4104, 12288, 16384]),
]


@pytest.mark.parametrize("name,scheme,Ns", FORCED, ids=[f[0] for f in FORCED])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("kind", ["layernorm", "rmsnorm"])
def test_forced_scheme(name, scheme, Ns, dt, kind):
    esize = 2 if dt == "bf16" else 4
    for N in Ns:
        if name == "wave" and N * esize > 64 * 8 * 16:
            continue  # longer than one wavefront's registers
        if name == "block" and N * esize > 1024 * 16:
            continue  # longer than a backward team's registers (1024 16-byte accesses)
        if name == "loop" and (N * esize > 2048 * 16 or N * esize % 8):
            continue  # beyond 512 threads x 4 16-byte accesses, or narrower than 8 bytes
        for M in (1, 5, 300):
            _say("forced %s %s %s %dx%d" % (name, kind, dt, M, N))
            with tuned(scheme=scheme):
                run_and_check(_small(kind, dt, M, N, seed=3 * M + N))
                run_and_check(_small(kind, dt, M, N, seed=3 * M + N + 1), stats=False)


# ---- the split scheme's two forms ----------------------------------------------------------------
# Single pass (the workgroups of a row exchange chunk partials, each chunk stays in registers)
# and two passes (the second re-reads its chunk). The backward's single pass needs the saved
# statistics; with stats=False it recomputes them and runs two passes either way.

SPLIT_FORMS = [("exchange", 1), ("two_pass", 0)]


def _split_form(kind, dt, pass_, M, N):
    p = nl.norm_plan(kind, inputs.TORCH_DTYPES[dt], pass_, M, N,
                     cu_count=torch.cuda.get_device_properties(0).multi_processor_count)
    return p["exchange_row_groups"]


@pytest.mark.parametrize("form,flag", SPLIT_FORMS, ids=[f[0] for f in SPLIT_FORMS])
@pytest.mark.parametrize("dt", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("kind", ["layernorm", "rmsnorm"])
def test_split_forms(form, flag, dt, kind):
    for N in (8200, 20000, 65536, 262144):
        for M in ((1, 3, 300) if N <= 65536 else (1, 17)):
            _say("split form %s %s %s %dx%d" % (form, kind, dt, M, N))
            with tuned(scheme=nl.SCHEME_SPLIT, exchange=flag):
                if flag and N % 8 == 0:
                    assert _split_form(kind, dt, nl.PASS_FWD, M, N) > 0
                    assert _split_form(kind, dt, nl.PASS_BWD, M, N) > 0
                run_and_check(_small(kind, dt, M, N, seed=5 * M + N))
                run_and_check(_small(kind, dt, M, N, seed=5 * M + N + 1), stats=False)


@pytest.mark.parametrize("knob", [dict(row_groups=1), dict(row_groups=7), dict()],
                         ids=["one_group", "seven_groups", "default"])
@pytest.mark.parametrize("kind", ["layernorm", "rmsnorm"])
def test_split_exchange_many_rows_per_group(kind, knob):
    """Each row group walks many rows: the prefetch of the next row, the exchange words of
    every row, and the column partials kept over the group's rows (one group writes dW and dB
    itself)."""
    M, N = 2000, 65536
    _say("split exchange %s %dx%d %s" % (kind, M, N, knob))
    with tuned(exchange=1, **knob):
        assert _split_form(kind, "bf16", nl.PASS_BWD, M, N) > 0
        run_and_check(_small(kind, "bf16", M, N, seed=M))


def test_split_exchange_mixed_weights_and_residual():
    for kind in ("layernorm", "rmsnorm"):
        for N in (20000, 262144):
            _say("split exchange fp32 weights %s N=%d" % (kind, N))
            w = dataclasses.replace(_small(kind, "bf16", 9, N, seed=N), wdtype="f32")
            with tuned(exchange=1):
                run_and_check(w)
    # the residual variant: its forward takes two passes, its backward (with dH) one
    for dr in ("alias", "separate"):
        _say("split exchange residual dr=%s" % dr)
        w = dataclasses.replace(_small("rmsnorm", "bf16", 9, 40000, seed=3,
                                       r=inputs.normal(0, 1)), wdtype="f32")
        with tuned(exchange=1):
            run_and_check(w, dr=dr, dh=True)


@pytest.mark.parametrize("N,knob", [(512, dict()), (4096, dict()), (4100, dict()),
                                    (12288, dict()), (65536, dict(exchange=1)),
                                    (65536, dict(exchange=0))],
                         ids=["wave", "block", "block8", "loop", "split1", "split2"])
@pytest.mark.parametrize("kind", ["layernorm", "rmsnorm"])
def test_nan_row_propagates(kind, N, knob):
    """A NaN in one row makes that row's statistics, output and dX NaN (and the column sums it
    enters) and leaves the other rows alone, on every scheme, the statistics pass included."""
    M = 5
    _say("nan row %s N=%d %s" % (kind, N, knob))
    w = _small(kind, "bf16", M, N, seed=N)
    t = inputs.make(w)
    t["X"][2, N // 3] = float("nan")
    X, W, B, dY = (t[k].cuda() if t[k] is not None else None for k in ("X", "W", "B", "dY"))
    with tuned(**knob):
        Y, _, mean, rstd = nl.forward(kind, X, W, B, w.eps)
        dX, dW, _ = nl.backward(kind, X, dY, W, mean, rstd, w.eps)
        dX2, _, _ = nl.backward(kind, X, dY, W, None, None, w.eps)
        ws = nl.workspace(kind, torch.bfloat16, nl.PASS_STATS, M, N)
        m3 = torch.empty(M, device="cuda") if kind == "layernorm" else None
        r3 = torch.empty(M, device="cuda")
        nl.norm_stats(kind, X, None, w.eps, None, m3, r3, ws)
        torch.cuda.synchronize()
    others = [0, 1, 3, 4]
    for r in (rstd, r3):
        assert torch.isnan(r[2]) and torch.isfinite(r[others]).all()
    for a in (Y, dX, dX2):
        assert torch.isnan(a[2].float()).all() and torch.isfinite(a[others].float()).all()
    assert torch.isnan(dW.float()).all()


@pytest.mark.parametrize("kind", ["layernorm", "rmsnorm"])
def test_split_exchange_chunk_limits(kind):
    """Rows at the single-pass form's limits: the most chunks of 8192 a forward takes (two row
    groups of 4 workgroups per CU, at most 512), 512 (the most the backward takes), and one
    chunk past each, which run two passes; every one must match the oracle. The chunk counts
    follow the device's CU count. The form is forced (by default LayerNorm rows of more than
    341 chunks take two passes)."""
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    fwd_max = min(512, 4 * cu // 2)
    bwd_max = min(512, 2 * cu)
    for C, ragged in ((fwd_max, 0), (fwd_max + 1, 0), (bwd_max, 0), (bwd_max, 8)):
        N = 8192 * C + ragged
        _say("split exchange limits %s N=%d" % (kind, N))
        with tuned(exchange=1):
            f = _split_form(kind, "bf16", nl.PASS_FWD, 2, N)
            b = _split_form(kind, "bf16", nl.PASS_BWD, 2, N)
            nchunks = -(-N // 8192)
            assert (f > 0) == (nchunks <= fwd_max) and (b > 0) == (nchunks <= bwd_max)
            run_and_check(_small(kind, "bf16", 2, N, seed=C + ragged))


def test_split_exchange_wait_is_bounded():
    """The exchange's wait gives up rather than hangs: with chunk 0 withholding its partials
    (a test-only flag) and a poll limit of 8, every row of the call comes out NaN, the kernels
    finish, the workspace reports the failure (once: the query clears it), and the next call on
    the same workspaces without the flag is correct again and reports nothing."""
    M, N = 64, 65536
    for kind in ("layernorm", "rmsnorm"):
        _say("split exchange bounded wait %s %dx%d" % (kind, M, N))
        w = _small(kind, "bf16", M, N, seed=9)
        t = inputs.make(w)
        X, W, B, dY = (t[k].cuda() if t[k] is not None else None for k in ("X", "W", "B", "dY"))
        ln = kind == "layernorm"
        wsf = nl.workspace(kind, X.dtype, nl.PASS_FWD, M, N)
        wsb = nl.workspace(kind, X.dtype, nl.PASS_BWD, M, N)

        def fwd():
            Y = torch.empty_like(X)
            mean = torch.empty(M, device="cuda") if ln else None
            rstd = torch.empty(M, device="cuda")
            nl.norm_fwd(kind, X, None, W, B, w.eps, Y, None, mean, rstd, wsf)
            return Y, mean, rstd

        def bwd(mean, rstd):
            dX, dW = torch.empty_like(X), torch.empty_like(W)
            dB = torch.empty_like(W) if ln else None
            nl.norm_bwd(kind, X, dY, None, W, mean, rstd, w.eps, dX, None, dW, dB, wsb)
            return dX, dW, dB

        with tuned(exchange=1):
            Y0, mean0, rstd0 = fwd()
            dX0, dW0, _ = bwd(mean0, rstd0)
            assert _split_form(kind, "bf16", nl.PASS_FWD, M, N) > 0
            assert _split_form(kind, "bf16", nl.PASS_BWD, M, N) > 0
        assert nl.norm_workspace_status(wsf) == nl.OK
        assert nl.norm_workspace_status(wsb) == nl.OK
        with tuned(exchange=1, polls=8, withhold=1):
            Y, _, rstd = fwd()
            dX, dW, dB = bwd(mean0, rstd0)
            torch.cuda.synchronize()
        assert torch.isnan(Y.float()).all() and torch.isnan(rstd).all()
        assert torch.isnan(dX.float()).all() and torch.isnan(dW.float()).all()
        assert nl.norm_workspace_status(wsf) == nl.ERR_EXCHANGE
        assert nl.norm_workspace_status(wsf) == nl.OK  # the query cleared it
        assert nl.norm_workspace_status(wsb) == nl.ERR_EXCHANGE
        assert nl.norm_workspace_status(wsb) == nl.OK
        with tuned(exchange=1):
            Y2, _, rstd2 = fwd()
            dX2, dW2, _ = bwd(mean0, rstd0)
            torch.cuda.synchronize()
        assert torch.equal(Y2.view(torch.int16), Y0.view(torch.int16))
        assert torch.equal(rstd2, rstd0)
        assert torch.equal(dX2.view(torch.int16), dX0.view(torch.int16))
        assert torch.equal(dW2.view(torch.int16), dW0.view(torch.int16))
        assert nl.norm_workspace_status(wsf) == nl.OK
        assert nl.norm_workspace_status(wsb) == nl.OK
        run_and_check(w)


def test_split_exchange_needs_no_clean_workspace():
    """The exchange words carry a tag of the call that wrote them, so no call needs its words
    cleared first: a workspace full of random bits, one last used by a call of another shape
    (whose words then sit where this call's go), and one reused call after call all give the
    bits of a fresh workspace, and match the oracle."""
    for kind in ("layernorm", "rmsnorm"):
        for M, N in ((64, 65536), (3, 262144)):
            _say("split exchange stale words %s %dx%d" % (kind, M, N))
            w = _small(kind, "bf16", M, N, seed=M + N)
            t = inputs.make(w)
            X, W, B, dY = (t[k].cuda() if t[k] is not None else None
                           for k in ("X", "W", "B", "dY"))
            ln = kind == "layernorm"
            nf = nl.norm_workspace_size(kind, X.dtype, nl.PASS_FWD, M, N)
            nb = nl.norm_workspace_size(kind, X.dtype, nl.PASS_BWD, M, N)
            big = max(nf, nb, nl.norm_workspace_size(kind, X.dtype, nl.PASS_BWD, 2 * M, N))

            def run(ws):
                Y = torch.empty_like(X)
                mean = torch.empty(M, device="cuda") if ln else None
                rstd = torch.empty(M, device="cuda")
                nl.norm_fwd(kind, X, None, W, B, w.eps, Y, None, mean, rstd, ws[:nf])
                dX, dW = torch.empty_like(X), torch.empty_like(W)
                dB = torch.empty_like(W) if ln else None
                nl.norm_bwd(kind, X, dY, None, W, mean, rstd, w.eps, dX, None, dW, dB, ws[:nb])
                torch.cuda.synchronize()
                return [v.view(torch.int16) if v.dtype == torch.bfloat16 else v
                        for v in (Y, rstd, dX, dW, dB) if v is not None]

            with tuned(exchange=1):
                assert _split_form(kind, "bf16", nl.PASS_FWD, M, N) > 0
                ref = run(torch.zeros(big, dtype=torch.uint8, device="cuda"))
                g = torch.Generator(device="cuda").manual_seed(M + N)
                noise = torch.randint(0, 256, (big,), dtype=torch.uint8, device="cuda",
                                      generator=g)
                for got in (run(noise), run(noise), run(noise)):
                    assert all(torch.equal(a, b) for a, b in zip(got, ref))
                # words of a call with twice the rows (another layout) left in the workspace
                other = torch.zeros(big, dtype=torch.uint8, device="cuda")
                X2 = torch.cat([X, X])
                Y2 = torch.empty_like(X2)
                nl.norm_bwd(kind, X2, torch.cat([dY, dY]), None, W,
                            torch.zeros(2 * M, device="cuda") if ln else None,
                            torch.ones(2 * M, device="cuda"), w.eps, Y2, None,
                            torch.empty_like(W), torch.empty_like(W) if ln else None, other)
                assert all(torch.equal(a, b) for a, b in zip(run(other), ref))
                assert nl.norm_workspace_status(noise[:nf]) == nl.OK
                assert nl.norm_workspace_status(other[:nb]) == nl.OK
            run_and_check(w)


# ---- bf16 activations with fp32 weight, bias, dW, dB --------------------------------------------

@pytest.mark.parametrize("kind", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("N", [8, 512, 1000, 4096, 5120, 20000, 300000])
def test_mixed_weight_type(kind, N):
    Ms = (1, 5, 300) if N <= 20000 else (1, 3)
    for M in Ms:
        _say("mixed weights %s %dx%d" % (kind, M, N))
        w = dataclasses.replace(_small(kind, "bf16", M, N, seed=M + N), wdtype="f32")
        run_and_check(w)
        run_and_check(dataclasses.replace(w, seed=M + N + 1), stats=False)


@pytest.mark.parametrize("name,scheme,N", [("wave", nl.SCHEME_WAVE, 1024),
                                           ("block", nl.SCHEME_BLOCK, 4104),
                                           ("split", nl.SCHEME_SPLIT, 20000)],
                         ids=["wave", "block", "split"])
def test_mixed_weight_type_forced_schemes(name, scheme, N):
    for kind in ("layernorm", "rmsnorm"):
        _say("mixed weights forced %s %s N=%d" % (name, kind, N))
        with tuned(scheme=scheme):
            w = dataclasses.replace(_small(kind, "bf16", 77, N, seed=N), wdtype="f32")
            run_and_check(w)


@pytest.mark.parametrize("dr", ["alias", "separate"])
def test_mixed_weight_type_residual(dr):
    for N in (1024, 7168, 40000):
        _say("mixed weights residual dr=%s N=%d" % (dr, N))
        w = dataclasses.replace(_small("rmsnorm", "bf16", 33, N, seed=N, r=inputs.normal(0, 1)),
                                wdtype="f32")
        run_and_check(w, dr=dr, dh=True)


def test_mixed_weight_type_unaligned():
    # N % 8 != 0: 8-byte (N % 4 == 0), 4-byte (N even) and element-wise (N odd) accesses with
    # fp32 weights
    for kind in ("layernorm", "rmsnorm"):
        for N in (100, 4100, 102, 4098, 101, 4097):
            _say("mixed weights narrow or element-wise %s N=%d" % (kind, N))
            w = dataclasses.replace(_small(kind, "bf16", 9, N, seed=N), wdtype="f32")
            run_and_check(w)


@pytest.mark.parametrize("wdtype", [None, "f32"])
def test_split_direct_dw_unaligned_outputs(wdtype):
    # one row group in the split scheme writes dW, dB itself; outputs that are not 16-byte
    # aligned take the reduction pass instead
    w = dataclasses.replace(_small("layernorm", "bf16", 2, 300000, seed=3), wdtype=wdtype)
    t = inputs.make(w)
    dev = "cuda"
    X, W, B, dY = (t[k].to(dev) for k in ("X", "W", "B", "dY"))
    _say("split direct dW, unaligned outputs, wdtype=%s" % wdtype)
    Y, _, mean, rstd = nl.forward("layernorm", X, W, B, w.eps)
    ref_dx, ref_dw, ref_db = nl.backward("layernorm", X, dY, W, mean, rstd, w.eps)
    big_w = torch.zeros(w.N + 1, dtype=W.dtype, device=dev)
    big_b = torch.zeros(w.N + 1, dtype=W.dtype, device=dev)
    dX = torch.empty_like(X)
    dW, dB = big_w[1:], big_b[1:]                  # one element past an aligned start
    ws = nl.workspace("layernorm", X.dtype, nl.PASS_BWD, w.M, w.N, device=dev)
    nl.norm_bwd("layernorm", X, dY, None, W, mean, rstd, w.eps, dX, None, dW, dB, ws)
    torch.cuda.synchronize()
    assert torch.equal(dX, ref_dx)
    # the same column sums in another order: within the dW/dB tolerance of each other
    check_colsums("dW", dW.double().cpu().numpy(), ref_dw.double().cpu().numpy(), "f32")
    check_colsums("dB", dB.double().cpu().numpy(), ref_db.double().cpu().numpy(), "f32")


# ---- fp16 storage, and fp16 activations with fp32 weights ---------------------------------------

F16_N = [1, 7, 64, 1000, 1024, 1025, 1002, 4096, 4100, 4098, 5120, 8192, 12288, 16384, 20000,
         262144]


def _f16_cases():
    out = []
    for N in F16_N:
        for kind in ("layernorm", "rmsnorm"):
            for wdt in (None, "f32"):
                out.append((kind, wdt, 129 if N <= 20000 else 5, N))
    return out


@pytest.mark.parametrize("kind,wdt,M,N", _f16_cases(), ids=lambda v: str(v))
def test_fp16(kind, wdt, M, N):
    _say("fp16 %s w=%s %dx%d" % (kind, wdt, M, N))
    w = dataclasses.replace(_small(kind, "f16", M, N, seed=M + N), wdtype=wdt)
    run_and_check(w)
    run_and_check(dataclasses.replace(w, seed=M + N + 1), stats=False)


@pytest.mark.parametrize("name,scheme,N", [("wave", nl.SCHEME_WAVE, 512),
                                           ("block", nl.SCHEME_BLOCK, 4096),
                                           ("loop", nl.SCHEME_LOOP, 4096),
                                           ("split", nl.SCHEME_SPLIT, 4096)],
                         ids=lambda v: str(v))
def test_fp16_forced_schemes(name, scheme, N):
    for kind in ("layernorm", "rmsnorm"):
        for wdt in (None, "f32"):
            _say("fp16 forced %s %s w=%s N=%d" % (name, kind, wdt, N))
            with tuned(scheme=scheme):
                run_and_check(dataclasses.replace(_small(kind, "f16", 77, N, seed=N), wdtype=wdt))


@pytest.mark.parametrize("N", [512, 7168, 4098])
def test_fp16_residual(N):
    for kind in ("rmsnorm", "layernorm"):
        _say("fp16 residual %s N=%d" % (kind, N))
        w = _small(kind, "f16", 65, N, seed=N, x=inputs.normal(0, 0.5), r=inputs.normal(0, 1))
        run_and_check(w, dr="alias", dh=True)
        run_and_check(dataclasses.replace(w, seed=N + 1, wdtype="f32"), dr="separate")


def test_fp16_overflow_and_subnormal_outputs():
    """Outputs beyond fp16's range round to infinity, tiny ones to subnormals, on both sides:
    a weight of 2^15 scales normalised values beyond 2 past 65504, one of 2^-20 into the
    subnormals."""
    for wscale in (2.0 ** 15, 2.0 ** -20):
        w = _small("rmsnorm", "f16", 33, 1000, seed=5, w=inputs.const(wscale))
        _say("fp16 range, weight %g" % wscale)
        out = run_and_check(w, want_bwd=False)
        y = out["Y"].float()
        if wscale > 1:
            assert torch.isinf(y).any()
        else:
            assert ((y != 0) & (y.abs() < 2.0 ** -14)).any()


# ---- 8- and 4-byte accesses ---------------------------------------------------------------------

# Even row lengths that are not a multiple of the 16-byte vector (bf16: N % 8 != 0; fp32:
# N % 4 != 0), across the wave, block and split schemes.
NARROW_N = [2, 6, 10, 12, 100, 1002, 1004, 1026, 1028, 2050, 4098, 4100, 5122, 7170, 8194, 8196,
            16386, 16388, 20002, 262146]


def _narrow_cases():
    out = []
    for N in NARROW_N:
        for kind in ("layernorm", "rmsnorm"):
            for dt, wdt in (("bf16", None), ("bf16", "f32"), ("f32", None)):
                if dt == "f32" and N % 4 == 0:
                    continue  # 16-byte accesses
                out.append((kind, dt, wdt, 129 if N <= 20002 else 9, N))
    return out


def _access_bytes(kind, dt, wdt, M, N, residual=False, align=16):
    code = nl.BF16_F32W if wdt == "f32" else inputs.TORCH_DTYPES[dt]
    return nl.norm_plan(kind, code, 0, M, N, residual, align=align)["access_bytes"]


# (The default takes 16-byte accesses over row phase classes for these rows when all tensors
# share a phase; these tests switch that off to cover the 8- and 4-byte kernels, which serve
# tensors at mixed phases.)

@pytest.mark.parametrize("kind,dt,wdt,M,N", _narrow_cases(), ids=lambda v: str(v))
def test_narrow_access_widths(kind, dt, wdt, M, N):
    with tuned(unaligned=0):
        width = _access_bytes(kind, dt, wdt, M, N)
        assert width == (8 if (dt == "f32" or N % 4 == 0) else 4)
        _say("narrow %d-byte %s %s w=%s %dx%d" % (width, kind, dt, wdt, M, N))
        w = dataclasses.replace(_small(kind, dt, M, N, seed=M + N), wdtype=wdt)
        run_and_check(w)
        run_and_check(dataclasses.replace(w, seed=M + N + 1), stats=False)


@pytest.mark.parametrize("N", [1002, 4098, 4100, 7170, 8194, 16386])
@pytest.mark.parametrize("kind", ["rmsnorm", "layernorm"])
def test_narrow_residual(kind, N):
    _say("narrow residual %s N=%d" % (kind, N))
    w = _small(kind, "bf16", 65, N, seed=N, x=inputs.normal(0, 0.5), r=inputs.normal(0, 1))
    with tuned(unaligned=0):
        run_and_check(w, dr="alias", dh=True)
        run_and_check(dataclasses.replace(w, seed=N + 1), dr="separate")


@pytest.mark.parametrize("N", [4098, 4100, 8196])
@pytest.mark.parametrize("knob", [dict(scheme=nl.SCHEME_SPLIT), dict(scheme=nl.SCHEME_BLOCK),
                                  dict(scheme=nl.SCHEME_LOOP), dict(team_threads=1024),
                                  dict(grid_per_cu=1)],
                         ids=lambda k: str(k))
def test_narrow_forced(knob, N):
    if knob.get("scheme") == nl.SCHEME_BLOCK and N * 2 > 1024 * 16:
        pytest.skip("longer than a backward team's registers (1024 16-byte accesses)")
    if knob.get("scheme") == nl.SCHEME_LOOP and N % 4:
        pytest.skip("the looped backward has no 4-byte kernels")
    for kind in ("layernorm", "rmsnorm"):
        _say("narrow knob %s %s N=%d" % (knob, kind, N))
        with tuned(unaligned=0, **knob):
            run_and_check(_small(kind, "bf16", 77, N, seed=N))


@pytest.mark.parametrize("N", [1600, 2048])
def test_rms_bf16_four_row_backward(N):
    """The default plan of bf16 RMSNorm backward rows of 1544-2048 elements holds four rows per
    256-thread team; every row (ragged counts, one to a few hundred groups) against the
    oracle."""
    p = nl.norm_plan("rmsnorm", torch.bfloat16, nl.PASS_BWD, 32768, N)
    assert (p["threads"], p["accesses_per_thread"], p["rows_per_iter"]) == (256, 1, 4)
    for M in (1, 5, 1003):
        _say("rms bf16 four-row backward %dx%d" % (M, N))
        run_and_check(_small("rmsnorm", "bf16", M, N, seed=M + N))
        run_and_check(_small("rmsnorm", "bf16", M, N, seed=M + N + 1), stats=False)


_WIDE_FWD = [(kind, N, res, dt) for dt in ("bf16", "f16", "bf16_f32w")
             for kind, N, res in [("layernorm", 10240, False), ("layernorm", 16384, False),
                                  ("rmsnorm", 12288, False), ("layernorm", 8200, False),
                                  ("rmsnorm", 10240, True), ("layernorm", 12288, True)]]
_WIDE_FWD += [("layernorm", N, False, "f32") for N in (4100, 4608, 5120)]


@pytest.mark.parametrize("kind,N,res,dt", _WIDE_FWD, ids=lambda v: str(v))
def test_wide_forward_persistent_grid(kind, N, res, dt):
    """The default forward plan of 16-bit rows (either weight type) on teams of more than 256
    threads with four accesses each (320-384 threads for RMSNorm and the residual form), and of
    fp32 LayerNorm rows on 320 threads, runs a persistent grid of two workgroups per CU: row
    counts below, at and past one row per workgroup, every row against the oracle."""
    wdt = None
    if dt == "bf16_f32w":
        dt, wdt = "bf16", "f32"
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    pdt = nl.BF16_F32W if wdt else inputs.TORCH_DTYPES[dt]
    p = nl.norm_plan(kind, pdt, nl.PASS_FWD, 16384, N, residual=res, cu_count=cu)
    assert p["threads"] > 256 and p["accesses_per_thread"] == 4 and p["grid"] == 2 * cu
    extra = dict(x=inputs.normal(0, 0.5), r=inputs.normal(0, 1)) if res else {}
    for M in (1, 7, 2 * cu, 2 * cu + 1, 1500):
        _say("wide forward %s %s/%s residual=%s %dx%d" % (kind, dt, wdt, res, M, N))
        w = dataclasses.replace(_small(kind, dt, M, N, seed=M + N, **extra), wdtype=wdt)
        if res:
            run_and_check(w, dr="alias", dh=True)
        else:
            run_and_check(w)


@pytest.mark.parametrize("kind,dt,N,res,wdt,seg", [("rmsnorm", "bf16", 8200, False, None, 4),
                                                   ("rmsnorm", "bf16", 14336, False, None, 4),
                                                   ("rmsnorm", "f16", 10240, True, None, 4),
                                                   ("layernorm", "f32", 4100, False, None, 4),
                                                   ("layernorm", "f32", 7168, True, None, 4),
                                                   ("rmsnorm", "f32", 6144, False, None, 4),
                                                   ("layernorm", "bf16", 8200, False, None, 3),
                                                   ("layernorm", "bf16", 12288, True, None, 3),
                                                   ("layernorm", "f16", 10240, False, None, 3),
                                                   ("layernorm", "bf16", 11264, False, "f32", 3),
                                                   ("layernorm", "bf16", 14336, False, None, 4),
                                                   ("layernorm", "bf16", 16384, True, None, 4),
                                                   ("layernorm", "bf16", 12800, False, "f32", 4),
                                                   ("layernorm", "f16", 14336, False, None, 4)])
def test_looped_backward_two_per_cu(kind, dt, N, res, wdt, seg):
    """The default looped backward runs two workgroups per CU where its registers allow two
    512-thread teams and rows are at most 28 KB (LayerNorm on 16-bit rows of at most 1536
    accesses through its three-segment kernel), and for every 16-bit LayerNorm row (its
    four-segment kernel keeps the dB sums in LDS): row counts below, at and past one row per
    workgroup, with and without saved statistics, every row and every dW/dB column against the
    oracle."""
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    p = nl.norm_plan(kind, inputs.TORCH_DTYPES[dt], nl.PASS_BWD, 16384, N, residual=res,
                     cu_count=cu)
    assert p["scheme"] == nl.SCHEME_LOOP and p["grid"] == 2 * cu
    assert (p["threads"], p["accesses_per_thread"]) == (512, seg)
    extra = dict(x=inputs.normal(0, 0.5), r=inputs.normal(0, 1)) if res else {}
    for M in (1, 7, 2 * cu, 2 * cu + 1, 1100):
        _say("looped two per CU %s %s/%s residual=%s %dx%d" % (kind, dt, wdt, res, M, N))
        w = dataclasses.replace(_small(kind, dt, M, N, seed=M + N, **extra), wdtype=wdt)
        if res:
            run_and_check(w, dr="alias", dh=True)
            run_and_check(dataclasses.replace(w, seed=M + N + 1), dr="separate", stats=False)
        else:
            run_and_check(w)
            run_and_check(dataclasses.replace(w, seed=M + N + 1), stats=False)


@pytest.mark.parametrize("kind,dt,N", [("layernorm", "bf16", 2049), ("rmsnorm", "bf16", 2049),
                                       ("layernorm", "f16", 2561), ("layernorm", "f32", 1025),
                                       ("rmsnorm", "f32", 1283)])
def test_phase_class_four_row_backward(kind, dt, N):
    """The default backward over phase classes on 320-384-thread teams with one access each
    holds four rows: row counts below, at and past one row group per workgroup, every row and
    every dW/dB column against the oracle, rows at every phase (odd N)."""
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    p = nl.norm_plan(kind, inputs.TORCH_DTYPES[dt], nl.PASS_BWD, 16384, N, cu_count=cu)
    assert p["phase_classes"] > 1 and p["accesses_per_thread"] == 1 and p["rows_per_iter"] == 4
    assert 320 <= p["threads"] <= 384
    for M in (1, 5, 4 * cu + 3, 3001):
        _say("phase-class four-row backward %s %s %dx%d" % (kind, dt, M, N))
        run_and_check(_small(kind, dt, M, N, seed=M + N))
        run_and_check(_small(kind, dt, M, N, seed=M + N + 1), stats=False)


@pytest.mark.parametrize("kind,dt,N", [("rmsnorm", "bf16", 256), ("layernorm", "bf16", 512),
                                       ("rmsnorm", "f16", 512), ("rmsnorm", "bf16", 1280),
                                       ("layernorm", "bf16", 1536), ("rmsnorm", "bf16", 2560),
                                       ("rmsnorm", "f16", 3072), ("layernorm", "bf16", 2304),
                                       ("layernorm", "f16", 2560), ("layernorm", "bf16", 3072),
                                       ("rmsnorm", "f32", 256), ("layernorm", "f32", 1280),
                                       ("rmsnorm", "f32", 1536), ("rmsnorm", "bf16_f32w", 512),
                                       ("layernorm", "bf16_f32w", 1536),
                                       ("layernorm", "bf16_f32w", 2560)])
def test_backward_team_rules(kind, dt, N):
    """The default backward plans of rows of up to 3072 elements (several rows per wavefront,
    three or two workgroups per CU, 256-thread LayerNorm teams of two accesses):
    ragged row counts from one to several row groups per workgroup, with and without saved
    statistics, every row and every dW/dB column against the oracle."""
    wdt = None
    if dt == "bf16_f32w":
        dt, wdt = "bf16", "f32"
    for M in (1, 7, 1003, 4099):
        _say("backward team rules %s %s/%s %dx%d" % (kind, dt, wdt, M, N))
        run_and_check(dataclasses.replace(_small(kind, dt, M, N, seed=M + N), wdtype=wdt))
        run_and_check(dataclasses.replace(_small(kind, dt, M, N, seed=M + N + 1), wdtype=wdt),
                      stats=False)


# ---- tuning knobs ----------------------------------------------------------------------------

KNOBS = [
    dict(rows=2), dict(rows=4), dict(grid_per_cu=1), dict(grid_per_cu=16),
    dict(team_threads=1024), dict(team_threads=128, rows=2),
    dict(scheme=nl.SCHEME_SPLIT, split_chunk=2048), dict(scheme=nl.SCHEME_SPLIT, split_chunk=4096),
    dict(scheme=nl.SCHEME_SPLIT, row_groups=1), dict(scheme=nl.SCHEME_SPLIT, row_groups=7),
    dict(scheme=nl.SCHEME_SPLIT, rows=1), dict(scheme=nl.SCHEME_SPLIT, rows=4),
    dict(teams=2), dict(team_threads=256, teams=4), dict(team_threads=512, teams=2, rows=2),
    dict(rows=1), dict(row_order=1), dict(row_order=1, rows=1),
    dict(row_order=1, grid_per_cu=16),         # more workgroups than row groups: some idle
    dict(row_order=1, team_threads=256, teams=4),
    dict(scheme=nl.SCHEME_LOOP), dict(scheme=nl.SCHEME_LOOP, grid_per_cu=3),
]


@pytest.mark.parametrize("knob", KNOBS, ids=lambda k: ",".join("%s=%s" % i for i in k.items()))
@pytest.mark.parametrize("kind,dt,M,N", [("layernorm", "bf16", 1000, 4096),
                                        ("rmsnorm", "bf16", 777, 1024),
                                        ("rmsnorm", "f32", 333, 7168),
                                        ("layernorm", "f32", 65, 520),
                                        ("layernorm", "bf16", 300, 12288)])
def test_tuning_knobs(knob, kind, dt, M, N):
    _say("knob %s %s %s %dx%d" % (knob, kind, dt, M, N))
    with tuned(**knob):
        run_and_check(_small(kind, dt, M, N, seed=M))


@pytest.mark.parametrize("kind", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("dt,wdt", [("bf16", None), ("f32", None), ("f16", None),
                                    ("bf16", "f32")])
def test_backward_ragged_row_groups(kind, dt, wdt):
    """The wave and block backwards on row counts that end a workgroup's walk part-way through
    a row group (rows past M load a clamped row in the RMSNorm kernels and must leave no trace),
    on rows shorter than a team (columns past the row end masked), with grids that leave
    workgroups one, two or many groups; the statistics recomputed, an incoming dH and a separate
    dR."""
    for N in (1024, 4096, 1000):
        for M in (1, 2, 3, 5, 257, 1000):
            for gpc in (-1, 1, 64):
                _say("ragged row groups %s %s/%s %dx%d grid/cu %d" % (kind, dt, wdt, M, N, gpc))
                w = dataclasses.replace(_small(kind, dt, M, N, seed=M * N + gpc), wdtype=wdt)
                with tuned(grid_per_cu=gpc):
                    run_and_check(w)
                    if M == 257:
                        run_and_check(dataclasses.replace(w, seed=M + 1), stats=False)
                        run_and_check(dataclasses.replace(w, seed=M + 2), dr="separate", dh=True)


# ---- residual variant -----------------------------------------------------------------------

@pytest.mark.parametrize("dr", ["none", "alias", "separate"])
@pytest.mark.parametrize("dh", [False, True])
@pytest.mark.parametrize("kind", ["rmsnorm", "layernorm"])
@pytest.mark.parametrize("N", [512, 7168, 12288, 20000])
def test_residual(dr, dh, kind, N):
    _say("residual %s N=%d dr=%s dh=%s" % (kind, N, dr, dh))
    w = _small(kind, "bf16", 129, N, seed=N, x=inputs.normal(0, 0.5), r=inputs.normal(0, 1))
    run_and_check(w, dr=dr, dh=dh)


def test_residual_full_shape_sample():
    """Residual RMSNorm at 65536 x 7168 with dR a separate buffer and an incoming dH."""
    w = dataclasses.replace(inputs.RESID_RMS_BF16_65536x7168, M=8192)
    _say("residual 8192x7168 separate dR + dH")
    run_and_check(w, dr="separate", dh=True)


# ---- statistics recomputed in the backward -----------------------------------------------------

@pytest.mark.parametrize("kind", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("N", [256, 4096, 12288, 300000])
def test_backward_without_saved_stats(kind, N):
    _say("no saved stats %s N=%d" % (kind, N))
    run_and_check(_small(kind, "bf16", 37, N, seed=N), stats=False)


# ---- the statistics pass alone ------------------------------------------------------------------

# wave, block, split, 8-byte, element-wise and fp16 rows, and the residual variant
STATS_CASES = [("layernorm", "bf16", 300, 512, False), ("rmsnorm", "bf16", 300, 512, False),
               ("layernorm", "bf16", 129, 4096, False), ("rmsnorm", "f32", 129, 8192, False),
               ("layernorm", "bf16", 5, 262144, False), ("rmsnorm", "bf16", 3, 300000, False),
               ("layernorm", "bf16", 129, 4100, False), ("layernorm", "bf16", 65, 4097, False),
               ("layernorm", "f16", 129, 4096, False), ("rmsnorm", "bf16", 129, 7168, True),
               ("layernorm", "bf16", 9, 262144, True)]


@pytest.mark.parametrize("kind,dt,M,N,resid", STATS_CASES, ids=lambda v: str(v))
def test_stats_only(kind, dt, M, N, resid):
    """norm_stats gives the oracle's mean and rstd (and H), bit for bit the statistics that
    norm_fwd writes on the same inputs."""
    extra = dict(x=inputs.normal(0, 0.5), r=inputs.normal(0, 1)) if resid else {}
    w = _small(kind, dt, M, N, seed=N + M, **extra)
    t = inputs.make(w)
    X = t["X"].cuda()
    R = t["R"].cuda() if resid else None
    ln = kind == "layernorm"
    mean = torch.full((M,), float("nan"), device="cuda") if ln else None
    rstd = torch.full((M,), float("nan"), device="cuda")
    H = torch.empty_like(X) if resid else None
    _say("stats only %s %s %dx%d resid=%s" % (kind, dt, M, N, resid))
    ws = nl.workspace(kind, X.dtype, nl.PASS_FWD, M, N, resid)
    nl.norm_stats(kind, X, R, w.eps, H, mean, rstd, ws)
    Y, H2, mean2, rstd2 = nl.forward(kind, X, t["W"].cuda(), t["B"].cuda() if ln else None,
                                     w.eps, R=R)
    torch.cuda.synchronize()
    assert torch.equal(rstd, rstd2)
    if ln:
        assert torch.equal(mean, mean2)
    if resid:
        assert torch.equal(H, H2)
    bits = {k: inputs.host_bits(t[k]) for k in ("X", "W", "B", "R")}
    code = {"f32": oracle.F32, "bf16": oracle.BF16, "f16": oracle.F16}[dt]
    k = oracle.LAYERNORM if ln else oracle.RMSNORM
    f = oracle.fwd(k, code, bits["X"], bits["W"], bits["B"], bits["R"],
                   eps=float(np.float32(w.eps)), want_h=resid)
    from tests.parity import check_stats
    check_stats(mean.double().cpu().numpy() if ln else None, rstd.double().cpu().numpy(),
                f["mean"] if ln else None, f["rstd"])
    if resid:
        check_h(H.double().cpu().numpy(), f["h"], dt)


# ---- row-strided tensors -----------------------------------------------------------------------

def _strided_like(src, ld, col0, fill):
    """A CUDA view with src's values, row stride ld, starting col0 elements into each row of a
    [M, ld] buffer filled with `fill` (whose other columns must stay untouched)."""
    M, N = src.shape
    buf = torch.full((M, ld), fill, dtype=src.dtype, device="cuda")
    v = buf[:, col0:col0 + N]
    v.copy_(src.to("cuda"))
    return buf, v


# (kind, N, input stride, input column offset, output stride): the query rows of a fused
# [M, 3N] projection (stride 3N, offset 0 or N), padded rows, and strides that only allow
# narrower accesses (4100 bf16 elements: 8 bytes)
STRIDED = [("layernorm", 512, 1536, 512, 520), ("rmsnorm", 512, 1536, 0, 512),
           ("layernorm", 4096, 12288, 4096, 4100), ("rmsnorm", 4096, 4104, 8, 4096),
           ("rmsnorm", 12288, 36864, 12288, 12296), ("layernorm", 20000, 20008, 0, 20004),
           ("layernorm", 4100, 4108, 4, 4100)]


@pytest.mark.parametrize("kind,N,ldi,col0,ldo", STRIDED, ids=lambda v: str(v))
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_row_strided_tensors(kind, N, ldi, col0, ldo, dt):
    """Inputs and outputs as row-strided views: results match the oracle on the contiguous
    values, and the columns between the rows of every output keep their fill."""
    M = 37 if N <= 12288 else 9
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
    _say("strided %s %s N=%d in ld %d (+%d) out ld %d" % (kind, dt, N, ldi, col0, ldo))
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
    floor = dx_floor(np.arange(M), t["dY"], t["W"], f["rstd"], N).reshape(M, N)
    check_values("dX", dX.double().cpu().numpy(), g["dx"], dt, floor)
    check_colsums("dW", dW.double().cpu().numpy(), g["dw"], dt)
    if dB is not None:
        check_colsums("dB", dB.double().cpu().numpy(), g["db"], dt)
    # the gaps between output rows are untouched
    for buf, c0 in ((ybuf, ldo - N), (xbuf, 0)):
        gap = torch.ones(ldo, dtype=torch.bool, device="cuda")
        gap[c0:c0 + N] = False
        assert (buf[:, gap] == sentinel).all()


@pytest.mark.parametrize("N", [512, 4096, 7168])
def test_row_strided_residual(N):
    """Residual RMSNorm with R, X, H, dY, dH, dX and dR all row-strided views."""
    M = 33
    w = _small("rmsnorm", "bf16", M, N, seed=N, x=inputs.normal(0, 0.5), r=inputs.normal(0, 1),
               dh=inputs.normal(0, 0.5))
    t = inputs.make(w)
    ld = N + 24
    _, X = _strided_like(t["X"], 3 * N, N, 0.0)
    _, R = _strided_like(t["R"], 3 * N, 0, 0.0)
    _, dY = _strided_like(t["dY"], ld, 8, 0.0)
    _, dH = _strided_like(t["dH"], ld, 16, 0.0)
    W = t["W"].cuda()
    _, Y = _strided_like(torch.zeros(M, N, dtype=X.dtype), ld, 0, 0.0)
    _, H = _strided_like(torch.zeros(M, N, dtype=X.dtype), ld, 24, 0.0)
    _, dX = _strided_like(torch.zeros(M, N, dtype=X.dtype), ld, 8, 0.0)
    _, dR = _strided_like(torch.zeros(M, N, dtype=X.dtype), ld + 8, 0, 0.0)
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    _say("strided residual N=%d" % N)
    nl.norm_fwd("rmsnorm", X, R, W, None, w.eps, Y, H, None, rstd,
                nl.workspace("rmsnorm", X.dtype, nl.PASS_FWD, M, N, True))
    dW = torch.empty_like(W)
    nl.norm_bwd("rmsnorm", H, dY, dH, W, None, rstd, w.eps, dX, dR, dW, None,
                nl.workspace("rmsnorm", X.dtype, nl.PASS_BWD, M, N))
    torch.cuda.synchronize()
    bits = {k: inputs.host_bits(t[k]) for k in ("X", "W", "R", "dY", "dH")}
    eps = float(np.float32(w.eps))
    f = oracle.fwd(oracle.RMSNORM, oracle.BF16, bits["X"], bits["W"], None, bits["R"], eps=eps,
                   want_h=True)
    check_h(H.double().cpu().numpy(), f["h"], "bf16")
    check_values("Y", Y.double().cpu().numpy(), f["y"], "bf16")
    hbits = oracle.round_bf16(f["h"])
    g = oracle.bwd(oracle.RMSNORM, oracle.BF16, hbits, bits["dY"], bits["W"], dH=bits["dH"],
                   eps=eps)
    check_values("dX", dX.double().cpu().numpy(), g["dx"], "bf16")
    assert torch.equal(dR, dX)
    check_colsums("dW", dW.double().cpu().numpy(), g["dw"], "bf16")


# ---- pointer alignment sets the access width -------------------------------------------------

# (dtype, weight dtype, shift of every tensor in elements of its own type, expected access bytes)
# A shift of s elements leaves a pointer aligned to s * element size bytes. The plan sees the
# alignment common to all pointers; fp32 weights beside bf16 activations need min(16, 4 E)
# bytes for an access of E elements, so 4-byte alignment leaves them element-wise and 8-byte
# alignment allows two elements per access.
SHIFTS = [("bf16", None, 1, 2), ("bf16", None, 2, 4), ("bf16", None, 4, 8),
          ("f32", None, 1, 4), ("f32", None, 2, 8),
          ("bf16", "f32", 1, 2), ("bf16", "f32", 2, 2), ("bf16", "f32", 4, 4)]


@pytest.mark.parametrize("dt,wdt,shift,width", SHIFTS, ids=lambda v: str(v))
@pytest.mark.parametrize("N", [100, 1000, 4096, 9000])
@pytest.mark.parametrize("unaligned", [0, -1], ids=["narrow", "phase_classes"])
def test_pointer_alignment_sets_width(dt, wdt, shift, width, N, unaligned):
    """Every tensor placed `shift` elements past a 16-byte boundary: without phase classes the
    plan takes the widest access that alignment allows; with them (the default; all tensors at
    one phase) 16-byte accesses over the classes where a team scheme holds the row. The results
    match the oracle either way."""
    with tuned(unaligned=unaligned):
        _pointer_shift_case(dt, wdt, shift, width, N, check_width=unaligned == 0)


def _pointer_shift_case(dt, wdt, shift, width, N, check_width):
    kind = "layernorm"
    w = dataclasses.replace(_small(kind, dt, 61, N, seed=N), wdtype=wdt)
    t = inputs.make(w)

    def shifted(src):
        buf = torch.empty(src.numel() + 16, dtype=src.dtype, device="cuda")
        v = buf[shift:shift + src.numel()].view(src.shape)
        v.copy_(src.to("cuda"))
        return v

    X, W, B, dY = (shifted(t[k]) for k in ("X", "W", "B", "dY"))
    align = X.data_ptr() & -X.data_ptr()
    assert align == shift * X.element_size()
    # row length and alignment together: N = 100 holds 4-element accesses at most
    expect = min(width, (N & -N) * X.element_size())
    if expect < 4:
        expect = X.element_size()
    if check_width:
        assert _access_bytes(kind, dt, wdt, 61, N,
                             align=min(align, W.data_ptr() & -W.data_ptr())) == expect
    _say("pointer shift %d (%s, w=%s) N=%d: %d-byte accesses" % (shift, dt, wdt, N, expect))
    Y = shifted(torch.zeros(61, N, dtype=X.dtype))
    mean = torch.empty(61, dtype=torch.float32, device="cuda")
    rstd = torch.empty(61, dtype=torch.float32, device="cuda")
    ws = nl.workspace(kind, X.dtype, nl.PASS_FWD, 61, N)
    nl.norm_fwd(kind, X, None, W, B, w.eps, Y, None, mean, rstd, ws)
    dX = shifted(torch.zeros(61, N, dtype=X.dtype))
    dW = shifted(torch.zeros(N, dtype=W.dtype))
    dB = shifted(torch.zeros(N, dtype=W.dtype))
    wsb = nl.workspace(kind, X.dtype, nl.PASS_BWD, 61, N)
    nl.norm_bwd(kind, X, dY, None, W, mean, rstd, w.eps, dX, None, dW, dB, wsb)
    bits = {k: inputs.host_bits(t[k]) for k in ("X", "W", "B", "dY")}
    eps = float(np.float32(w.eps))
    code = {"f32": oracle.F32, "bf16": oracle.BF16}[dt] if wdt is None else oracle.BF16_F32W
    f = oracle.fwd(oracle.LAYERNORM, code, bits["X"], bits["W"], bits["B"], eps=eps)
    g = oracle.bwd(oracle.LAYERNORM, code, bits["X"], bits["dY"], bits["W"], eps=eps)
    check_values("Y", Y.double().cpu().numpy(), f["y"], dt)
    check_values("dX", dX.double().cpu().numpy(), g["dx"], dt)
    check_colsums("dW", dW.double().cpu().numpy(), g["dw"], wdt or dt)
    check_colsums("dB", dB.double().cpu().numpy(), g["db"], wdt or dt)

# ---- numerically hard rows ---------------------------------------------------------------------

@pytest.mark.parametrize("N", [512, 4096, 100000])
def test_large_mean_rows_fp32(N):
    """|mean| >> std: a one-pass E[x^2] - mean^2 in fp32 would lose the variance."""
    w = _small("layernorm", "f32", 19, N, seed=N, x=inputs.normal(1000.0, 1.0))
    _say("large mean N=%d" % N)
    run_and_check(w)


@pytest.mark.parametrize("form,flag", SPLIT_FORMS, ids=[f[0] for f in SPLIT_FORMS])
def test_split_hard_rows(form, flag):
    """Long rows on both split forms where the chunk combine does the most work: fp32 rows far
    from zero mean (mean 1000, sd 1), and bf16 rows with 1% of their columns scaled by 20
    (chunks whose variances differ by orders of magnitude)."""
    with tuned(exchange=flag):
        for N in (65536, 262144):
            _say("split hard rows %s N=%d" % (form, N))
            run_and_check(_small("layernorm", "f32", 9, N, seed=N, x=inputs.normal(1000.0, 1.0)))
            for kind in ("layernorm", "rmsnorm"):
                w = dataclasses.replace(_small(kind, "bf16", 33, N, seed=N + 1),
                                        outlier_frac=0.01)
                run_and_check(w)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_outlier_channels(dt):
    w = dataclasses.replace(inputs.rms_hidden(5120, M=512), dtype=dt)
    run_and_check(w)


def test_golden_exact_cases_on_gpu():
    """Hand-derived exact cases: outputs are exactly representable, so the device must
    reproduce them up to its reciprocal-square-root rounding."""
    gold = json.load(open(GOLDEN))
    for c in gold["cases"]:
        for dt, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
            X = torch.tensor(c["X"], dtype=tdt, device="cuda")
            W = torch.tensor(c["W"], dtype=tdt, device="cuda")
            B = torch.tensor(c["B"], dtype=tdt, device="cuda") if c["B"] is not None else None
            dY = torch.tensor(c["dY"], dtype=tdt, device="cuda")
            for scheme in (nl.SCHEME_WAVE, nl.SCHEME_BLOCK, nl.SCHEME_SPLIT):
                with tuned(scheme=scheme):
                    Y, _, mean, rstd = nl.forward(c["kind"], X, W, B, c["eps"])
                    dX, dW, dB = nl.backward(c["kind"], X, dY, W, mean, rstd, c["eps"])
                tol = 1e-6 if dt == "f32" else 2 ** -8
                what = "%s %s scheme %d" % (c["name"], dt, scheme)
                np.testing.assert_allclose(Y.double().cpu().numpy(), c["Y"], rtol=tol, atol=1e-6,
                                           err_msg=what + " Y")
                np.testing.assert_allclose(rstd.double().cpu().numpy(), c["rstd"], rtol=1e-6,
                                           err_msg=what + " rstd")
                np.testing.assert_allclose(dX.double().cpu().numpy(), c["dX"], rtol=tol,
                                           atol=1e-5, err_msg=what + " dX")
                np.testing.assert_allclose(dW.double().cpu().numpy(), c["dW"], rtol=tol,
                                           atol=1e-5, err_msg=what + " dW")
                if c["dB"] is not None:
                    np.testing.assert_allclose(dB.double().cpu().numpy(), c["dB"], rtol=tol,
                                               atol=1e-5, err_msg=what + " dB")


def test_constant_and_zero_rows():
    """Degenerate rows inside a normal batch: a constant LayerNorm row gives Y = B and
    dX = rstd (g - mean(g)); an all-zero RMSNorm row gives Y = 0 and dX = g / sqrt(eps)."""
    for kind in ("layernorm", "rmsnorm"):
        w = _small(kind, "f32", 64, 3000, seed=5)
        t = inputs.make(w)
        t["X"][7] = 2.5 if kind == "layernorm" else 0.0
        t["X"][40] = 0.0
        X = t["X"].cuda()
        W, B, dY = (t[k].cuda() if t[k] is not None else None for k in ("W", "B", "dY"))
        Y, _, mean, rstd = nl.forward(kind, X, W, B, w.eps)
        dX, dW, dB = nl.backward(kind, X, dY, W, mean, rstd, w.eps)
        ok = oracle.LAYERNORM if kind == "layernorm" else oracle.RMSNORM
        bits = {k: inputs.host_bits(t[k]) for k in ("X", "W", "B", "dY")}
        e = float(np.float32(w.eps))
        f = oracle.fwd(ok, oracle.F32, bits["X"], bits["W"], bits["B"], eps=e)
        g = oracle.bwd(ok, oracle.F32, bits["X"], bits["dY"], bits["W"], eps=e)
        check_values("Y", Y.double().cpu().numpy(), f["y"], "f32")
        # a constant or zero LayerNorm row has rstd = 1/sqrt(eps): dX elements near zero are
        # differences of terms ~300x larger, resolved to fp32 ulps of those terms
        fl = dx_floor(torch.arange(64), t["dY"], t["W"], f["rstd"], 3000)
        check_values("dX", dX.double().cpu().numpy(), g["dx"], "f32", floor=fl)
        check_colsums("dW", dW.double().cpu().numpy(), g["dw"], "f32")


# ---- empty input -----------------------------------------------------------------------------

def test_zero_rows():
    for kind in ("layernorm", "rmsnorm"):
        X = torch.empty(0, 4096, dtype=torch.bfloat16, device="cuda")
        W = torch.randn(4096, device="cuda").to(torch.bfloat16)
        Y, _, mean, rstd = nl.forward(kind, X, W, None, 1e-5)
        assert Y.shape == (0, 4096)
        dW = torch.full((4096,), 3.0, dtype=torch.bfloat16, device="cuda")
        dB = torch.full((4096,), 3.0, dtype=torch.bfloat16, device="cuda") \
            if kind == "layernorm" else None
        nl.norm_bwd(kind, X, X, None, W, None, None, 1e-5, X, None, dW, dB, None)
        torch.cuda.synchronize()
        assert (dW.float() == 0).all()
        if dB is not None:
            assert (dB.float() == 0).all()


# ---- determinism --------------------------------------------------------------------------------

@pytest.mark.parametrize("kind,dt,M,N", [("layernorm", "bf16", 4096, 4096),
                                        ("rmsnorm", "bf16", 3000, 1024),
                                        ("layernorm", "bf16", 64, 100000),
                                        ("layernorm", "f16", 17, 262144),
                                        ("rmsnorm", "bf16", 4, 1048576),
                                        ("rmsnorm", "f32", 513, 7168)])
def test_bitwise_deterministic(kind, dt, M, N):
    """No atomics and fixed reduction orders: repeated runs, also on another stream, give the
    same bits."""
    w = _small(kind, dt, M, N, seed=11)
    t = inputs.make(w)
    X, W, B, dY = (t[k].cuda() if t[k] is not None else None for k in ("X", "W", "B", "dY"))
    results = []
    s2 = torch.cuda.Stream()
    for stream in (None, None, s2):
        with torch.cuda.stream(stream) if stream is not None else torch.cuda.stream(
                torch.cuda.current_stream()):
            Y, _, mean, rstd = nl.forward(kind, X, W, B, w.eps)
            dX, dW, dB = nl.backward(kind, X, dY, W, mean, rstd, w.eps)
        torch.cuda.synchronize()
        results.append([a.view(torch.int16) if a is not None and a.dtype == torch.bfloat16
                        else a for a in (Y, rstd, dX, dW, dB)])
    for other in results[1:]:
        for a, b in zip(results[0], other):
            if a is not None:
                assert torch.equal(a, b)


# ---- guard bands -------------------------------------------------------------------------------

@pytest.mark.parametrize("scheme", [nl.SCHEME_AUTO, nl.SCHEME_WAVE, nl.SCHEME_BLOCK,
                                    nl.SCHEME_SPLIT])
@pytest.mark.parametrize("N", [1000, 1032])
def test_guard_bands_untouched(scheme, N):
    """Every buffer sits between 4 KiB guard regions filled with a pattern; no kernel may write
    outside its buffer."""
    if scheme == nl.SCHEME_WAVE and N > 1024:
        pytest.skip("row longer than a wavefront's registers")
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


# ---- workspace and two-stage backward ---------------------------------------------------------

def test_workspace_too_small_is_rejected():
    M, N = 1024, 4096
    X = torch.randn(M, N, device="cuda").to(torch.bfloat16)
    W = torch.ones(N, device="cuda", dtype=torch.bfloat16)
    # what this call's plan needs (norm_workspace_size covers every pointer alignment and can be
    # larger)
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    need = nl.norm_plan("layernorm", torch.bfloat16, nl.PASS_BWD, M, N,
                        cu_count=cu)["workspace_bytes"]
    assert need <= nl.norm_workspace_size("layernorm", torch.bfloat16, nl.PASS_BWD, M, N)
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(nl.NormError) as e:
        nl.norm_bwd("layernorm", X, X, None, W, None, None, 1e-5, torch.empty_like(X), None,
                    torch.empty_like(W), torch.empty_like(W), small)
    assert e.value.status == nl.ERR_WORKSPACE
    with pytest.raises(nl.NormError) as e:
        nl.norm_bwd("layernorm", X, X, None, W, None, None, 1e-5, torch.empty_like(X), None,
                    torch.empty_like(W), torch.empty_like(W), None)
    assert e.value.status == nl.ERR_WORKSPACE


@pytest.mark.parametrize("kind,M,N", [("layernorm", 2048, 4096), ("rmsnorm", 256, 262144),
                                      ("rmsnorm", 4, 1 << 20), ("layernorm", 999, 777),
                                      ("layernorm", 256, 262144), ("layernorm", 17, 262144),
                                      ("rmsnorm", 3, 20000), ("layernorm", 64, 65536)])
def test_two_stage_backward_matches_norm_bwd(kind, M, N):
    w = _small(kind, "bf16", M, N, seed=2)
    t = inputs.make(w)
    X, W, dY = (t[k].cuda() for k in ("X", "W", "dY"))
    Y, _, mean, rstd = nl.forward(kind, X, W, None, w.eps)
    dX1, dW1, dB1 = nl.backward(kind, X, dY, W, mean, rstd, w.eps)
    ws = nl.workspace(kind, X.dtype, nl.PASS_BWD, M, N)
    dX2 = torch.empty_like(X)
    dW2 = torch.empty_like(W)
    dB2 = torch.empty_like(W) if kind == "layernorm" else None
    nl.norm_bwd_fused(kind, X, dY, None, W, mean, rstd, w.eps, dX2, None, ws)
    nl.norm_bwd_reduce(kind, M, N, dW2, dB2, ws)
    torch.cuda.synchronize()
    assert torch.equal(dX1.view(torch.int16), dX2.view(torch.int16))
    # the split scheme's single-group shortcut sums in the same order as the reduce stage
    assert torch.equal(dW1.view(torch.int16), dW2.view(torch.int16))
    if dB1 is not None:
        assert torch.equal(dB1.view(torch.int16), dB2.view(torch.int16))


@pytest.mark.parametrize("dt,wdt", [("bf16", None), ("f32", None), ("f16", None),
                                    ("bf16", "f32")])
@pytest.mark.parametrize("kind", ["layernorm", "rmsnorm"])
def test_split_row_group_counts(kind, dt, wdt):
    """The single-pass split backward with 2, 3, 7, 16, 32 and 33 row groups (each writes a
    partial row of column sums that the reduction pass adds): norm_bwd matches the oracle and
    gives the same bits as the two-stage calls; ragged last chunks, rows per group uneven."""
    for N in (20000, 65536, 8192 * 5 + 8):
        for M, groups in ((40, 2), (40, 3), (45, 7), (80, 16), (64, 32), (70, 33)):
            _say("split row groups %s %s/%s %dx%d groups %d" % (kind, dt, wdt, M, N, groups))
            w = dataclasses.replace(_small(kind, dt, M, N, seed=M + N + groups), wdtype=wdt)
            with tuned(exchange=1, row_groups=groups):
                p = nl.norm_plan(kind, inputs.TORCH_DTYPES[dt], nl.PASS_BWD, M, N,
                                 cu_count=torch.cuda.get_device_properties(0).multi_processor_count)
                if p["exchange_row_groups"] == 0:
                    continue  # this width runs two passes
                out = run_and_check(w)
                X = inputs.make(w)["X"].cuda()
                t = inputs.make(w)
                W, dY = t["W"].cuda(), t["dY"].cuda()
                ws = nl.workspace(kind, X.dtype, nl.PASS_BWD, M, N)
                dX2, dW2 = torch.empty_like(X), torch.empty_like(W)
                dB2 = torch.empty_like(W) if kind == "layernorm" else None
                nl.norm_bwd_fused(kind, X, dY, None, W, out["mean"], out["rstd"], w.eps, dX2,
                                  None, ws)
                nl.norm_bwd_reduce(kind, M, N, dW2, dB2, ws)
                torch.cuda.synchronize()
                bits = (lambda v: v.view(torch.int16) if v.element_size() == 2 else v)
                assert torch.equal(bits(out["dX"]), bits(dX2))
                assert torch.equal(bits(out["dW"]), bits(dW2))
                if dB2 is not None:
                    assert torch.equal(bits(out["dB"]), bits(dB2))
                assert nl.norm_workspace_status(out["ws"]) == nl.OK


def test_reduce_on_a_foreign_workspace_gives_nan():
    """The reduce stage reads the partial count from the header the fused pass wrote; on a
    workspace that holds no such header it writes NaN rather than reading past the partials."""
    N = 4096
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    dW = torch.zeros(N, dtype=torch.bfloat16, device="cuda")
    nl.norm_bwd_reduce("rmsnorm", 100, N, dW, None, ws)
    torch.cuda.synchronize()
    assert torch.isnan(dW.float()).all()


def test_binding_checks_tensors():
    """The Python binding refuses tensors the C ABI cannot check (wrong dtype, shape, device,
    columns not contiguous) before calling the library, and passes row-strided views with their
    strides."""
    _say("binding checks")
    M, N = 64, 1024
    w = _small("layernorm", "bf16", M, N, seed=5)
    t = inputs.make(w)
    X, W, B = (t[k].cuda() for k in ("X", "W", "B"))
    Y = torch.empty_like(X)
    bad_y = [torch.empty(M, N, dtype=torch.float16, device="cuda"),       # dtype
             torch.empty(M, N + 1, dtype=torch.bfloat16, device="cuda"),  # shape
             torch.empty(M, N, dtype=torch.bfloat16),                     # host memory
             torch.empty(N, M, dtype=torch.bfloat16, device="cuda").t()]  # columns strided
    for y in bad_y:
        with pytest.raises(ValueError):
            nl.norm_fwd("layernorm", X, None, W, B, w.eps, y)
    with pytest.raises(ValueError):
        nl.norm_fwd("layernorm", X, None, W[:-1], B, w.eps, Y)
    # row-strided views: the slices of a wider buffer
    big = torch.zeros(M, 3 * N, dtype=torch.bfloat16, device="cuda")
    big[:, N:2 * N] = X
    out = torch.full((M, 2 * N), 7.0, dtype=torch.bfloat16, device="cuda")
    nl.norm_fwd("layernorm", big[:, N:2 * N], None, W, B, w.eps, out[:, :N])
    nl.norm_fwd("layernorm", X, None, W, B, w.eps, Y)
    torch.cuda.synchronize()
    assert torch.equal(out[:, :N].view(torch.int16), Y.view(torch.int16))
    assert (out[:, N:] == 7.0).all()
