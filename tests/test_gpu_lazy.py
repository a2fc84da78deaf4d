"""The norm deferred into a following projection (norm_fold_projection, norm_lazy_linear)
against the oracle's Norm(X) L^T + c, through the C ABI.

The oracle evaluates the definition (the norm row in float64, then the dot products); the
device evaluates rstd * (X G^T - mean * s) + t with G = bf16(L * gamma) on the matrix cores.
The tolerance is the error bound of that arithmetic (tests/parity.py, norm_linear_bound).
Shapes span several 256 x 256 output tiles with ragged edges in M, Nout and K (K = 200 and
K = 520 end in a partial 64-wide step)."""
import numpy as np
import pytest
import torch

import oracle
from deep_learning_normalization_amd import inputs, normlib as nl
from tests import parity

pytestmark = pytest.mark.gpu

ORC = {"layernorm": oracle.LAYERNORM, "rmsnorm": oracle.RMSNORM}


def _say(msg):
    print("[gpu] " + msg, flush=True)


def _rng(seed):
    return torch.Generator().manual_seed(seed)


def _case(kind, M, K, Nout, seed, wdt=torch.bfloat16, shift=0.4, scale=1.3, bias=True):
    X = (torch.randn(M, K, generator=_rng(seed)) * scale + shift).to(torch.bfloat16)
    g = (torch.randn(K, generator=_rng(seed + 1)) * 0.1 + 1.0).to(wdt)
    b = ((torch.randn(K, generator=_rng(seed + 2)) * 0.1).to(wdt)
         if kind == "layernorm" else None)
    L = (torch.randn(Nout, K, generator=_rng(seed + 3)) * K ** -0.5).to(torch.bfloat16)
    c = (torch.randn(Nout, generator=_rng(seed + 4)) * 0.1).float() if bias else None
    return X, g, b, L, c


def _odt(wdt):
    return oracle.BF16 if wdt == torch.bfloat16 else oracle.BF16_F32W


def _reference(kind, X, g, b, L, c, eps, rows):
    """Oracle rows and their error bound."""
    hb = inputs.host_bits
    rows = np.asarray(rows)
    ref, xs = [], []
    # contiguous runs of rows in one oracle call each
    starts = np.flatnonzero(np.diff(rows, prepend=rows[0] - 2) != 1)
    ends = np.append(starts[1:], len(rows))
    Xb = hb(X)
    for s0, e0 in zip(starts, ends):
        r0, r1 = int(rows[s0]), int(rows[e0 - 1]) + 1
        ref.append(oracle.norm_linear(ORC[kind], _odt(g.dtype), Xb, hb(g), hb(b), hb(L),
                                      None if c is None else c.numpy(), eps=eps, rows=(r0, r1)))
    ref = np.concatenate(ref, axis=0)
    xd = X[torch.from_numpy(rows)].double().numpy()
    return ref, xd


def _run(kind, X, g, b, L, c, eps, mode, dev="cuda", ld_pad=0):
    """Fold, then the product; mode 'formed' (statistics from the X tiles) or 'given' (from
    norm_stats). ld_pad > 0 runs X, G and Y as row slices of wider buffers."""
    M, K = X.shape
    Nout = L.shape[0]
    Xd, gd_, Ld = X.to(dev), g.to(dev), L.to(dev)
    bd_ = b.to(dev) if b is not None else None
    cd = c.to(dev) if c is not None else None
    if ld_pad:
        Xw = torch.full((M, K + ld_pad), float("nan"), dtype=torch.bfloat16, device=dev)
        Xw[:, :K] = Xd
        Xd = Xw[:, :K]
        Gw = torch.full((Nout, K + ld_pad), float("nan"), dtype=torch.bfloat16, device=dev)
        G = Gw[:, :K]
    else:
        G = torch.empty_like(Ld)
    ln = kind == "layernorm"
    s = torch.empty(Nout, device=dev) if ln else None
    t = torch.empty(Nout, device=dev) if (bd_ is not None or cd is not None) else None
    nl.norm_fold_projection(kind, Ld, gd_, bd_, cd, G, s, t)
    Yw = torch.full((M, Nout + 2 * ld_pad), float("nan"), dtype=torch.bfloat16, device=dev)
    Y = Yw[:, :Nout]
    mean = torch.empty(M, device=dev) if ln else None
    rstd = torch.empty(M, device=dev)
    if mode == "given":
        ws = nl.workspace(kind, torch.bfloat16, nl.PASS_FWD, M, K)
        nl.norm_stats(kind, Xd, None, eps, None, mean, rstd, ws)
        nl.norm_lazy_linear(kind, Xd, eps, G, s, t, Y, mean_in=mean, rstd_in=rstd)
    else:
        nl.norm_lazy_linear(kind, Xd, eps, G, s, t, Y, mean_out=mean, rstd_out=rstd)
    torch.cuda.synchronize()
    if ld_pad:
        assert torch.isnan(Yw[:, Nout:].float()).all(), "columns beyond Y's rows were written"
    return Y, mean, rstd, (G, s, t)


def _bits(Y, rows=None):
    Y = Y.cpu() if rows is None else Y[torch.from_numpy(np.asarray(rows)).to(Y.device)].cpu()
    return inputs.host_bits(Y.contiguous())


SHAPES = [(1, 8, 1), (5, 64, 7), (130, 200, 129), (257, 512, 300), (64, 4096, 256),
          (600, 520, 530), (768, 128, 772)]


@pytest.mark.parametrize("M,K,Nout", SHAPES, ids=lambda v: str(v))
@pytest.mark.parametrize("mode", ["formed", "given"])
@pytest.mark.parametrize("kind", ["layernorm", "rmsnorm"])
def test_lazy_linear_vs_oracle(kind, mode, M, K, Nout):
    _say("lazy %s %s M=%d K=%d Nout=%d" % (kind, mode, M, K, Nout))
    eps = 1e-5
    X, g, b, L, c = _case(kind, M, K, Nout, seed=M * 7 + K)
    Y, mean, rstd, _ = _run(kind, X, g, b, L, c, eps, mode)
    rows = np.arange(M)
    ref, xd = _reference(kind, X, g, b, L, c, eps, rows)
    x0 = xd[:, 0] if (mode == "formed" and kind == "layernorm") else None
    bound = parity.norm_linear_bound(ORC[kind], xd, g.double().numpy(),
                                     None if b is None else b.double().numpy(),
                                     L.double().numpy(), None if c is None else c.numpy(), eps,
                                     x0)
    parity.check_norm_linear("Y", _bits(Y), ref, bound)
    if mode == "formed":
        st = oracle.fwd(ORC[kind], oracle.BF16, inputs.host_bits(X), inputs.host_bits(g),
                        inputs.host_bits(b), eps=eps)
        r = st["rstd"]
        tol = 4 * (K / 8 + 8) * 2.0 ** -24 * (1 + ((xd[:, 0] - st["mean"]) * r) ** 2)
        if kind == "rmsnorm":
            tol = np.full(M, 4 * (K / 8 + 8) * 2.0 ** -24)
        got_r = rstd.cpu().double().numpy()
        assert (np.abs(got_r - r) <= tol * r).all(), "formed rstd"
        if mean is not None:
            got_m = mean.cpu().double().numpy()
            assert (np.abs(got_m - st["mean"]) <= tol * (np.abs(st["mean"]) + 1 / r)).all()


@pytest.mark.parametrize("kind", ["layernorm", "rmsnorm"])
def test_lazy_linear_fp32_gamma_and_no_bias(kind):
    _say("lazy %s fp32 gamma" % kind)
    eps = 1e-5
    X, g, b, L, _ = _case(kind, 200, 320, 136, seed=31, wdt=torch.float32, bias=False)
    for mode in ("formed", "given"):
        Y, _, _, _ = _run(kind, X, g, b, L, None, eps, mode)
        rows = np.arange(200)
        ref, xd = _reference(kind, X, g, b, L, None, eps, rows)
        bound = parity.norm_linear_bound(ORC[kind], xd, g.double().numpy(),
                                         None if b is None else b.double().numpy(),
                                         L.double().numpy(), None, eps,
                                         xd[:, 0] if kind == "layernorm" else None)
        parity.check_norm_linear("Y " + mode, _bits(Y), ref, bound)


@pytest.mark.parametrize("mode", ["formed", "given"])
def test_lazy_linear_large_mean_rows(mode):
    """Rows far from zero mean (mean 64, sd 1): the mean correction cancels most of X G^T."""
    _say("lazy large mean %s" % mode)
    eps = 1e-5
    X, g, b, L, c = _case("layernorm", 136, 256, 72, seed=77, shift=64.0, scale=1.0)
    Y, _, _, _ = _run("layernorm", X, g, b, L, c, eps, mode)
    ref, xd = _reference("layernorm", X, g, b, L, c, eps, np.arange(136))
    bound = parity.norm_linear_bound(ORC["layernorm"], xd, g.double().numpy(),
                                     b.double().numpy(), L.double().numpy(), c.numpy(), eps,
                                     xd[:, 0] if mode == "formed" else None)
    parity.check_norm_linear("Y", _bits(Y), ref, bound)


def test_lazy_linear_row_strided():
    _say("lazy row strided")
    eps = 1e-5
    X, g, b, L, c = _case("layernorm", 150, 192, 140, seed=5)
    Y, _, _, _ = _run("layernorm", X, g, b, L, c, eps, "formed", ld_pad=24)
    Y0, _, _, _ = _run("layernorm", X, g, b, L, c, eps, "formed")
    assert torch.equal(Y.contiguous(), Y0), "strided and contiguous results differ"
    ref, xd = _reference("layernorm", X, g, b, L, c, eps, np.arange(150))
    bound = parity.norm_linear_bound(ORC["layernorm"], xd, g.double().numpy(),
                                     b.double().numpy(), L.double().numpy(), c.numpy(), eps,
                                     xd[:, 0])
    parity.check_norm_linear("Y", _bits(Y), ref, bound)


def test_fold_projection_values():
    """G is bf16(L * gamma) exactly (the fp32 product, rounded to nearest even, as torch's CPU
    conversion does it); s and t are within an fp32 sum's bound of their float64 values."""
    _say("fold values")
    for wdt in (torch.bfloat16, torch.float32):
        X, g, b, L, c = _case("layernorm", 1, 1000, 67, seed=3, wdt=wdt)
        _, _, _, (G, s, t) = _run("layernorm", X, g, b, L, c, 1e-5, "given")
        want_G = (L.float() * g.float()).to(torch.bfloat16)
        assert torch.equal(G.cpu(), want_G)
        Gd = want_G.double()
        gK = (1000 + 8) * 2.0 ** -23
        assert (np.abs(s.cpu().double().numpy() - Gd.sum(1).numpy())
                <= gK * Gd.abs().sum(1).numpy()).all()
        want_t = L.double() @ b.double() + c.double()
        bt = gK * (L.double().abs() @ b.double().abs()) + 2.0 ** -23 * c.double().abs()
        assert (np.abs(t.cpu().double() - want_t) <= bt).all().item()


def test_lazy_linear_deterministic():
    _say("lazy determinism")
    X, g, b, L, c = _case("layernorm", 300, 512, 260, seed=9)
    Y1, m1, r1, _ = _run("layernorm", X, g, b, L, c, 1e-5, "formed")
    Y2, m2, r2, _ = _run("layernorm", X, g, b, L, c, 1e-5, "formed")
    assert torch.equal(Y1, Y2) and torch.equal(m1, m2) and torch.equal(r1, r2)


def test_lazy_linear_zero_rows():
    X, g, b, L, c = _case("layernorm", 1, 64, 8, seed=1)
    G, s, t = nl.fold_projection("layernorm", L.cuda(), g.cuda(), b.cuda(), c.cuda())
    Y = torch.empty(0, 8, dtype=torch.bfloat16, device="cuda")
    nl.norm_lazy_linear("layernorm", X.cuda()[:0], 1e-5, G, s, t, Y)
    torch.cuda.synchronize()


@pytest.mark.parametrize("proj", [inputs.LN_LINEAR_BF16_16384x4096x4096,
                                  inputs.RMS_LINEAR_BF16_16384x4096x4096],
                         ids=lambda p: p.name)
def test_lazy_linear_full_size(proj):
    """The full-size projections in the configuration the benchmark times, on sampled rows
    (first, last, the tile edges 255/256 and 8191/8192, and random ones) against the
    oracle. Rows are sampled because every row would cost the double-precision oracle
    2 * 16384 * 4096 * 4096 = 550 G multiply-adds in plain loops (many minutes on the host);
    the smaller projection tests compare every row."""
    w = proj.norm
    _say("lazy full size %s" % proj.name)
    t = inputs.make(w)
    p = inputs.make_projection(proj)
    X, g, b = t["X"], t["W"], t["B"]
    L, c = p["L"], p["c"]
    rows = sorted(set(parity.sample_rows(w.M, k=16, seed=4).tolist()) | {255, 256, 8191, 8192})
    for mode in ("formed", "given"):
        Y, _, _, _ = _run(w.kind, X, g, b, L, c, w.eps, mode)
        ref, xd = _reference(w.kind, X, g, b, L, c, w.eps, rows)
        bound = parity.norm_linear_bound(ORC[w.kind], xd, g.double().numpy(),
                                         None if b is None else b.double().numpy(),
                                         L.double().numpy(), None if c is None else c.numpy(),
                                         w.eps,
                                         xd[:, 0] if (mode == "formed" and w.kind == "layernorm")
                                         else None)
        parity.check_norm_linear("Y %s" % mode, _bits(Y, rows), ref, bound)
        del Y
