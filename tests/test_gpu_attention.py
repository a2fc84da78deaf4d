"""Attention over normalised queries and keys (norm_attention_fwd) against the fp64 oracle.

Page "Towards Free Normalization: Fusing Normalization into GEMM and Attention Kernels"
(brifing.si), item 5: norms fused around an attention kernel, read as the norm of every query
and key vector along the head dimension (QK-norm).

Tolerances. With a norm, the kernel folds the key gamma into each normalised query and rounds
that once to bf16 (relative error up to 2^-9 per element); the keys enter the product exactly
and their statistics scale the scores in fp32. The rounding moves each logit by a few 1e-3 at
the logit spread of these inputs (gammas near 1.5); the softmax weights enter the second product
as bf16, and O is rounded to bf16, which alone moves an output by up to 2^-9 |O|. So every bound
has a part relative to |O| for that rounding: |err| <= a + 2^-8 |O_ref| per element, mean |err|
<= m + 2^-9 mean |O_ref|. An emulation of exactly those rounding steps in torch against the
oracle, over every shape below, gives a <= 0.014 and m <= 0.00041 with RMSNorm, a <= 0.0021
and m <= 1e-5 without a norm (the inputs are exact then), and lse errors up to 0.017 (mean
0.0030) with RMSNorm, 6e-7 without. The bounds are about 1.8x the largest and 3x the mean of
those. LayerNorm's deferred form also rounds the centred keys to bf16 (emulated a <= 0.023,
m <= 0.00081, lse <= 0.024), and the key pass and the two-pass form (norms stored in bf16,
then the attention) round the normalised queries and keys separately (emulated a <= 0.031,
m <= 0.00076, lse <= 0.020); those are held to TWO_PASS_TOL.
"""
import numpy as np
import pytest
import torch

import oracle
from deep_learning_normalization_amd import inputs
from deep_learning_normalization_amd import normlib as nl
from tests.parity import tuned

pytestmark = pytest.mark.gpu

TOL = {  # kind: (a, m, lse max, lse mean) in the bounds above
    "rmsnorm": (0.025, 0.0012, 0.03, 0.009),
    "layernorm": (0.025, 0.0012, 0.03, 0.009),
    "none": (0.004, 0.0002, 1e-3, 1e-4),
}
# the key pass and the two-pass form round the normalised queries and keys separately
TWO_PASS_TOL = (0.05, 0.0025, 0.035, 0.014)
OKIND = {"rmsnorm": oracle.RMSNORM, "layernorm": oracle.LAYERNORM, "none": oracle.NO_NORM}
DEV = "cuda:0"


def _run(a, t, packed=False, want_lse=True, key_pass=False):
    """Device O (and lse) for workload a with CPU tensors t. packed: Q, K, V as slices of one
    [B, S, (Hq + 2 Hk) D] tensor, O a slice of a wider buffer (token strides above the heads).
    key_pass: with a workspace, the keys normalised by a pass of their own (forced); else the
    key norm deferred into the attention kernel (no workspace)."""
    print("attention case %s kind %s causal %d packed %d key pass %d" % (
        a.name, a.kind, a.causal, packed, key_pass), flush=True)
    if packed:
        hd = (a.Hq + 2 * a.Hk) * a.D
        qkv = torch.cat([t["Q"].reshape(a.B, a.S, -1), t["K"].reshape(a.B, a.S, -1),
                         t["V"].reshape(a.B, a.S, -1)], dim=2).to(DEV)
        assert qkv.shape[2] == hd
        Q = qkv[:, :, :a.Hq * a.D].view(a.B, a.S, a.Hq, a.D)
        K = qkv[:, :, a.Hq * a.D:(a.Hq + a.Hk) * a.D].view(a.B, a.S, a.Hk, a.D)
        V = qkv[:, :, (a.Hq + a.Hk) * a.D:].view(a.B, a.S, a.Hk, a.D)
        obuf = torch.full((a.B, a.S, a.Hq * a.D + 64), 7.0, dtype=torch.bfloat16, device=DEV)
        O = obuf[:, :, :a.Hq * a.D].view(a.B, a.S, a.Hq, a.D)
    else:
        Q, K, V = (t[n].to(DEV) for n in ("Q", "K", "V"))
        obuf = None
        O = torch.empty_like(Q)
    vec = {n: (t[n].to(DEV) if t[n] is not None else None) for n in ("wq", "bq", "wk", "bk")}
    lse = (torch.empty(a.B, a.Hq, a.S, dtype=torch.float32, device=DEV) if want_lse else None)
    ws = (torch.empty(nl.attention_workspace_bytes(a.B, a.S, a.Hk, a.D), dtype=torch.uint8,
                      device=DEV) if key_pass else None)
    with tuned(attn_key_pass=1 if key_pass else -1):
        nl.norm_attention_fwd(a.kind, Q, K, V, vec["wq"], vec["bq"], vec["wk"], vec["bk"],
                              a.eps, a.D ** -0.5, O, lse, a.causal, workspace=ws)
    torch.cuda.synchronize()
    if obuf is not None:  # the padding past the heads is untouched
        assert bool((obuf[:, :, a.Hq * a.D:] == 7.0).all())
    return O.float().cpu(), (lse.cpu() if lse is not None else None)


def _oracle(a, t, b, h, rows=None):
    hb = inputs.host_bits
    return oracle.norm_attention(OKIND[a.kind], hb(t["Q"]), hb(t["K"]), hb(t["V"]),
                                 hb(t["wq"]), hb(t["bq"]), hb(t["wk"]), hb(t["bk"]), eps=a.eps,
                                 scale=a.D ** -0.5, causal=a.causal, b=b, h=h, rows=rows)


def _compare(a, O, lse, pairs, rows=None, tol=None):
    """O and lse of the (b, h) pairs over query rows [r0, r1) against the oracle, within TOL."""
    omax, omean, lmax, lmean = tol or TOL[a.kind]
    errs, refs, lerrs = [], [], []
    r0, r1 = (0, a.S) if rows is None else rows
    for b, h in pairs:
        Oref, lref = _oracle(a, t_cache[a.name], b, h, (r0, r1))
        got = O[b, r0:r1, h].double().numpy()
        assert np.isfinite(got).all(), "non-finite output (b %d h %d)" % (b, h)
        e = np.abs(got - Oref)
        errs.append(e)
        refs.append(np.abs(Oref))
        if lse is not None:
            lerrs.append(np.abs(lse[b, h, r0:r1].double().numpy() - lref))
        excess = e - (omax + 2.0 ** -8 * np.abs(Oref))
        k = np.unravel_index(np.argmax(excess), e.shape)
        assert excess[k] <= 0, "%s b %d h %d: O error %.4g at row %d dim %d (got %r want %r)" % (
            a.name, b, h, e[k], r0 + k[0], k[1], got[k], Oref[k])
    e = np.concatenate([x.ravel() for x in errs])
    ref = np.concatenate([x.ravel() for x in refs])
    assert e.mean() <= omean + 2.0 ** -9 * ref.mean(), "%s: mean O error %.4g (mean |O| %.3g)" % (
        a.name, e.mean(), ref.mean())
    if lerrs:
        le = np.concatenate(lerrs)
        assert le.max() <= lmax and le.mean() <= lmean, "%s: lse error max %.4g mean %.4g" % (
            a.name, le.max(), le.mean())


t_cache = {}


def _case(a):
    if a.name not in t_cache:
        t_cache.clear()
        t_cache[a.name] = inputs.make_attention(a)
    return t_cache[a.name]


BASE = inputs.Attention("attn", "rmsnorm", 1, 1, 1, 1, seed=5)
# (B, S, Hq, Hk): one token; ragged tiles (7, 65, 300: tails of the 64-key tile and of the
# 256-query block); exactly one block (256); several blocks with grouped heads (513, 4 over 2);
# a grid whose size is a multiple of 8 (the XCD renumbering) and one that is not.
SHAPES = [(1, 1, 1, 1), (1, 7, 2, 1), (2, 65, 2, 2), (1, 256, 4, 1), (1, 300, 3, 3),
          (2, 513, 4, 2), (1, 1100, 8, 2)]


@pytest.mark.parametrize("kind,key_pass", [("rmsnorm", False), ("layernorm", False),
                                           ("rmsnorm", True), ("layernorm", True),
                                           ("none", False)],
                         ids=["rms-deferred", "ln-deferred", "rms-keypass", "ln-keypass", "none"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_attention_matches_oracle(kind, key_pass, causal, shape):
    Bn, S, Hq, Hk = shape
    a = BASE.with_shape(Bn, S, Hq, Hk, kind=kind, causal=causal,
                        name="attn_%s_%d_%s" % (kind, causal, "x".join(map(str, shape))))
    t = _case(a)
    O, lse = _run(a, t, key_pass=key_pass)
    _compare(a, O, lse, [(b, h) for b in range(Bn) for h in range(Hq)],
             tol=TWO_PASS_TOL if (key_pass or kind == "layernorm") else None)


@pytest.mark.parametrize("key_pass", [False, True], ids=["deferred", "keypass"])
@pytest.mark.parametrize("kind", ["rmsnorm", "layernorm"])
def test_attention_packed_qkv(kind, key_pass):
    """Q, K and V as slices of one packed projection output, O inside a wider buffer."""
    a = BASE.with_shape(2, 333, 4, 2, kind=kind, causal=True, name="attn_packed_" + kind)
    t = _case(a)
    O, lse = _run(a, t, packed=True, key_pass=key_pass)
    _compare(a, O, lse, [(b, h) for b in range(2) for h in range(4)],
             tol=TWO_PASS_TOL if (key_pass or kind == "layernorm") else None)


@pytest.mark.parametrize("key_pass", [False, True], ids=["deferred", "keypass"])
def test_layernorm_without_betas(key_pass):
    a = BASE.with_shape(1, 200, 2, 1, kind="layernorm", causal=False, name="attn_ln_nobeta")
    t = dict(_case(a))
    t["bq"] = t["bk"] = None
    t_cache[a.name] = t
    O, lse = _run(a, t, key_pass=key_pass)
    _compare(a, O, lse, [(0, 0), (0, 1)], tol=TWO_PASS_TOL)


def test_fused_matches_two_pass():
    """The fused call against the same computation in two passes: norm_fwd on the query and
    key vectors (rows of D), then the attention without a norm. Both are held to the oracle.
    With the key pass the fused call rounds the normalised queries and keys as the two-pass
    form does, so the two agree but for the odd rounding a different summation order flips."""
    a = BASE.with_shape(2, 777, 4, 2, kind="rmsnorm", causal=True, name="attn_two_pass")
    t = _case(a)
    Q, K, V = (t[n].to(DEV) for n in ("Q", "K", "V"))
    wq, wk = t["wq"].to(DEV), t["wk"].to(DEV)
    O1, l1 = nl.attention("rmsnorm", Q, K, V, wq, None, wk, None, a.eps, causal=True,
                          want_lse=True, key_pass=False)
    with tuned(attn_key_pass=1):
        O3 = nl.attention("rmsnorm", Q, K, V, wq, None, wk, None, a.eps, causal=True)
    Qn = nl.forward("rmsnorm", Q.reshape(-1, a.D), wq, None, a.eps)[0].view_as(Q)
    Kn = nl.forward("rmsnorm", K.reshape(-1, a.D), wk, None, a.eps)[0].view_as(K)
    O2 = nl.attention("rmsnorm", Qn, Kn, V, causal=True)
    torch.cuda.synchronize()
    pairs = [(b, h) for b in range(2) for h in range(4)]
    _compare(a, O1.float().cpu(), l1.cpu(), pairs)
    _compare(a, O2.float().cpu(), None, pairs, tol=TWO_PASS_TOL)
    _compare(a, O3.float().cpu(), None, pairs, tol=TWO_PASS_TOL)
    d = (O3.float() - O2.float()).abs()
    assert d.max().item() <= 0.02 and d.mean().item() <= 1e-4, (d.max().item(), d.mean().item())


def test_attention_deterministic():
    a = BASE.with_shape(1, 600, 4, 1, kind="layernorm", causal=True, name="attn_det")
    t = _case(a)
    O1, l1 = _run(a, t)
    O2, l2 = _run(a, t)
    assert torch.equal(O1, O2) and torch.equal(l1, l2)


def test_attention_unsupported_head_size():
    Q = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(nl.NormError):
        nl.attention("none", Q, Q, Q)


@pytest.mark.slow
@pytest.mark.parametrize("key_pass", [False, True], ids=["deferred", "keypass"])
def test_attention_full_size(key_pass):
    """The 2 x 4096-token, 32-over-8-head RMSNorm causal layer in the launch configuration the
    benchmark times (with a workspace each key is read by 64 (query block, head) pairs, so the
    key pass runs by default): every output finite, and sampled queries (the first and last 64
    tokens and 64 in the middle, of 6 (batch, head) pairs spread over the key/value groups)
    against the oracle."""
    a = inputs.ATTN_QKNORM_B2_S4096
    t = _case(a)
    O, lse = _run(a, t, key_pass=key_pass)
    assert bool(torch.isfinite(O).all()) and bool(torch.isfinite(lse).all())
    pairs = [(0, 0), (0, 5), (0, 31), (1, 8), (1, 17), (1, 30)]
    for rows in ((0, 64), (2016, 2080), (a.S - 64, a.S)):
        _compare(a, O, lse, pairs, rows, tol=TWO_PASS_TOL if key_pass else None)
