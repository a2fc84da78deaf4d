"""Seeded synthetic inputs for the norm workloads.

This module only draws random numbers and casts them; it holds none of the normalisation
arithmetic. The device path and the CPU oracle both receive exactly the tensors made here
(sampled in fp32 on the CPU, then cast to the storage dtype with round-to-nearest-even).

Every tensor has its own generator, seeded with ``seed + offset``:
X 0, W 1, B 2, dY 3, R 4, outlier-channel permutation 5, dH 6, projection L 7, its bias c 8;
attention Q 10, K 11, V 12, query gamma 13 and beta 14, key gamma 15 and beta 16.

The pages print no data set for these kernels; the shapes follow the workloads they discuss
(LLM hidden sizes, and the very-large-row regression class named on the page "PyTorch atinge
desempenho SOTA em normalização com torch.compile", para. 6). Distributions N(a, b) use b as
the standard deviation.
"""
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np
import torch

OFF_X, OFF_W, OFF_B, OFF_DY, OFF_R, OFF_PERM, OFF_DH, OFF_L, OFF_C = 0, 1, 2, 3, 4, 5, 6, 7, 8
OFF_Q, OFF_K, OFF_V, OFF_WQ, OFF_BQ, OFF_WK, OFF_BK = 10, 11, 12, 13, 14, 15, 16

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclass(frozen=True)
class Dist:
    """A value distribution: ("normal", mean, std), ("uniform", lo, hi) or ("const", v)."""
    kind: str
    a: float = 0.0
    b: float = 1.0


def normal(mean, std):
    return Dist("normal", mean, std)


def uniform(lo, hi):
    return Dist("uniform", lo, hi)


def const(v):
    return Dist("const", v)


@dataclass(frozen=True)
class Workload:
    """One synthetic problem: kind ("layernorm"/"rmsnorm"), dtype ("f32"/"bf16"), shape,
    eps, distributions, and which passes and options it exercises."""
    name: str
    kind: str
    dtype: str
    M: int
    N: int
    eps: float
    x: Dist = normal(0.0, 1.0)
    w: Dist = normal(1.0, 0.1)
    b: Optional[Dist] = None          # LayerNorm bias; None means no bias tensor
    dy: Optional[Dist] = normal(0.0, 1.0)  # None: forward only
    r: Optional[Dist] = None          # residual input R (residual variant)
    dh: Optional[Dist] = None         # incoming gradient of the residual output
    wdtype: Optional[str] = None      # storage of W, B (and dW, dB); None: the same as dtype
    outlier_frac: float = 0.0         # fraction of columns scaled by outlier_scale
    outlier_scale: float = 20.0
    seed: int = 0
    tags: Tuple[str, ...] = field(default_factory=tuple)

    def with_shape(self, M, N, name=None):
        return replace(self, M=M, N=N, name=name or "%s[%dx%d]" % (self.name, M, N))


def _draw(dist: Dist, shape, seed: int) -> torch.Tensor:
    g = torch.Generator().manual_seed(int(seed))
    n = int(np.prod(shape)) if len(shape) else 1
    if dist.kind == "normal":
        t = torch.randn(n, generator=g, dtype=torch.float32)
        if dist.b != 1.0:
            t.mul_(dist.b)
        if dist.a != 0.0:
            t.add_(dist.a)
    elif dist.kind == "uniform":
        t = torch.empty(n, dtype=torch.float32).uniform_(dist.a, dist.b, generator=g)
    elif dist.kind == "const":
        t = torch.full((n,), float(dist.a), dtype=torch.float32)
    else:
        raise ValueError("unknown distribution %r" % (dist.kind,))
    return t.view(*shape)


def outlier_columns(N: int, frac: float, seed: int) -> torch.Tensor:
    """round(frac * N) distinct column indices from a seeded permutation (outlier channels)."""
    k = int(round(frac * N))
    g = torch.Generator().manual_seed(int(seed) + OFF_PERM)
    return torch.randperm(N, generator=g)[:k]


def make(w: Workload, M: Optional[int] = None) -> dict:
    """CPU tensors for a workload, in its storage dtype.

    Keys: X, W, B (None if absent), dY (None if forward-only), R (None unless residual),
    dH (None unless given). ``M`` overrides the row count (rows are drawn from the same
    streams, so the first rows match the full-size tensors only when M equals w.M).
    """
    M = w.M if M is None else M
    N = w.N
    dt = TORCH_DTYPES[w.dtype]
    wdt = TORCH_DTYPES[w.wdtype or w.dtype]
    s = w.seed
    X = _draw(w.x, (M, N), s + OFF_X)
    if w.outlier_frac > 0.0:
        cols = outlier_columns(N, w.outlier_frac, s)
        X[:, cols] *= w.outlier_scale
    out = {
        "X": X.to(dt),
        "W": _draw(w.w, (N,), s + OFF_W).to(wdt),
        "B": _draw(w.b, (N,), s + OFF_B).to(wdt) if w.b is not None else None,
        "dY": _draw(w.dy, (M, N), s + OFF_DY).to(dt) if w.dy is not None else None,
        "R": _draw(w.r, (M, N), s + OFF_R).to(dt) if w.r is not None else None,
        "dH": _draw(w.dh, (M, N), s + OFF_DH).to(dt) if w.dh is not None else None,
    }
    return out


def host_bits(t: Optional[torch.Tensor]):
    """The raw storage bits of a CPU tensor as numpy: uint16 for bf16 and fp16, float32 for
    fp32."""
    if t is None:
        return None
    t = t.detach().contiguous().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError("unsupported dtype %s" % t.dtype)


# ---- the workloads -----------------------------------------------------------------------

# RMSNorm forward, fp32, 2048 x 1024: one row per wavefront.
RMS_F32_2048x1024 = Workload("rmsnorm_f32_2048x1024_fwd", "rmsnorm", "f32", 2048, 1024, 1e-6,
                             x=normal(0, 1), w=normal(1, 0.1), dy=None)

# LayerNorm forward + backward, bf16 storage, fp32 accumulation, 16384 x 4096.
LN_BF16_16384x4096 = Workload("layernorm_bf16_16384x4096", "layernorm", "bf16", 16384, 4096,
                              1e-5, x=normal(0, 1), w=normal(1, 0.1), b=normal(0, 0.1),
                              dy=normal(0, 1))

# The same LayerNorm with fp32 weight, bias, dW and dB beside the bf16 activations.
LN_BF16_F32W_16384x4096 = replace(LN_BF16_16384x4096,
                                  name="layernorm_bf16_f32w_16384x4096", wdtype="f32")


# RMSNorm forward + backward, bf16, LLM hidden sizes at 32768 tokens, with 1% of the
# columns (channels) scaled by 20.
def rms_hidden(N: int, M: int = 32768) -> Workload:
    return Workload("rmsnorm_bf16_%dx%d_outliers" % (M, N), "rmsnorm", "bf16", M, N, 1e-6,
                    x=normal(0, 1), w=normal(1, 0.05), dy=normal(0, 1e-2), outlier_frac=0.01)


RMS_HIDDEN_SIZES = (2048, 4096, 5120, 8192)

# Fused residual add + RMSNorm forward + backward, bf16, 65536 x 7168.
RESID_RMS_BF16_65536x7168 = Workload("resid_rmsnorm_bf16_65536x7168", "rmsnorm", "bf16", 65536,
                                     7168, 1e-6, x=normal(0, 0.5), r=normal(0, 1),
                                     w=normal(1, 0.1), dy=normal(0, 1))


# Very long rows (split-row class): LayerNorm and RMSNorm forward + backward, bf16.
def long_rows(kind: str, M: int, N: int) -> Workload:
    eps = 1e-5 if kind == "layernorm" else 1e-6
    return Workload("%s_bf16_%dx%d_longrow" % (kind, M, N), kind, "bf16", M, N, eps,
                    x=uniform(-3, 3), w=normal(1, 0.1),
                    b=const(0.0) if kind == "layernorm" else None, dy=normal(0, 1))


LONG_ROW_SHAPES = ((256, 262144), (4, 4194304))


# Beyond the shapes above: row lengths that are not a multiple of the 16-byte access (LayerNorm
# 16384 x 4100 and 16384 x 4097), a hidden size whose backward rows no longer fit a team's registers
# (RMSNorm 16384 x 16384, the looped backward), and fp16 storage, with the same draws as their
# neighbours.
LN_BF16_16384x4100 = LN_BF16_16384x4096.with_shape(16384, 4100, "layernorm_bf16_16384x4100")
# An odd row length (rows at eight different 16-byte phases).
LN_BF16_16384x4097 = LN_BF16_16384x4096.with_shape(16384, 4097, "layernorm_bf16_16384x4097")
# The LayerNorm in fp16 storage.
LN_F16_16384x4096 = replace(LN_BF16_16384x4096, name="layernorm_f16_16384x4096", dtype="f16")
RMS_BF16_16384x16384 = rms_hidden(16384, M=16384)


@dataclass(frozen=True)
class Projection:
    """A norm (the workload `norm`, M x K with K = norm.N) followed by a linear projection
    L [Nout, K] (bf16, row j = output column j) with bias c [Nout] (fp32, or None)."""
    name: str
    norm: Workload
    Nout: int
    l: Dist = normal(0.0, 1.0)  # scaled by K ** -0.5 when drawn
    c: Optional[Dist] = normal(0.0, 0.1)


def make_projection(p: Projection) -> dict:
    """CPU tensors L (bf16, N(0, 1/K) when l is N(0, 1): outputs of unit scale) and c."""
    K = p.norm.N
    s = p.norm.seed
    L = _draw(p.l, (p.Nout, K), s + OFF_L)
    L.mul_(K ** -0.5)
    return {"L": L.to(torch.bfloat16),
            "c": _draw(p.c, (p.Nout,), s + OFF_C) if p.c is not None else None}


# LayerNorm 16384 x 4096 (bf16, the draws of the LayerNorm workload above) into a 4096 x 4096
# projection: a pre-norm block's first matrix product at 16384 tokens.
LN_LINEAR_BF16_16384x4096x4096 = Projection(
    "layernorm_linear_bf16_16384x4096x4096",
    replace(LN_BF16_16384x4096, name="layernorm_bf16_16384x4096_proj", dy=None), 4096)
# The RMSNorm variant (hidden 4096, the outlier-channel draws) into the same projection.
RMS_LINEAR_BF16_16384x4096x4096 = Projection(
    "rmsnorm_linear_bf16_16384x4096x4096",
    replace(rms_hidden(4096, M=16384), name="rmsnorm_bf16_16384x4096_proj", dy=None), 4096,
    c=None)


@dataclass(frozen=True)
class Attention:
    """Attention over B sequences of S tokens: Hq query heads of D dims reading Hk key/value
    heads, with the query and key vectors normalised by `kind` ("layernorm", "rmsnorm" or
    "none") before the scores. Gammas near 1.5 spread the logits over a few units, so the
    softmax weights are neither flat nor one-hot."""
    name: str
    kind: str
    B: int
    S: int
    Hq: int
    Hk: int
    D: int = 128
    causal: bool = True
    eps: float = 1e-6
    q: Dist = normal(0.4, 1.3)
    k: Dist = normal(-0.3, 0.8)
    v: Dist = normal(0.0, 1.0)
    gamma: Dist = normal(1.5, 0.5)
    beta: Dist = normal(0.0, 0.3)
    seed: int = 0

    def with_shape(self, B, S, Hq, Hk, name=None, **kw):
        return replace(self, B=B, S=S, Hq=Hq, Hk=Hk,
                       name=name or "%s[%d,%d,%d,%d]" % (self.name, B, S, Hq, Hk), **kw)


def make_attention(a: Attention) -> dict:
    """CPU bf16 tensors Q [B, S, Hq, D], K and V [B, S, Hk, D], and the norm vectors wq, wk
    (None without a norm), bq, bk (LayerNorm only, else None), each [D]."""
    s = a.seed
    bf = torch.bfloat16
    out = {"Q": _draw(a.q, (a.B, a.S, a.Hq, a.D), s + OFF_Q).to(bf),
           "K": _draw(a.k, (a.B, a.S, a.Hk, a.D), s + OFF_K).to(bf),
           "V": _draw(a.v, (a.B, a.S, a.Hk, a.D), s + OFF_V).to(bf),
           "wq": None, "bq": None, "wk": None, "bk": None}
    if a.kind != "none":
        out["wq"] = _draw(a.gamma, (a.D,), s + OFF_WQ).to(bf)
        out["wk"] = _draw(a.gamma, (a.D,), s + OFF_WK).to(bf)
    if a.kind == "layernorm":
        out["bq"] = _draw(a.beta, (a.D,), s + OFF_BQ).to(bf)
        out["bk"] = _draw(a.beta, (a.D,), s + OFF_BK).to(bf)
    return out


# A QK-norm attention layer at 4096 tokens: 2 sequences, 32 query heads of 128 dims over 8
# key/value heads (grouped), RMSNorm on queries and keys, causal.
ATTN_QKNORM_B2_S4096 = Attention("qknorm_attention_bf16_b2_s4096_hq32_hk8_d128_causal",
                                 "rmsnorm", 2, 4096, 32, 8)


def all_workloads():
    """Every full-size workload, in a fixed order."""
    out = [RMS_F32_2048x1024, LN_BF16_16384x4096, LN_BF16_F32W_16384x4096]
    out += [rms_hidden(N) for N in RMS_HIDDEN_SIZES]
    out.append(RESID_RMS_BF16_65536x7168)
    for M, N in LONG_ROW_SHAPES:
        out += [long_rows("layernorm", M, N), long_rows("rmsnorm", M, N)]
    out += [LN_BF16_16384x4100, LN_BF16_16384x4097, RMS_BF16_16384x16384, LN_F16_16384x4096]
    return out


# The workloads the benchmark reports per shape: the 2048 x 1024 fp32 forward, the LayerNorm
# 16384 x 4096, the four hidden sizes, the residual variant and the four long-row shapes (the
# others above are parity and sweep cases).
CONFIG_WORKLOADS = tuple(
    [RMS_F32_2048x1024.name, LN_BF16_16384x4096.name]
    + [rms_hidden(N).name for N in RMS_HIDDEN_SIZES] + [RESID_RMS_BF16_65536x7168.name]
    + [long_rows(k, M, N).name for M, N in LONG_ROW_SHAPES for k in ("layernorm", "rmsnorm")])
