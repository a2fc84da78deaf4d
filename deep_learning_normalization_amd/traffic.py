"""Algorithmic (minimum) HBM bytes of each pass, the yardstick for achieved bandwidth.

Every [M, N] tensor a pass must read or write moves once, [N] vectors once, and the fp32 row
statistics 4 bytes per row each. Workspace traffic (the backward's column partials, the split
scheme's re-reads) is not counted: it is overhead the kernels must earn back. The unfused
alternative moves several times this (web page "Otimização de Performance de GPU: Maximizando
Throughput para Treinamento e Inferência de LLM", introl.com, section on kernel fusion).
"""


def elem_size(dtype):
    return {"bf16": 2, "f16": 2, "f32": 4}[dtype]


def fwd_bytes(kind, dtype, M, N, residual=False, bias=None, wdtype=None):
    """Read X (and R), W (and B); write Y (and H), rstd (and mean for LayerNorm). `wdtype` is
    the storage of W and B when it differs from the activations'."""
    s = elem_size(dtype)
    layernorm = kind == "layernorm"
    bias = layernorm if bias is None else bias
    mats = (4 if residual else 2) * M * N * s
    vecs = (2 if bias else 1) * N * elem_size(wdtype or dtype)
    stats = (8 if layernorm else 4) * M
    return mats + vecs + stats


def bwd_fused_bytes(kind, dtype, M, N, dh=False, dr_separate=False, wdtype=None):
    """The fused pass: read X, dY (and dH), W, the saved statistics; write dX (and dR)."""
    s = elem_size(dtype)
    mats = (3 + (1 if dh else 0) + (1 if dr_separate else 0)) * M * N * s
    stats = (8 if kind == "layernorm" else 4) * M
    return mats + N * elem_size(wdtype or dtype) + stats


def bwd_bytes(kind, dtype, M, N, dh=False, dr_separate=False, wdtype=None):
    """The whole backward: the fused pass plus writing dW (and dB for LayerNorm), which are
    stored like W."""
    return bwd_fused_bytes(kind, dtype, M, N, dh, dr_separate, wdtype) + \
        (2 if kind == "layernorm" else 1) * N * elem_size(wdtype or dtype)
