"""ctypes front end of the double-precision CPU oracle (norm_oracle.c).

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's CPU-baseline
leg import this module. It shares nothing with the HIP library: inputs are passed as the same
bit patterns the device receives (bf16 and fp16 as uint16, fp32 as float32) and every result
comes back as unrounded float64.

Definitions followed (web page "PyTorch atinge desempenho SOTA em normalização com
torch.compile", matsubara.tec.br): para. 2 for what LayerNorm and RMSNorm compute, para. 3 for
the reduction along the contiguous dimension, para. 7 for the gradients dX, dW and dB; and
(web page "Towards Free Normalization: Fusing Normalization into GEMM and Attention Kernels",
brifing.si) items 3-4 and 9-10 for a norm whose output feeds a matrix product, and item 5 for
norms on the queries and keys of an attention.
"""
import ctypes
import os

import numpy as np

from . import build as _build

LAYERNORM, RMSNORM = 0, 1
NO_NORM = -1  # attention with its queries and keys used as given
# storage types: every tensor fp32, bf16 or fp16, or bf16 / fp16 activations and gradients
# with fp32 weight and bias
F32, BF16, BF16_F32W, F16, F16_F32W = 0, 1, 2, 3, 4


def act_dtype(dtype):
    """Storage type of X, R, dY, dH for a call's dtype."""
    return {BF16_F32W: BF16, F16_F32W: F16}.get(dtype, dtype)


def weight_dtype(dtype):
    """Storage type of W and B (and of dW, dB) for a call's dtype."""
    return F32 if dtype in (BF16_F32W, F16_F32W) else dtype


class Oracle:
    """One loaded copy of the oracle library (a path other than the default is used by the
    tests that plant mistakes in a copy of the oracle and check that the pins catch them)."""

    def __init__(self, path=None):
        path = path or _build.LIB
        if not os.path.exists(path):
            raise RuntimeError("oracle library missing: build it with oracle/build.py")
        lib = ctypes.CDLL(path)
        i64, vp, dbl, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p
        lib.oracle_fwd_rows.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, i64,
                                        vp, vp, vp, vp, dbl, dp, dp, dp, dp]
        lib.oracle_fwd_rows.restype = ctypes.c_int
        lib.oracle_bwd_rows.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, i64,
                                        vp, vp, vp, vp, dbl, dp, dp, dp]
        lib.oracle_bwd_rows.restype = ctypes.c_int
        lib.oracle_norm_linear_rows.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                                i64, i64, vp, vp, vp, vp, vp, dbl, dp]
        lib.oracle_norm_linear_rows.restype = ctypes.c_int
        lib.oracle_norm_attention.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i64, i64,
                                              i64, i64, vp, vp, vp, vp, vp, vp, vp, dbl, dbl,
                                              ctypes.c_int, dp, dp]
        lib.oracle_norm_attention.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [ctypes.c_int, vp, i64, dp]
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_round_bf16.argtypes = [dp, i64, vp]
        lib.oracle_round_bf16.restype = ctypes.c_int
        lib.oracle_round_f16.argtypes = [dp, i64, vp]
        lib.oracle_round_f16.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        self.lib = lib
        self.path = path

    def fwd(self, kind, dtype, X, W, B=None, R=None, eps=1e-5, rows=None, want_h=False):
        return _fwd(self.lib, kind, dtype, X, W, B, R, eps, rows, want_h)

    def bwd(self, kind, dtype, X, dY, W, dH=None, eps=1e-5, rows=None, want_dx=True,
            want_dw=True):
        return _bwd(self.lib, kind, dtype, X, dY, W, dH, eps, rows, want_dx, want_dw)

    def norm_linear(self, kind, dtype, X, W, B, L, c=None, eps=1e-5, rows=None):
        return _norm_linear(self.lib, kind, dtype, X, W, B, L, c, eps, rows)

    def norm_attention(self, kind, Q, K, V, Wq=None, Bq=None, Wk=None, Bk=None, eps=1e-6,
                       scale=None, causal=False, b=0, h=0, rows=None):
        return _norm_attention(self.lib, kind, Q, K, V, Wq, Bq, Wk, Bk, eps, scale, causal, b,
                               h, rows)

    def decode(self, dtype, bits):
        return _decode(self.lib, dtype, bits)

    def round_bf16(self, values):
        return _round_bf16(self.lib, values)

    def round_f16(self, values):
        return _round_f16(self.lib, values)

    def num_threads(self):
        return self.lib.oracle_num_threads()

    def set_num_threads(self, n):
        self.lib.oracle_set_num_threads(int(n))


_default = None


def default():
    """The oracle built from oracle/norm_oracle.c (loaded once)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def _bits(a, dtype, shape=None):
    """Validate and return a C-contiguous numpy array of input bits."""
    if a is None:
        return None
    want = np.float32 if dtype == F32 else np.uint16
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        raise TypeError("expected %s bits, got %s" % (np.dtype(want).name, a.dtype))
    if shape is not None and a.shape != shape:
        raise ValueError("expected shape %s, got %s" % (shape, a.shape))
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def _fwd(lib, kind, dtype, X, W, B, R, eps, rows, want_h):
    """Forward over rows [r0, r1) (all rows by default).

    Returns a dict of float64 arrays: y (r x N), mean (r), rstd (r), and h (r x N, the
    rounded R + X) when want_h is set and R is given.
    """
    X = _bits(X, act_dtype(dtype))
    M, N = X.shape
    W = _bits(W, weight_dtype(dtype), (N,))
    B = _bits(B, weight_dtype(dtype), (N,))
    R = _bits(R, act_dtype(dtype), (M, N))
    r0, r1 = (0, M) if rows is None else rows
    n = r1 - r0
    y = np.empty((n, N), np.float64)
    mean = np.empty(n, np.float64)
    rstd = np.empty(n, np.float64)
    h = np.empty((n, N), np.float64) if (want_h and R is not None) else None
    st = lib.oracle_fwd_rows(kind, dtype, M, N, r0, r1, _ptr(X), _ptr(R), _ptr(W), _ptr(B),
                             float(eps), _ptr(y), _ptr(h), _ptr(mean), _ptr(rstd))
    if st:
        raise ValueError("oracle_fwd_rows failed with status %d" % st)
    return {"y": y, "mean": mean, "rstd": rstd, "h": h}


def _bwd(lib, kind, dtype, X, dY, W, dH, eps, rows, want_dx, want_dw):
    """Backward over rows [r0, r1) (all rows by default).

    X is the norm's input (the stored h for the residual variant). Returns float64 arrays:
    dx (r x N, or None), dw (N, summed over the rows given, or None) and db (N, LayerNorm
    only, or None).
    """
    X = _bits(X, act_dtype(dtype))
    M, N = X.shape
    dY = _bits(dY, act_dtype(dtype), (M, N))
    dH = _bits(dH, act_dtype(dtype), (M, N))
    W = _bits(W, weight_dtype(dtype), (N,))
    r0, r1 = (0, M) if rows is None else rows
    n = r1 - r0
    dx = np.empty((n, N), np.float64) if want_dx else None
    dw = np.empty(N, np.float64) if want_dw else None
    db = np.empty(N, np.float64) if (want_dw and kind == LAYERNORM) else None
    st = lib.oracle_bwd_rows(kind, dtype, M, N, r0, r1, _ptr(X), _ptr(dY), _ptr(dH), _ptr(W),
                             float(eps), _ptr(dx), _ptr(dw), _ptr(db))
    if st:
        raise ValueError("oracle_bwd_rows failed with status %d" % st)
    return {"dx": dx, "dw": dw, "db": db}


def _norm_linear(lib, kind, dtype, X, W, B, L, c, eps, rows):
    """Norm(X) @ L.T + c over rows [r0, r1) (all rows by default), unrounded float64.

    X is M x K, W and B (gamma, beta) K each, L the Nout x K projection in the activation
    type, c an Nout fp32 projection bias or None. Returns an (r1-r0) x Nout float64 array.
    Definition: the page "Towards Free Normalization: Fusing Normalization into GEMM and
    Attention Kernels" (brifing.si), items 3-4 and 9-10: a norm whose output feeds a matrix
    product.
    """
    X = _bits(X, act_dtype(dtype))
    M, K = X.shape
    W = _bits(W, weight_dtype(dtype), (K,))
    B = _bits(B, weight_dtype(dtype), (K,))
    L = _bits(L, act_dtype(dtype))
    if L.ndim != 2 or L.shape[1] != K:
        raise ValueError("projection must be Nout x %d, got %s" % (K, L.shape))
    Nout = L.shape[0]
    if c is not None:
        c = np.ascontiguousarray(c, dtype=np.float32)
        if c.shape != (Nout,):
            raise ValueError("projection bias must have %d entries" % Nout)
    r0, r1 = (0, M) if rows is None else rows
    out = np.empty((r1 - r0, Nout), np.float64)
    st = lib.oracle_norm_linear_rows(kind, dtype, M, K, Nout, r0, r1, _ptr(X), _ptr(W), _ptr(B),
                                     _ptr(L), _ptr(c), float(eps), _ptr(out))
    if st:
        raise ValueError("oracle_norm_linear_rows failed with status %d" % st)
    return out


def _norm_attention(lib, kind, Q, K, V, Wq, Bq, Wk, Bk, eps, scale, causal, b, h, rows):
    """Attention of query head h of batch b over query positions [s0, s1) (all by default),
    with the queries and keys normalised first (kind LAYERNORM or RMSNORM) or used as given
    (NO_NORM). Q is B x S x Hq x D, K and V B x S x Hk x D, the four norm vectors D each, all
    bf16 bits (uint16). scale defaults to D ** -0.5. Returns (O, lse): (s1-s0) x D and (s1-s0)
    unrounded float64 arrays. Definition: the page "Towards Free Normalization: Fusing
    Normalization into GEMM and Attention Kernels" (brifing.si), item 5.
    """
    Q = _bits(Q, BF16)
    if Q.ndim != 4:
        raise ValueError("Q must be B x S x Hq x D")
    Bn, S, Hq, D = Q.shape
    K = _bits(K, BF16)
    if K.ndim != 4 or K.shape[:2] != (Bn, S) or K.shape[3] != D:
        raise ValueError("K must be %d x %d x Hk x %d, got %s" % (Bn, S, D, K.shape))
    Hk = K.shape[2]
    V = _bits(V, BF16, K.shape)
    Wq, Bq, Wk, Bk = (_bits(t, BF16, (D,)) for t in (Wq, Bq, Wk, Bk))
    s0, s1 = (0, S) if rows is None else rows
    O = np.empty((s1 - s0, D), np.float64)
    lse = np.empty(s1 - s0, np.float64)
    scale = D ** -0.5 if scale is None else scale
    st = lib.oracle_norm_attention(kind, Bn, S, Hq, Hk, D, b, h, s0, s1, _ptr(Q), _ptr(K),
                                   _ptr(V), _ptr(Wq), _ptr(Bq), _ptr(Wk), _ptr(Bk), float(eps),
                                   float(scale), int(bool(causal)), _ptr(O), _ptr(lse))
    if st:
        raise ValueError("oracle_norm_attention failed with status %d" % st)
    return O, lse


def _decode(lib, dtype, bits):
    """Widen an array of bf16 or fp16 (uint16) or fp32 bits to float64 with the oracle's
    decoder."""
    a = _bits(bits, dtype)
    out = np.empty(a.shape, np.float64)
    if lib.oracle_decode(dtype, _ptr(a), a.size, _ptr(out)):
        raise ValueError("oracle_decode failed")
    return out


def _round_bf16(lib, values):
    """Round float64 values to bf16 bit patterns (nearest, ties to even)."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    if lib.oracle_round_bf16(_ptr(v), v.size, _ptr(out)):
        raise ValueError("oracle_round_bf16 failed")
    return out


def _round_f16(lib, values):
    """Round float64 values to fp16 bit patterns (nearest, ties to even)."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    if lib.oracle_round_f16(_ptr(v), v.size, _ptr(out)):
        raise ValueError("oracle_round_f16 failed")
    return out


def fwd(kind, dtype, X, W, B=None, R=None, eps=1e-5, rows=None, want_h=False):
    return default().fwd(kind, dtype, X, W, B, R, eps, rows, want_h)


def bwd(kind, dtype, X, dY, W, dH=None, eps=1e-5, rows=None, want_dx=True, want_dw=True):
    return default().bwd(kind, dtype, X, dY, W, dH, eps, rows, want_dx, want_dw)


def norm_linear(kind, dtype, X, W, B, L, c=None, eps=1e-5, rows=None):
    return default().norm_linear(kind, dtype, X, W, B, L, c, eps, rows)


def norm_attention(kind, Q, K, V, Wq=None, Bq=None, Wk=None, Bk=None, eps=1e-6, scale=None,
                   causal=False, b=0, h=0, rows=None):
    return default().norm_attention(kind, Q, K, V, Wq, Bq, Wk, Bk, eps, scale, causal, b, h,
                                    rows)


def decode(dtype, bits):
    return default().decode(dtype, bits)


def round_bf16(values):
    return default().round_bf16(values)


def round_f16(values):
    return default().round_f16(values)


def num_threads():
    return default().num_threads()


def set_num_threads(n):
    default().set_num_threads(n)
