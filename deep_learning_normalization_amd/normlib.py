"""Python binding of the C ABI in include/norm.h (libnorm.so, HIP kernels for gfx950).

Argument marshalling only: every function here takes torch tensors (device memory and streams
come from PyTorch), checks their shape, dtype, device and contiguity, and passes raw pointers to
the library. All computation happens in the HIP kernels. If libnorm.so is missing the first call
raises; there is no fallback path.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnorm.so")

LAYERNORM, RMSNORM = 0, 1
F32, BF16, BF16_F32W, F16, F16_F32W = 0, 1, 2, 3, 4
PASS_FWD, PASS_BWD, PASS_STATS = 0, 1, 2
SCHEME_AUTO, SCHEME_WAVE, SCHEME_BLOCK, SCHEME_SPLIT, SCHEME_LOOP = -1, 0, 1, 2, 3
TUNE_SCHEME, TUNE_GRID_PER_CU, TUNE_ROWS_PER_ITER, TUNE_TEAM_THREADS = 0, 1, 2, 3
TUNE_SPLIT_CHUNK, TUNE_ROW_GROUPS, TUNE_TEAMS_PER_WG, TUNE_ROW_ORDER = 4, 5, 6, 7
TUNE_SPLIT_EXCHANGE, TUNE_EXCHANGE_POLLS, TUNE_EXCHANGE_WITHHOLD = 8, 9, 10
TUNE_UNALIGNED = 11
TUNE_ATTN_KEY_PASS = 12
N_TUNE_KEYS = 13

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_EXCHANGE = 0, 1, 2, 3, 4, 5
SIZE_MAX = (1 << 64) - 1

KINDS = {"layernorm": LAYERNORM, "rmsnorm": RMSNORM}
DTYPES = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
MIXED = {torch.bfloat16: BF16_F32W, torch.float16: F16_F32W}


def dtype_code(act, weight=None):
    """norm_dtype_t for activations of torch dtype `act` and weights of `weight` (default: the
    same): one type for both (fp32, bf16, fp16), or bf16 / fp16 activations with fp32
    weights."""
    weight = act if weight is None else weight
    if act == weight:
        return DTYPES[act]
    if act in MIXED and weight == torch.float32:
        return MIXED[act]
    raise ValueError("unsupported dtype pair: activations %s, weights %s" % (act, weight))

SYMBOLS = ("norm_fwd", "norm_bwd", "norm_bwd_fused", "norm_bwd_reduce", "norm_fwd_ex",
           "norm_bwd_ex", "norm_bwd_fused_ex", "norm_stats", "norm_workspace_size",
           "norm_workspace_bytes", "norm_workspace_status", "norm_plan",
           "norm_set_tuning", "norm_set_launch_events", "norm_status_string", "norm_version",
           "norm_fold_projection", "norm_lazy_linear", "norm_bwd_noalloc",
           "norm_attention_fwd", "norm_attention_workspace_bytes")


class NormError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s" % (where, status_string(status)))


class RowStrides(ctypes.Structure):
    """norm_row_strides_t: elements between row starts of each [M, N] tensor (0: N)."""
    _fields_ = [(name, ctypes.c_int64) for name in ("x", "r", "y", "h", "dy", "dh", "dx", "dr")]


class _Plan(ctypes.Structure):
    _fields_ = [("scheme", ctypes.c_int32), ("access_bytes", ctypes.c_int32),
                ("elems_per_access", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("team_threads", ctypes.c_int32), ("accesses_per_thread", ctypes.c_int32),
                ("rows_per_iter", ctypes.c_int32), ("row_order", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("chunks", ctypes.c_int64),
                ("chunk_elems", ctypes.c_int64), ("row_groups", ctypes.c_int64),
                ("partials", ctypes.c_int64), ("workspace_bytes", ctypes.c_uint64),
                ("exchange_row_groups", ctypes.c_int64), ("phase_classes", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded libnorm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libnorm.so is not built (run __graft_entry__.build() or "
                               "deep_learning_normalization_amd/_build.py)")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp, f32, sz = (ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float,
                                 ctypes.c_size_t)
        L.norm_fwd.argtypes = [i32, vp, vp, vp, vp, f32, i64, i64, i32, vp, vp, vp, vp, vp, sz,
                               vp]
        L.norm_bwd.argtypes = [i32, vp, vp, vp, vp, vp, vp, f32, i64, i64, i32, vp, vp, vp, vp,
                               vp, sz, vp]
        L.norm_bwd_fused.argtypes = [i32, vp, vp, vp, vp, vp, vp, f32, i64, i64, i32, vp, vp,
                                     vp, sz, vp]
        L.norm_bwd_reduce.argtypes = [i32, i64, i64, i32, vp, vp, vp, sz, vp]
        L.norm_bwd_noalloc.argtypes = [i32, vp, vp, vp, vp, vp, vp, f32, i64, i64, i32, vp, vp,
                                       vp, vp, vp]
        ld = ctypes.POINTER(RowStrides)
        L.norm_fwd_ex.argtypes = L.norm_fwd.argtypes[:-1] + [ld, vp]
        L.norm_bwd_ex.argtypes = L.norm_bwd.argtypes[:-1] + [ld, vp]
        L.norm_bwd_fused_ex.argtypes = L.norm_bwd_fused.argtypes[:-1] + [ld, vp]
        L.norm_stats.argtypes = [i32, vp, vp, f32, i64, i64, i32, vp, vp, vp, vp, sz, ld, vp]
        L.norm_workspace_size.argtypes = [i32, i32, i32, i64, i64, i32,
                                          ctypes.POINTER(ctypes.c_size_t)]
        L.norm_workspace_bytes.argtypes = [i32, i32, i64, i64, i32, i32]
        L.norm_workspace_bytes.restype = sz
        L.norm_workspace_status.argtypes = [vp, sz, vp]
        L.norm_plan.argtypes = [i32, i32, i32, i64, i64, i32, i32, i32, ctypes.POINTER(_Plan)]
        L.norm_set_tuning.argtypes = [i32, i64]
        L.norm_set_launch_events.argtypes = [vp, vp]
        L.norm_status_string.argtypes = [i32]
        L.norm_status_string.restype = ctypes.c_char_p
        L.norm_version.argtypes = []
        L.norm_fold_projection.argtypes = [i32, i32, vp, i64, vp, vp, vp, i64, i64, vp, i64, vp,
                                           vp, vp]
        L.norm_lazy_linear.argtypes = [i32, vp, i64, i64, i64, f32, vp, i64, i64, vp, vp, vp,
                                       vp, vp, vp, vp, i64, vp]
        L.norm_attention_fwd.argtypes = [i32, ctypes.c_uint32, i64, i64, i64, i64, i64, vp, i64,
                                         vp, i64, vp, i64, vp, vp, vp, vp, f32, f32, vp, i64, vp,
                                         vp, sz, vp]
        L.norm_attention_workspace_bytes.argtypes = [i64, i64, i64, i64]
        L.norm_attention_workspace_bytes.restype = sz
        for name in ("norm_fwd", "norm_bwd", "norm_bwd_fused", "norm_bwd_reduce",
                     "norm_fwd_ex", "norm_bwd_ex", "norm_bwd_fused_ex", "norm_stats",
                     "norm_workspace_size", "norm_workspace_status", "norm_plan",
                     "norm_set_tuning",
                     "norm_set_launch_events", "norm_fold_projection", "norm_lazy_linear",
                     "norm_bwd_noalloc", "norm_attention_fwd"):
            getattr(L, name).restype = ctypes.c_int
        L.norm_version.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status):
    return lib().norm_status_string(int(status)).decode()


def _kind(kind):
    return KINDS[kind] if isinstance(kind, str) else int(kind)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr() or None


_raw_stream = torch._C._cuda_getCurrentRawStream


def _stream(stream, like=None):
    """The hipStream_t of `stream`; None: the current stream of `like`'s device (or of the
    current device)."""
    if stream is None:
        return _raw_stream(like.get_device() if like is not None else torch.cuda.current_device())
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _mat_err(name, dtype, M, N):
    return ValueError("%s must be a CUDA %s tensor of %d x %d elements with contiguous rows"
                      % (name, dtype, M, N))


def _check_mat(t, M, N, dtype, name):
    """A CUDA [M, N] tensor of `dtype` whose rows are contiguous (row stride >= N allowed).
    Returns whether its row stride differs from N (False for None)."""
    if t is None:
        return False
    if t.dtype is not dtype or t.shape != (M, N) or not t.is_cuda:
        raise _mat_err(name, dtype, M, N)
    if t.is_contiguous():
        return False
    if (N > 1 and t.stride(1) != 1) or (M > 1 and t.stride(0) < N):
        raise _mat_err(name, dtype, M, N)
    return M > 1 and t.stride(0) != N


def _strides(**mats):
    """RowStrides for the named [M, N] tensors, or None when every row stride is N."""
    ld = RowStrides()
    strided = False
    for name, t in mats.items():
        if t is None or t.shape[0] <= 1:
            continue
        setattr(ld, name, t.stride(0))
        strided |= t.stride(0) != t.shape[1]
    return ctypes.byref(ld) if strided else None


def _check_vec(t, n, dtype, name):
    if t is None:
        return
    if t.dtype is not dtype or t.numel() != n or not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous CUDA %s tensor of %d elements" % (name, dtype, n))


def _raise(st, where):
    if st != OK:
        raise NormError(st, where)


def _ws(ws):
    if ws is None:
        return None, 0
    return ws.data_ptr(), ws.numel() * ws.element_size()


def norm_fwd(kind, X, R, W, B, eps, Y, H=None, mean=None, rstd=None, workspace=None,
             stream=None):
    """Queue the forward. X, R, Y, H are [M, N]; W, B are [N]; mean, rstd are [M] fp32."""
    M, N = X.shape
    dt, wdt = X.dtype, W.dtype
    strided = _check_mat(X, M, N, dt, "X")
    strided |= _check_mat(R, M, N, dt, "R")
    strided |= _check_mat(Y, M, N, dt, "Y")
    strided |= _check_mat(H, M, N, dt, "H")
    _check_vec(W, N, wdt, "W")
    _check_vec(B, N, wdt, "B")
    _check_vec(mean, M, torch.float32, "mean")
    _check_vec(rstd, M, torch.float32, "rstd")
    wp, wb = _ws(workspace)
    st = lib().norm_fwd_ex(_kind(kind), _ptr(X), _ptr(R), _ptr(W), _ptr(B), float(eps), M, N,
                           dtype_code(dt, wdt), _ptr(Y), _ptr(H), _ptr(mean), _ptr(rstd), wp, wb,
                           _strides(x=X, r=R, y=Y, h=H) if strided else None,
                           _stream(stream, X))
    _raise(st, "norm_fwd")


def norm_stats(kind, X, R, eps, H=None, mean=None, rstd=None, workspace=None, stream=None):
    """Queue the statistics pass alone: mean (LayerNorm) and rstd, and H = R + X with R."""
    M, N = X.shape
    dt = X.dtype
    strided = _check_mat(X, M, N, dt, "X")
    strided |= _check_mat(R, M, N, dt, "R")
    strided |= _check_mat(H, M, N, dt, "H")
    _check_vec(mean, M, torch.float32, "mean")
    _check_vec(rstd, M, torch.float32, "rstd")
    wp, wb = _ws(workspace)
    st = lib().norm_stats(_kind(kind), _ptr(X), _ptr(R), float(eps), M, N, DTYPES[dt], _ptr(H),
                          _ptr(mean), _ptr(rstd), wp, wb,
                          _strides(x=X, r=R, h=H) if strided else None, _stream(stream, X))
    _raise(st, "norm_stats")


def _check_rows(t, rows, cols, dtype, name):
    """A CUDA [rows, cols] tensor of `dtype` with contiguous rows (any row stride >= cols)."""
    if (t.dtype != dtype or tuple(t.shape) != (rows, cols) or not t.is_cuda or
            (cols > 1 and t.stride(1) != 1) or (rows > 1 and t.stride(0) < cols)):
        raise ValueError("%s must be a CUDA %s tensor of %d x %d elements with contiguous rows"
                         % (name, dtype, rows, cols))


def _ld(t):
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def norm_fold_projection(kind, L, gamma, beta, c, G, s, t, stream=None):
    """Queue the fold of the norm's gamma (and beta) into a projection L [Nout, K] (bf16):
    G = bf16(L * gamma), s = row sums of G (LayerNorm), t = L beta + c."""
    Nout, K = L.shape
    _check_rows(L, Nout, K, torch.bfloat16, "L")
    _check_rows(G, Nout, K, torch.bfloat16, "G")
    wdt = gamma.dtype
    _check_vec(gamma, K, wdt, "gamma")
    _check_vec(beta, K, wdt, "beta")
    for v, nm in ((c, "c"), (s, "s"), (t, "t")):
        _check_vec(v, Nout, torch.float32, nm)
    st = lib().norm_fold_projection(_kind(kind), dtype_code(torch.bfloat16, wdt), _ptr(L),
                                    _ld(L), _ptr(gamma), _ptr(beta), _ptr(c), Nout, K, _ptr(G),
                                    _ld(G), _ptr(s), _ptr(t), _stream(stream))
    _raise(st, "norm_fold_projection")


def norm_lazy_linear(kind, X, eps, G, s, t, Y, mean_in=None, rstd_in=None, mean_out=None,
                     rstd_out=None, stream=None):
    """Queue Y = rstd * (X G^T - mean * s) + t (bf16): the norm applied in the projection's
    epilogue, with given statistics (rstd_in) or statistics formed from X's tiles."""
    M, K = X.shape
    Nout = G.shape[0]
    _check_rows(X, M, K, torch.bfloat16, "X")
    _check_rows(G, Nout, K, torch.bfloat16, "G")
    _check_rows(Y, M, Nout, torch.bfloat16, "Y")
    for v, n, nm in ((s, Nout, "s"), (t, Nout, "t"), (mean_in, M, "mean_in"),
                     (rstd_in, M, "rstd_in"), (mean_out, M, "mean_out"), (rstd_out, M, "rstd_out")):
        _check_vec(v, n, torch.float32, nm)
    st = lib().norm_lazy_linear(_kind(kind), _ptr(X), _ld(X), M, K, float(eps), _ptr(G), _ld(G),
                                Nout, _ptr(s), _ptr(t), _ptr(mean_in), _ptr(rstd_in),
                                _ptr(mean_out), _ptr(rstd_out), _ptr(Y), _ld(Y),
                                _stream(stream))
    _raise(st, "norm_lazy_linear")


ATTN_CAUSAL, ATTN_NO_NORM = 1, 2


def _token_stride(t, B, S, H, D, name):
    """Elements between consecutive tokens of a CUDA bf16 [B, S, H, D] tensor whose tokens are
    evenly spaced and whose (head, dim) block is contiguous."""
    if t.dtype is not torch.bfloat16 or tuple(t.shape) != (B, S, H, D) or not t.is_cuda:
        raise ValueError("%s must be a CUDA bfloat16 tensor of shape %s" % (name, (B, S, H, D)))
    ld = t.stride(1) if S > 1 else (t.stride(0) if B > 1 else H * D)
    if ((D > 1 and t.stride(3) != 1) or (H > 1 and t.stride(2) != D) or
            (S > 1 and t.stride(1) != ld) or (B > 1 and t.stride(0) != S * ld)):
        raise ValueError("%s: tokens must be evenly spaced with contiguous heads" % name)
    return ld


def attention_workspace_bytes(B, S, Hk, D):
    """Bytes of workspace norm_attention_fwd's key pass uses."""
    return lib().norm_attention_workspace_bytes(B, S, Hk, D)


def norm_attention_fwd(kind, Q, K, V, wq, bq, wk, bk, eps, scale, O, lse=None, causal=False,
                       normalize=True, workspace=None, stream=None):
    """Queue attention over normalised queries and keys: Q, O [B, S, Hq, D], K, V
    [B, S, Hk, D] (bf16, evenly spaced tokens, e.g. slices of one packed QKV tensor), gammas
    wq, wk and betas bq, bk [D] bf16, lse [B, Hq, S] fp32 or None. normalize=False: the
    queries and keys as given (the norm vectors must be None), as does kind "none". workspace:
    a CUDA tensor of at least attention_workspace_bytes() bytes for the key pass, or None."""
    Bn, S, Hq, D = Q.shape
    Hk = K.shape[2]
    ldq = _token_stride(Q, Bn, S, Hq, D, "Q")
    ldk = _token_stride(K, Bn, S, Hk, D, "K")
    ldv = _token_stride(V, Bn, S, Hk, D, "V")
    ldo = _token_stride(O, Bn, S, Hq, D, "O")
    for v, nm in ((wq, "wq"), (bq, "bq"), (wk, "wk"), (bk, "bk")):
        _check_vec(v, D, torch.bfloat16, nm)
    if lse is not None and (lse.dtype is not torch.float32 or tuple(lse.shape) != (Bn, Hq, S)
                            or not lse.is_cuda or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous CUDA float32 tensor of shape %s"
                         % ((Bn, Hq, S),))
    if kind == "none":
        kind, normalize = RMSNORM, False
    flags = (ATTN_CAUSAL if causal else 0) | (0 if normalize else ATTN_NO_NORM)
    st = lib().norm_attention_fwd(_kind(kind), flags, Bn, S, Hq, Hk, D, _ptr(Q), ldq, _ptr(K),
                                  ldk, _ptr(V), ldv, _ptr(wq), _ptr(bq), _ptr(wk), _ptr(bk),
                                  float(eps), float(scale), _ptr(O), ldo, _ptr(lse),
                                  *_ws(workspace), _stream(stream, Q))
    _raise(st, "norm_attention_fwd")


def norm_bwd(kind, X, dY, dH, W, mean, rstd, eps, dX, dR, dW, dB, workspace, stream=None):
    """Queue the backward (fused pass, then the column reduction)."""
    M, N = X.shape
    dt, wdt = X.dtype, W.dtype
    strided = _check_mat(X, M, N, dt, "X")
    strided |= _check_mat(dY, M, N, dt, "dY")
    strided |= _check_mat(dH, M, N, dt, "dH")
    strided |= _check_mat(dX, M, N, dt, "dX")
    strided |= _check_mat(dR, M, N, dt, "dR")
    for t, nm in ((W, "W"), (dW, "dW"), (dB, "dB")):
        _check_vec(t, N, wdt, nm)
    _check_vec(mean, M, torch.float32, "mean")
    _check_vec(rstd, M, torch.float32, "rstd")
    wp, wb = _ws(workspace)
    st = lib().norm_bwd_ex(_kind(kind), _ptr(X), _ptr(dY), _ptr(dH), _ptr(W), _ptr(mean),
                           _ptr(rstd), float(eps), M, N, dtype_code(dt, wdt), _ptr(dX), _ptr(dR),
                           _ptr(dW), _ptr(dB), wp, wb,
                           _strides(x=X, dy=dY, dh=dH, dx=dX, dr=dR) if strided else None,
                           _stream(stream, X))
    _raise(st, "norm_bwd")


def norm_bwd_noalloc(kind, X, dY, dH, W, mean, rstd, eps, dX, dR, dW, dB, stream=None):
    """Queue the backward with the library's own device scratch as its workspace (no
    allocation anywhere). Contiguous [M, N] tensors only."""
    M, N = X.shape
    dt, wdt = X.dtype, W.dtype
    for t, nm in ((X, "X"), (dY, "dY"), (dH, "dH"), (dX, "dX"), (dR, "dR")):
        _check_mat(t, M, N, dt, nm)
        if t is not None and not t.is_contiguous():
            raise ValueError("%s must be contiguous" % nm)
    for t, nm in ((W, "W"), (dW, "dW"), (dB, "dB")):
        _check_vec(t, N, wdt, nm)
    _check_vec(mean, M, torch.float32, "mean")
    _check_vec(rstd, M, torch.float32, "rstd")
    st = lib().norm_bwd_noalloc(_kind(kind), _ptr(X), _ptr(dY), _ptr(dH), _ptr(W), _ptr(mean),
                                _ptr(rstd), float(eps), M, N, dtype_code(dt, wdt), _ptr(dX),
                                _ptr(dR), _ptr(dW), _ptr(dB), _stream(stream))
    _raise(st, "norm_bwd_noalloc")


def norm_bwd_fused(kind, X, dY, dH, W, mean, rstd, eps, dX, dR, workspace, stream=None):
    """Queue the backward's fused pass: dX (and dR), column partials into the workspace."""
    M, N = X.shape
    dt, wdt = X.dtype, W.dtype
    strided = _check_mat(X, M, N, dt, "X")
    strided |= _check_mat(dY, M, N, dt, "dY")
    strided |= _check_mat(dH, M, N, dt, "dH")
    strided |= _check_mat(dX, M, N, dt, "dX")
    strided |= _check_mat(dR, M, N, dt, "dR")
    _check_vec(W, N, wdt, "W")
    _check_vec(mean, M, torch.float32, "mean")
    _check_vec(rstd, M, torch.float32, "rstd")
    wp, wb = _ws(workspace)
    st = lib().norm_bwd_fused_ex(_kind(kind), _ptr(X), _ptr(dY), _ptr(dH), _ptr(W), _ptr(mean),
                                 _ptr(rstd), float(eps), M, N, dtype_code(dt, wdt), _ptr(dX),
                                 _ptr(dR), wp, wb,
                                 _strides(x=X, dy=dY, dh=dH, dx=dX, dr=dR) if strided else None,
                                 _stream(stream, X))
    _raise(st, "norm_bwd_fused")


def norm_bwd_reduce(kind, M, N, dW, dB, workspace, stream=None):
    """Queue the column reduction of the partials a fused pass left in the workspace (the
    outputs' dtype selects the store type: fp32 dW, dB for F32 and the fp32-weight types)."""
    dt = dW.dtype
    _check_vec(dW, N, dt, "dW")
    _check_vec(dB, N, dt, "dB")
    wp, wb = _ws(workspace)
    st = lib().norm_bwd_reduce(_kind(kind), M, N, DTYPES[dt], _ptr(dW), _ptr(dB), wp, wb,
                               _stream(stream))
    _raise(st, "norm_bwd_reduce")


def norm_workspace_size(kind, dtype, pass_, M, N, residual=False):
    """Workspace bytes for a call on the current device."""
    out = ctypes.c_size_t(0)
    dt = DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)  # int: norm_dtype_t
    st = lib().norm_workspace_size(_kind(kind), dt, int(pass_), M, N, int(bool(residual)),
                                   ctypes.byref(out))
    _raise(st, "norm_workspace_size")
    return out.value


def norm_workspace_bytes(kind, pass_, M, N, dtype, residual=False):
    """Workspace bytes enough for a call on any gfx950 device (host only, no GPU needed);
    SIZE_MAX for arguments no call accepts."""
    dt = dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    return lib().norm_workspace_bytes(_kind(kind), int(pass_), M, N, dt, int(bool(residual)))


def norm_workspace_status(workspace, stream=None):
    """Synchronise `stream`, read and clear the workspace's exchange-failure word: OK, or
    ERR_EXCHANGE if a call on it gave up a wait (and wrote NaN) since the last query."""
    wp, wb = _ws(workspace)
    return lib().norm_workspace_status(wp, wb, _stream(stream))


def norm_plan(kind, dtype, pass_, M, N, residual=False, align=16, cu_count=256):
    """The dispatcher's plan for a shape, as a dict (pure host logic, no GPU needed). align:
    the largest power of two (up to 16) dividing every tensor's address."""
    p = _Plan()
    dt = DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    st = lib().norm_plan(_kind(kind), dt, int(pass_), M, N, int(bool(residual)),
                         int(align), int(cu_count), ctypes.byref(p))
    _raise(st, "norm_plan")
    return {name: getattr(p, name) for name, _ in _Plan._fields_}


def norm_set_tuning(key, value):
    _raise(lib().norm_set_tuning(int(key), int(value)), "norm_set_tuning")


def norm_set_launch_events(start, stop):
    """Arm two raw hipEvent_t handles (ints) for this thread's next entry-point call."""
    _raise(lib().norm_set_launch_events(start or None, stop or None), "norm_set_launch_events")


def norm_version():
    return lib().norm_version()


class KernelTimer:
    """HIP events that take the kernels' own start and end timestamps (see
    norm_set_launch_events): `arm()` before an entry-point call, `elapsed_ms()` after the
    stream has passed it. Events come from the HIP runtime the library is linked against."""

    _hip = None

    @classmethod
    def _rt(cls):
        if cls._hip is None:
            lib()  # the runtime libnorm.so loaded
            h = ctypes.CDLL("libamdhip64.so.7")
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                              ctypes.c_void_p]
            h.hipGetLastError.argtypes = []
            for f in ("hipEventCreateWithFlags", "hipEventDestroy", "hipEventElapsedTime",
                      "hipGetLastError"):
                getattr(h, f).restype = ctypes.c_int
            cls._hip = h
        return cls._hip

    def __init__(self):
        h = self._rt()
        self.start, self.stop = ctypes.c_void_p(), ctypes.c_void_p()
        for e in (self.start, self.stop):
            if h.hipEventCreateWithFlags(ctypes.byref(e), 0) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")

    def arm(self):
        norm_set_launch_events(self.start.value, self.stop.value)

    def elapsed_ms(self):
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.start, self.stop) != 0:
            # the failed call also left the runtime's per-thread last error set; consume it so
            # that the next error check (torch's, after its own kernel launches) does not see it
            self._hip.hipGetLastError()
            raise RuntimeError("hipEventElapsedTime failed (events not recorded?)")
        return ms.value

    def __del__(self):
        h = self._hip
        if h is not None:
            for e in (self.start, self.stop):
                if e.value:
                    h.hipEventDestroy(e)


# ---- allocating conveniences (torch allocates; the kernels compute) ------------------------

def workspace(kind, dtype, pass_, M, N, residual=False, device="cuda"):
    n = norm_workspace_size(kind, dtype, pass_, M, N, residual)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def forward(kind, X, W, B=None, eps=1e-5, R=None, stream=None):
    """Y, H (or None), mean (LayerNorm, else None), rstd of the forward."""
    M, N = X.shape
    k = _kind(kind)
    Y = torch.empty_like(X)
    H = torch.empty_like(X) if R is not None else None
    mean = torch.empty(M, dtype=torch.float32, device=X.device) if k == LAYERNORM else None
    rstd = torch.empty(M, dtype=torch.float32, device=X.device)
    ws = workspace(k, X.dtype, PASS_FWD, M, N, R is not None, X.device)
    norm_fwd(k, X, R, W, B, eps, Y, H, mean, rstd, ws, stream)
    return Y, H, mean, rstd


def fold_projection(kind, L, gamma, beta=None, c=None, stream=None):
    """G, s (LayerNorm, else None), t (or None) for a projection L [Nout, K] after the norm."""
    Nout, K = L.shape
    k = _kind(kind)
    G = torch.empty_like(L)
    s = torch.empty(Nout, dtype=torch.float32, device=L.device) if k == LAYERNORM else None
    t = (torch.empty(Nout, dtype=torch.float32, device=L.device)
         if (beta is not None or c is not None) else None)
    norm_fold_projection(k, L, gamma, beta, c, G, s, t, stream)
    return G, s, t


def lazy_linear(kind, X, eps, G, s=None, t=None, mean=None, rstd=None, stream=None):
    """Norm(X) L^T + c as bf16 [M, Nout] from the fold's G, s, t; statistics from `rstd` (and
    `mean`) when given, else formed inside the product."""
    Y = torch.empty(X.shape[0], G.shape[0], dtype=torch.bfloat16, device=X.device)
    norm_lazy_linear(kind, X, eps, G, s, t, Y, mean, rstd, None, None, stream)
    return Y


def attention(kind, Q, K, V, wq=None, bq=None, wk=None, bk=None, eps=1e-6, scale=None,
              causal=False, want_lse=False, key_pass=True, stream=None):
    """O (and lse when want_lse) of attention over queries and keys normalised by `kind` with
    the given gammas (and betas); with wq and wk None (or kind "none") the queries and keys are
    used as given. key_pass: give the call a workspace for its key pass."""
    normalize = kind != "none" and (wq is not None or wk is not None)
    Bn, S, _, D = Q.shape
    ws = None
    if normalize and key_pass:
        ws = torch.empty(attention_workspace_bytes(Bn, S, K.shape[2], D), dtype=torch.uint8,
                         device=Q.device)
    O = torch.empty(Q.shape, dtype=torch.bfloat16, device=Q.device)
    lse = (torch.empty(Q.shape[0], Q.shape[2], Q.shape[1], dtype=torch.float32, device=Q.device)
           if want_lse else None)
    norm_attention_fwd(kind, Q, K, V, wq, bq, wk, bk, eps, D ** -0.5 if scale is None else scale,
                       O, lse, causal, normalize, ws, stream)
    return (O, lse) if want_lse else O


def backward(kind, X, dY, W, mean=None, rstd=None, eps=1e-5, dH=None, stream=None):
    """dX, dW, dB (LayerNorm, else None) of the backward."""
    M, N = X.shape
    k = _kind(kind)
    dX = torch.empty_like(X)
    dW = torch.empty_like(W)
    dB = torch.empty_like(W) if k == LAYERNORM else None
    ws = workspace(k, X.dtype, PASS_BWD, M, N, False, X.device)
    norm_bwd(k, X, dY, dH, W, mean, rstd, eps, dX, None, dW, dB, ws, stream)
    return dX, dW, dB
