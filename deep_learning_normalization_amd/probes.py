"""Binding of libhbmprobe.so (include/hbm_probe.h): streaming kernels that measure the HBM
bandwidth a stream mix reaches on this device (read, write, copy, two reads and one write, two
reads and two writes), the ceilings the benchmark reports beside the norm passes, and a
matrix-core probe, the ceiling for the bf16 products.

ceilings() times every probe over buffers that rotate through more than 1 GiB (so no call finds
its inputs in the 256 MB memory-side cache), each launch bracketed by its own kernel timestamps,
for a few access shapes, and returns the best rate per mix."""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhbmprobe.so")

# name: (input streams, output streams)
MIXES = {"read": (1, 0), "write": (0, 1), "copy": (1, 1), "triad": (2, 1), "2r2w": (2, 2)}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libhbmprobe.so is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        L.hbm_probe.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, ctypes.c_size_t,
                                ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_uint32, vp,
                                vp, vp]
        L.hbm_probe.restype = ctypes.c_int
        L.mfma_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int, vp,
                                 vp, vp, vp]
        L.mfma_probe.restype = ctypes.c_int
        L.lds_probe.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, vp, vp, vp, vp]
        L.lds_probe.restype = ctypes.c_int
        _lib = L
    return _lib


def probe(nin, nout, ins, outs, nbytes, unroll=4, nt_loads=0, grid=0, key=0x9E3779B9,
          timer=None, stream=None):
    """Queue one probe; `timer` (a normlib.KernelTimer) takes the kernel's own timestamps."""
    ins = list(ins) + [None] * (2 - len(ins))
    outs = list(outs) + [None] * (2 - len(outs))
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    e0 = timer.start.value if timer is not None else None
    e1 = timer.stop.value if timer is not None else None
    st = lib().hbm_probe(nin, nout, ptr(ins[0]), ptr(ins[1]), ptr(outs[0]), ptr(outs[1]),
                         nbytes, unroll, nt_loads, grid, key, e0, e1, s)
    if st != 0:
        raise RuntimeError("hbm_probe(%d, %d) failed: %d" % (nin, nout, st))


def ceilings(stream_bytes=256 << 20, pool=8, iters=12, variants=None):
    """Best measured GB/s per stream mix. A pool of `pool` buffers of `stream_bytes` rotates
    (each call takes the next nin + nout buffers), so a buffer is touched again only after at
    least pool - 4 others (1 GiB at the defaults): every call streams from HBM. Each variant
    (unroll, nontemporal loads, grid) runs `iters` timed launches; the median launch gives its
    rate (bytes moved = (nin + nout) * stream_bytes), and the best variant is the ceiling."""
    from deep_learning_normalization_amd import normlib as nl
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    n = stream_bytes // 4
    bufs = [torch.empty(n, dtype=torch.int32, device="cuda") for _ in range(pool)]
    for i, b in enumerate(bufs):
        b.random_(generator=torch.Generator(device="cuda").manual_seed(i))
    sink = torch.empty(4, dtype=torch.int32, device="cuda")
    if variants is None:
        variants = [(u, nt, g) for u in (2, 4, 8) for nt in (0, 1) for g in (0, 8 * cu)]
    timers = [nl.KernelTimer() for _ in range(iters)]
    out = {}
    k = 0
    for name, (nin, nout) in MIXES.items():
        best = None
        for (u, nt, g) in variants:
            def call(timer):
                nonlocal k
                ins = [bufs[(k + j) % pool] for j in range(nin)]
                outs = [bufs[(k + nin + j) % pool] for j in range(nout)] or [sink]
                k += nin + nout
                probe(nin, nout, ins, outs, stream_bytes, u, nt, g, timer=timer)
            for _ in range(2):
                call(None)
            for t in timers:
                call(t)
            torch.cuda.synchronize()
            us = sorted(1e3 * t.elapsed_ms() for t in timers)
            med = us[len(us) // 2]
            gbps = (nin + nout) * stream_bytes / (med * 1e-6) / 1e9
            if best is None or gbps > best["GBps"]:
                best = {"GBps": round(gbps, 1), "us": round(med, 2), "unroll": u,
                        "nt_loads": nt, "grid": g or "one workgroup per tile",
                        "streams": "%dR%dW" % (nin, nout),
                        "bytes_per_launch": (nin + nout) * stream_bytes}
        out[name] = best
    del bufs
    torch.cuda.empty_cache()
    return out


# flops of one matrix operation of each probed shape
MFMA_FLOPS = {32: 2 * 32 * 32 * 16, 16: 2 * 16 * 16 * 32}


def mfma_ceiling(iters=4096, launches=8):
    """Measured bf16 matrix-core rate in TFLOP/s per operation shape (32x32x16, 16x16x32) and
    occupancy (one or two wavefronts per SIMD): one workgroup per compute unit, each wavefront
    running `iters` x 8 independent operations; the median of `launches` timed launches. The
    best figure per shape is the ceiling for kernels built on that shape."""
    from deep_learning_normalization_amd import normlib as nl
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(cu * 512, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    timers = [nl.KernelTimer() for _ in range(launches)]
    res = {}
    for shape in (32, 16):
        best = None
        for waves in (1, 2):
            for t in [None, None] + timers:
                st = lib().mfma_probe(shape, waves, cu, iters, out.data_ptr(),
                                      t.start.value if t else None,
                                      t.stop.value if t else None, s)
                if st != 0:
                    raise RuntimeError("mfma_probe(%d, %d) failed: %d" % (shape, waves, st))
            torch.cuda.synchronize()
            us = sorted(1e3 * t.elapsed_ms() for t in timers)
            med = us[len(us) // 2]
            flops = cu * 4 * waves * iters * 8 * MFMA_FLOPS[shape]
            tf = flops / (med * 1e-6) / 1e12
            if best is None or tf > best["TFLOPs"]:
                best = {"TFLOPs": round(tf, 1), "waves_per_simd": waves, "us": round(med, 2)}
        res["%dx%dx%d" % ((32, 32, 16) if shape == 32 else (16, 16, 32))] = best
    del out
    return res


def lds_read_rate(iters=4096, launches=8):
    """Measured LDS read bandwidth in bytes per clock per compute unit (at the 2.4 GHz peak
    clock) for 16-byte conflict-free reads, per occupancy (1, 2, 4 wavefronts per SIMD): one
    workgroup per compute unit; the median of `launches` timed launches."""
    from deep_learning_normalization_amd import normlib as nl
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(cu * 1024, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    timers = [nl.KernelTimer() for _ in range(launches)]
    res = {}
    for waves in (1, 2, 4):
        for t in [None, None] + timers:
            st = lib().lds_probe(waves, cu, iters, out.data_ptr(), t.start.value if t else None,
                                 t.stop.value if t else None, s)
            if st != 0:
                raise RuntimeError("lds_probe(%d) failed: %d" % (waves, st))
        torch.cuda.synchronize()
        us = sorted(1e3 * t.elapsed_ms() for t in timers)
        med = us[len(us) // 2]
        nbytes = cu * 256 * waves * iters * 8 * 16
        res["%d_waves_per_simd" % waves] = {
            "bytes_per_clk_per_cu": round(nbytes / (med * 1e-6) / cu / 2.4e9, 1),
            "us": round(med, 2)}
    del out
    return res
