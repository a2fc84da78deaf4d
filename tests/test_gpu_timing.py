"""Kernel timestamps through norm_set_launch_events (needs a gfx950 GPU): the events bracket
the kernels of exactly one call, outputs are unchanged by timing, and a failing call disarms."""
import time

import pytest
import torch

from deep_learning_normalization_amd import inputs, normlib as nl

pytestmark = pytest.mark.gpu


def _data(M=4096, N=4096):
    w = inputs.Workload("timing", "layernorm", "bf16", M, N, 1e-5, x=inputs.normal(0, 1),
                        w=inputs.normal(1, 0.1), b=inputs.normal(0, 0.1), dy=inputs.normal(0, 1))
    h = inputs.make(w)
    return {k: (v.cuda() if v is not None else None) for k, v in h.items()}


def test_timer_brackets_one_call_and_leaves_outputs_unchanged():
    print("[gpu] launch-event timing, layernorm bf16 4096 x 4096", flush=True)
    d = _data()
    X, W, B, dY = d["X"], d["W"], d["B"], d["dY"]
    Y0, _, mean, rstd = nl.forward("layernorm", X, W, B, 1e-5)
    dX0, dW0, dB0 = nl.backward("layernorm", X, dY, W, mean, rstd, 1e-5)
    torch.cuda.synchronize()

    tf, tb = nl.KernelTimer(), nl.KernelTimer()
    t0 = time.perf_counter()
    tf.arm()
    Y1, _, m1, r1 = nl.forward("layernorm", X, W, B, 1e-5)
    tb.arm()
    dX1, dW1, dB1 = nl.backward("layernorm", X, dY, W, m1, r1, 1e-5)   # two kernels
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    f_ms, b_ms = tf.elapsed_ms(), tb.elapsed_ms()
    assert 0 < f_ms < wall_ms and 0 < b_ms < wall_ms
    assert f_ms + b_ms < wall_ms
    # 64 MiB read + 32 MiB written at no more than 8 TB/s: at least 12 us
    assert f_ms > 0.012
    for a, b in ((Y0, Y1), (mean, m1), (rstd, r1), (dX0, dX1), (dW0, dW1), (dB0, dB1)):
        assert torch.equal(a, b)


def test_failing_call_disarms():
    print("[gpu] launch-event disarm on error", flush=True)
    d = _data(256, 1024)
    X, W, B = d["X"], d["W"], d["B"]
    t = nl.KernelTimer()
    t.arm()
    with pytest.raises(ValueError):
        nl.norm_fwd("layernorm", X, None, W, B, 1e-5, torch.empty(3, device="cuda"))
    # the binding rejected that one before the library saw it: disarm through the library
    t.arm()
    Y = torch.empty_like(X)
    with pytest.raises(nl.NormError):
        nl.norm_fwd("layernorm", X, None, W, B, -1.0, Y)          # eps < 0: checked, no launch
    nl.forward("layernorm", X, W, B, 1e-5)                        # not timed
    torch.cuda.synchronize()
    with pytest.raises(RuntimeError):
        t.elapsed_ms()                                            # never recorded
    # and that failed query leaves no error behind for the next kernel launch's check
    z = torch.zeros(1024, device="cuda")
    assert torch.equal(z + 1, torch.ones_like(z))
    torch.cuda.synchronize()
