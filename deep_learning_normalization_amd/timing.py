"""Cache-cold timing of one workload's passes on the GPU (used by bench.py and by the profiling
driver, so the benchmark and the rocprofv3 captures see the same access pattern).

A workload's tensors are held in S buffer sets on the device (inputs copied once from the host,
the other sets cloned on the device). Every timed loop cycles through the sets so that, between
two uses of one set, the loop moves at least 1 GiB (four times the 256 MB memory-side cache) of
its own algorithmic traffic:
  fwd  loop  norm_fwd on set i mod S: S >= 1 GiB / forward bytes;
  bwd  loop  norm_bwd on set i mod S: S >= 1 GiB / backward bytes;
  step loop  norm_fwd on set i, then the backward on set i + S/2: a set is read by a backward
             and by a forward S/2 steps apart, so S/2 >= 1 GiB / step bytes; S >= 4, so the
             forward never reads what the backward just before it touched.
Each loop runs twice. The first run is bracketed by a synchronize and a pair of events on the
launch stream and has nothing else in it: its time per call (launch gaps included) is the loop
time. In the second run HIP events take each launch's own kernel start and end timestamps
(norm_set_launch_events), for the per-kernel durations; attaching them costs the stream a few
microseconds per launch, so that run's loop time is not used.
"""
import time

ONE_GIB = 1 << 30


def _ceil(a, b):
    return -(-a // b)


def set_count(fwd_bytes, bwd_bytes, min_footprint=ONE_GIB, max_sets=256):
    """Buffer sets for the three loops above."""
    need = [_ceil(min_footprint, fwd_bytes)]
    if bwd_bytes:
        need += [_ceil(min_footprint, bwd_bytes), 2 * _ceil(min_footprint, fwd_bytes + bwd_bytes)]
    S = max([4] + need)
    S += S % 2
    return min(S, max_sets)


def _pct(sorted_vals, q):
    return sorted_vals[min(len(sorted_vals) - 1, int(q * len(sorted_vals)))]


class Rotation:
    """S device buffer sets of one workload (inputs and outputs), shared weights and
    workspaces, and the three pass closures."""

    def __init__(self, w, torch, nl, sets=None, min_footprint=ONE_GIB):
        from deep_learning_normalization_amd import inputs, traffic
        self.w, self.torch, self.nl = w, torch, nl
        dev = torch.device("cuda:0")
        res = w.r is not None
        self.fb = traffic.fwd_bytes(w.kind, w.dtype, w.M, w.N, residual=res, wdtype=w.wdtype)
        self.bb = (traffic.bwd_bytes(w.kind, w.dtype, w.M, w.N, wdtype=w.wdtype)
                   if w.dy is not None else 0)
        self.bfb = (traffic.bwd_fused_bytes(w.kind, w.dtype, w.M, w.N, wdtype=w.wdtype)
                    if w.dy is not None else 0)
        self.S = sets or set_count(self.fb, self.bb, min_footprint)
        host = inputs.make(w)
        first = {k: (v.to(dev) if v is not None else None) for k, v in host.items()}
        self.W, self.B = first["W"], first["B"]
        M, N = w.M, w.N
        ln = w.kind == "layernorm"
        self.sets = []
        for i in range(self.S):
            t = {k: (None if first[k] is None else (first[k] if i == 0 else first[k].clone()))
                 for k in ("X", "R", "dY")}
            X = t["X"]
            t["Y"] = torch.empty_like(X)
            t["H"] = torch.empty_like(X) if res else None
            t["mean"] = torch.empty(M, dtype=torch.float32, device=dev) if ln else None
            t["rstd"] = torch.empty(M, dtype=torch.float32, device=dev)
            t["dX"] = torch.empty_like(X) if w.dy is not None else None
            self.sets.append(t)
        self.set_bytes = sum(v.numel() * v.element_size() for v in self.sets[0].values()
                             if v is not None and v.dim() == 2)
        self.dW = torch.empty_like(self.W)
        self.dB = torch.empty_like(self.W) if ln else None
        adt = host["X"].dtype
        # the split scheme's norm_bwd may sum its column partials inside the fused pass, which
        # the two-stage calls (norm_bwd_fused, then norm_bwd_reduce) cannot
        self.split = (w.dy is not None and nl.norm_plan(
            w.kind, nl.dtype_code(adt, self.W.dtype), nl.PASS_BWD, M, N,
            cu_count=torch.cuda.get_device_properties(0).multi_processor_count)["scheme"]
            == nl.SCHEME_SPLIT)
        self.wsf = nl.workspace(w.kind, adt, nl.PASS_FWD, M, N, res)
        self.wsb = nl.workspace(w.kind, adt, nl.PASS_BWD, M, N) if w.dy is not None else None
        for s in self.sets:  # every set gets its statistics (and H) before a backward reads it
            self.fwd(s)
        torch.cuda.synchronize()

    def fwd(self, s):
        w = self.w
        self.nl.norm_fwd(w.kind, s["X"], s["R"], self.W, self.B, w.eps, s["Y"], s["H"],
                         s["mean"], s["rstd"], self.wsf)

    def _xin(self, s):
        return s["H"] if s["H"] is not None else s["X"]

    def bwd_fused(self, s):
        w = self.w
        self.nl.norm_bwd_fused(w.kind, self._xin(s), s["dY"], None, self.W, s["mean"],
                               s["rstd"], w.eps, s["dX"], None, self.wsb)

    def bwd_reduce(self):
        w = self.w
        self.nl.norm_bwd_reduce(w.kind, w.M, w.N, self.dW, self.dB, self.wsb)

    def bwd(self, s):
        w = self.w
        self.nl.norm_bwd(w.kind, self._xin(s), s["dY"], None, self.W, s["mean"], s["rstd"],
                         w.eps, s["dX"], None, self.dW, self.dB, self.wsb)

    def free(self):
        del self.sets
        self.torch.cuda.empty_cache()


def timed_workload(w, steps, warmup, torch, nl, two_stage=True, settle_s=0.3, rot=None):
    """Time the step, forward and backward loops of workload w (see the module docstring).

    two_stage: the step's backward is norm_bwd_fused (its kernels' timestamps taken on every
    launch) followed by norm_bwd_reduce, which is what norm_bwd runs for the wave, block and
    looped schemes; else, and always for the split scheme, norm_bwd as a whole (timed the same
    way). Returns loop times per call and per-launch kernel statistics (mean, p10, median, p90 in
    microseconds)."""
    rot = rot or Rotation(w, torch, nl)
    two_stage = two_stage and not rot.split
    S = rot.S
    want_bwd = w.dy is not None
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def run(body, n, timed):
        for i in range(warmup):
            body(i, None)
        torch.cuda.synchronize()
        marks = [nl.KernelTimer() for _ in range(n)] if timed else [None] * n
        start, end = ev(), ev()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        for i in range(n):
            body(i, marks[i])
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ks = sorted(1e3 * m.elapsed_ms() for m in marks) if timed else []
        return start.elapsed_time(end) / n, wall, ks

    def kstats(ks):
        return {"mean": sum(ks) / len(ks), "p10": _pct(ks, 0.1), "p50": _pct(ks, 0.5),
                "p90": _pct(ks, 0.9), "min": ks[0], "launches": len(ks)}

    def step(i, timer):
        rot.fwd(rot.sets[i % S])
        if want_bwd:
            if timer:
                timer.arm()
            s = rot.sets[(i + S // 2) % S]
            if two_stage:
                rot.bwd_fused(s)
                rot.bwd_reduce()
            else:
                rot.bwd(s)

    # the GPU clock settles within a few hundred ms of load
    t_end = time.perf_counter() + settle_s
    i = 0
    while time.perf_counter() < t_end or i < warmup:
        step(i, None)
        i += 1
        if i % 50 == 0:
            torch.cuda.synchronize()
    out = {"sets": S, "set_bytes": rot.set_bytes, "footprint_bytes": S * rot.set_bytes,
           "fwd_bytes": rot.fb, "bwd_bytes": rot.bb, "bwd_fused_bytes": rot.bfb}
    if want_bwd:
        ms, wall, _ = run(step, steps, False)
        out["ms_per_step"], out["wall_s"] = ms, wall
        _, _, ks = run(step, steps, True)
        out["step_bwd_kernels_us"] = kstats(ks)

    def fwd_body(i, timer):
        if timer:
            timer.arm()
        rot.fwd(rot.sets[i % S])
    ms, _, _ = run(fwd_body, steps, False)
    out["fwd_us"] = ms * 1e3
    _, _, ks = run(fwd_body, steps, True)
    out["fwd_kernels_us"] = kstats(ks)
    if want_bwd:
        def bwd_body(i, timer):
            if timer:
                timer.arm()
            rot.bwd(rot.sets[i % S])
        ms, _, _ = run(bwd_body, steps, False)
        out["bwd_us"] = ms * 1e3
        _, _, ks = run(bwd_body, steps, True)
        out["bwd_kernels_us"] = kstats(ks)
    return out


def graph_fwd_us(w, torch, nl, replays=10):
    """Forward calls replayed from a captured HIP graph: one forward per buffer set, the sets
    rotating over more than 1 GiB, replayed `replays` times; microseconds per forward. For
    shapes bound by the launch rather than by HBM."""
    from deep_learning_normalization_amd import traffic
    fb = traffic.fwd_bytes(w.kind, w.dtype, w.M, w.N, residual=w.r is not None, wdtype=w.wdtype)
    rot = Rotation(w, torch, nl, sets=max(20, set_count(fb, 0)))

    def body():
        for s in rot.sets:
            rot.fwd(s)
    body()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / (replays * rot.S)
    del g
    rot.free()
    return us
