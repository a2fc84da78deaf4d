"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph): every replay must give
the bits the same calls give eagerly on the same inputs. Replays run several times with eager
work and new input values between them (a graph's memory nodes are its weak point, and the
library records none: it has no memsets and allocates nothing)."""
import pytest
import torch

from deep_learning_normalization_amd import inputs, normlib as nl

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[gpu] " + msg, flush=True)


def _case(kind, dtype, M, N):
    return inputs.Workload("%s_%s_%dx%d" % (kind, dtype, M, N), kind, dtype, M, N,
                           1e-5 if kind == "layernorm" else 1e-6, x=inputs.normal(0.2, 1.3),
                           w=inputs.normal(1, 0.1),
                           b=inputs.normal(0, 0.1) if kind == "layernorm" else None,
                           dy=inputs.normal(0, 1))


# wave (fp32 2048 x 1024, the launch-bound shape), block, looped backward, split
CASES = [("rmsnorm", "f32", 2048, 1024), ("layernorm", "bf16", 1024, 4096),
         ("rmsnorm", "bf16", 512, 12288), ("layernorm", "bf16", 16, 262144)]


def _calls(kind, d, out, ws_f, ws_b):
    ln = kind == "layernorm"
    nl.norm_fwd(kind, d["X"], None, d["W"], d["B"] if ln else None, d["eps"], out["Y"], None,
                out["mean"], out["rstd"], ws_f)
    nl.norm_bwd(kind, d["X"], d["dY"], None, d["W"], out["mean"], out["rstd"], d["eps"],
                out["dX"], None, out["dW"], out["dB"], ws_b)
    nl.norm_stats(kind, d["X"], None, d["eps"], None, out["smean"], out["srstd"], ws_f)


def _outputs(kind, X, W):
    M = X.shape[0]
    ln = kind == "layernorm"
    return {"Y": torch.empty_like(X), "dX": torch.empty_like(X), "dW": torch.empty_like(W),
            "dB": torch.empty_like(W) if ln else None,
            "mean": torch.empty(M, device="cuda") if ln else None,
            "rstd": torch.empty(M, device="cuda"),
            "smean": torch.empty(M, device="cuda") if ln else None,
            "srstd": torch.empty(M, device="cuda")}


@pytest.mark.parametrize("kind,dt,M,N", CASES, ids=lambda v: str(v))
def test_graph_replays_match_eager(kind, dt, M, N):
    w = _case(kind, dt, M, N)
    t = inputs.make(w)
    d = {k: (t[k].cuda() if t[k] is not None else None) for k in ("X", "W", "B", "dY")}
    d["eps"] = w.eps
    ws_f = nl.workspace(kind, d["X"].dtype, nl.PASS_FWD, M, N)
    ws_b = nl.workspace(kind, d["X"].dtype, nl.PASS_BWD, M, N)
    g_out = _outputs(kind, d["X"], d["W"])
    e_out = _outputs(kind, d["X"], d["W"])
    ws_fe = torch.empty_like(ws_f)
    ws_be = torch.empty_like(ws_b)
    _say("graph capture %s %s %dx%d" % (kind, dt, M, N))
    _calls(kind, d, g_out, ws_f, ws_b)      # warm up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _calls(kind, d, g_out, ws_f, ws_b)
    torch.cuda.synchronize()
    for rep in range(4):
        # new input values in place, then the graph, then the same calls eagerly
        seed = 100 + rep
        fresh = inputs.make(inputs.Workload(w.name, kind, dt, M, N, w.eps, seed=seed, x=w.x, w=w.w,
                                            b=w.b, dy=w.dy))
        for k in ("X", "W", "B", "dY"):
            if d[k] is not None:
                d[k].copy_(fresh[k])
        for v in g_out.values():
            if v is not None:
                v.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        _calls(kind, d, e_out, ws_fe, ws_be)
        torch.cuda.synchronize()
        for k in g_out:
            if g_out[k] is not None:
                assert torch.equal(g_out[k], e_out[k]), "replay %d: %s differs" % (rep, k)
        _say("replay %d matches eager" % rep)
