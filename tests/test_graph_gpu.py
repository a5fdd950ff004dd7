"""The entry points inside a captured HIP graph.

Every entry point launches on the stream it is given, allocates nothing and
makes no synchronising or memset call, so a caller can capture a whole
forward + backward into a graph and replay it without the host's per-call
cost.  Each test captures the calls (through the Python binding, which passes
torch's current stream, the capture stream), then replays the graph three
times with eager work and a synchronisation between replays: the outputs are
reset (and in-place inputs restored) eagerly, and every replay must give
results bit-identical to the same calls run eagerly — the kernels are
deterministic for a fixed shape and launch plan, so anything else means a
replay read or wrote something other than what the eager calls did.
"""
import pytest
import torch

import row_normalization_amd as rn
import workloads as wl

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _case(*what):
    print("case:", *what, flush=True)


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # one warm-up call off the default stream, as capture requires
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_check(g, reset, outputs, ref):
    for k in range(REPLAYS):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t in outputs.items():
            assert torch.equal(t, ref[name]), f"replay {k}: {name} differs from the eager result"


def test_rmsnorm_fwd_bwd_graph():
    w = wl.C2.scaled(M=3001, N=4096)
    _case(w.name, w.M, w.N)
    t = wl.make_inputs(w)
    x, g_, dy = t["x"].cuda(), t["gamma"].cuda(), t["dy"].cuda()
    y, dx = torch.empty_like(x), torch.empty_like(x)
    rstd = torch.empty(w.M, dtype=torch.float32, device="cuda")
    dgamma = torch.empty(w.N, dtype=torch.float32, device="cuda")
    ws = torch.empty(rn.rmsnorm_bwd_workspace_bytes(w.M, w.N, x.dtype) // 4, dtype=torch.float32, device="cuda")

    def step():
        rn.rmsnorm_fwd(x, g_, y, rstd, eps=w.eps)
        rn.rmsnorm_bwd(x, g_, dy, rstd, dx, dgamma, ws)

    outputs = {"y": y, "rstd": rstd, "dx": dx, "dgamma": dgamma}
    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outputs.items()}
    graph = _capture(step)

    def reset():
        for v in outputs.values():
            v.fill_(float("nan"))
        ws.fill_(float("nan"))

    _replay_and_check(graph, reset, outputs, ref)


def test_rmsnorm_gemma_in_place_graph():
    w = wl.C3.scaled(M=2048)
    _case(w.name, w.M, w.N, "dx in place")
    t = wl.make_inputs(w)
    x, g_, dy0 = t["x"].cuda(), t["gamma"].cuda(), t["dy"].cuda()
    dy = dy0.clone()
    y = torch.empty_like(x)
    rstd = torch.empty(w.M, dtype=torch.float32, device="cuda")
    dgamma = torch.empty(w.N, dtype=torch.float32, device="cuda")
    ws = torch.empty(rn.rmsnorm_bwd_workspace_bytes(w.M, w.N, x.dtype) // 4, dtype=torch.float32, device="cuda")

    def step():
        rn.rmsnorm_fwd(x, g_, y, rstd, eps=w.eps, gemma=True)
        rn.rmsnorm_bwd(x, g_, dy, rstd, dy, dgamma, ws, gemma=True)

    outputs = {"y": y, "rstd": rstd, "dx": dy, "dgamma": dgamma}
    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outputs.items()}
    dy.copy_(dy0)
    graph = _capture(step)

    def reset():
        dy.copy_(dy0)
        for v in (y, rstd, dgamma):
            v.fill_(float("nan"))

    _replay_and_check(graph, reset, outputs, ref)


@pytest.mark.parametrize("M,N,dtype", [(1500, 3000, "f16"), (300, 20480, "bf16"), (257, 32768, "f16")])
def test_layernorm_fwd_bwd_graph(M, N, dtype):
    """Register plans (3000), and 16-bit rows beyond 16384: the forward in a
    register plan and the wide backward (20480), both wide (32768)."""
    w = wl.LN1.scaled(M=M, N=N, dtype=dtype)
    _case(w.name, w.M, w.N)
    t = wl.make_inputs(w)
    x, wt, b, dy = (t[k].cuda() for k in ("x", "gamma", "beta", "dy"))
    y, dx = torch.empty_like(x), torch.empty_like(x)
    mean = torch.empty(w.M, dtype=torch.float32, device="cuda")
    rstd = torch.empty(w.M, dtype=torch.float32, device="cuda")
    dw = torch.empty(w.N, dtype=torch.float32, device="cuda")
    db = torch.empty(w.N, dtype=torch.float32, device="cuda")
    ws = torch.empty(rn.layernorm_bwd_workspace_bytes(w.M, w.N, x.dtype) // 4, dtype=torch.float32, device="cuda")

    def step():
        rn.layernorm_fwd(x, wt, b, y, mean, rstd, eps=w.eps)
        rn.layernorm_bwd(x, wt, dy, mean, rstd, dx, dw, db, ws)

    outputs = {"y": y, "mean": mean, "rstd": rstd, "dx": dx, "dw": dw, "db": db}
    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outputs.items()}
    graph = _capture(step)

    def reset():
        for v in outputs.values():
            v.fill_(float("nan"))

    _replay_and_check(graph, reset, outputs, ref)


def test_rope_and_swiglu_graph():
    rw = wl.ROPE1.scaled(tokens=1000)
    sw = wl.SWIGLU1.scaled(M=300, N=1000)
    _case(rw.name, rw.tokens, sw.name, sw.M, sw.N)
    rt = wl.make_rope_inputs(rw)
    q0, cos, sin, pos = rt["q"].cuda(), rt["cos"].cuda(), rt["sin"].cuda(), rt["positions"].cuda()
    q = q0.clone()
    st = wl.make_swiglu_inputs(sw)
    e, g_, dh = st["e"].cuda(), st["g"].cuda(), st["dh"].cuda()
    h, h2, df, de = (torch.empty_like(e) for _ in range(4))

    def step():
        rn.rope_fwd(q, cos, sin, pos)
        rn.swiglu_fwd(e, g_, h)
        rn.swiglu_bwd(dh, e, g_, h2, df, de)

    outputs = {"q": q, "h": h, "h2": h2, "df": df, "de": de}
    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outputs.items()}
    q.copy_(q0)
    graph = _capture(step)

    def reset():
        q.copy_(q0)
        for v in (h, h2, df, de):
            v.fill_(float("nan"))

    _replay_and_check(graph, reset, outputs, ref)
