"""The autograd adapter (RMSNormFunction / RMSNorm) against the fp64 oracle.

GPU tests: gradients through ``loss.backward()`` are the C-ABI kernels' and are
compared with ``oracle.backward``.  The training test follows the integration
check of the Triton RMSNorm tutorial ("Kết nối Autograd và thực sự huấn luyện":
Linear -> RMSNorm -> SiLU -> Linear, a kernel branch against a reference branch
from the same initialisation); the reference branch here runs on the CPU in
float64 with ``torch.nn.RMSNorm``.  Plain SGD stands in for the tutorial's Adam
so that fp32-vs-fp64 noise on near-zero gradients cannot flip update signs.
"""
import numpy as np
import pytest
import torch

import oracle
import row_normalization_amd as rn
import workloads as wl
from tests.parity import check_close

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,shape,gemma", [("f32", (3, 5, 96), False), ("bf16", (2, 64, 8192), True),
                                               ("bf16", (130, 1000), False), ("f32", (7, 257), True)])
def test_autograd_matches_oracle(dtype, shape, gemma):
    N = shape[-1]
    M = int(np.prod(shape[:-1]))
    base = wl.C3 if gemma else wl.C2
    w = base.scaled(M=M, N=N, dtype=dtype, gemma=gemma, seed=M + N)
    if dtype == "f32":
        w = w.scaled(dy=("normal", 0.0, 1.0))
    t = wl.make_inputs(w)
    x = t["x"].reshape(shape).cuda().requires_grad_(True)
    g = t["gamma"].cuda().requires_grad_(True)
    dy = t["dy"].reshape(shape).cuda()
    before = dict(rn.CALLS)
    y = rn.rmsnorm(x, g, eps=w.eps, gemma=gemma)
    y.backward(dy)
    torch.cuda.synchronize()
    assert rn.CALLS["forward"] == before["forward"] + 1 and rn.CALLS["backward"] == before["backward"] + 1
    xs, gs, dys = (wl.to_f64(t[k]) for k in ("x", "gamma", "dy"))
    y_o, r_o = oracle.forward(xs, gs, w.eps, gemma)
    dx_o, dg_o = oracle.backward(xs, gs, dys, w.eps, gemma)
    direct = r_o[:, None] * dys * oracle.weight(gs, gemma)[None, :]
    check_close("autograd y", wl.to_f64(y).reshape(M, N), y_o, dtype, "y")
    check_close("autograd dx", wl.to_f64(x.grad).reshape(M, N), dx_o, dtype, "dx", direct=direct)
    # gamma.grad has gamma's dtype: the fp32 sum rounded once more to bf16
    got = wl.to_f64(g.grad)
    if dtype == "f32":
        check_close("autograd dgamma", got, dg_o, dtype, "dgamma")
    else:
        assert np.all(np.abs(got - dg_o) <= 2.0**-8 * np.abs(dg_o) + 1e-3 * np.sqrt(np.mean(dg_o**2)))


def test_module_and_noncontiguous_grad():
    layer = rn.RMSNorm(512, eps=1e-6, gemma=True, dtype=torch.float32, device="cuda")
    with torch.no_grad():
        layer.weight.copy_(torch.linspace(-0.2, 0.2, 512))
    x = torch.randn(40, 512, device="cuda", requires_grad=True)
    y = layer(x)
    # a transposed upstream gradient (non-contiguous) goes through dy.contiguous()
    dyT = torch.randn(512, 40, device="cuda").t()
    y.backward(dyT)
    xs = x.detach().double().cpu().numpy()
    gs = layer.weight.detach().double().cpu().numpy()
    dys = dyT.double().cpu().numpy()
    dx_o, dg_o = oracle.backward(xs, gs, dys, 1e-6, True)
    r_o = oracle.inverse_rms(xs, 1e-6)
    check_close("module dx", x.grad.double().cpu().numpy(), dx_o, "f32", "dx",
                direct=r_o[:, None] * dys * (1 + gs)[None, :])
    check_close("module dgamma", layer.weight.grad.double().cpu().numpy(), dg_o, "f32", "dgamma")


def test_training_matches_cpu_reference():
    torch.manual_seed(0)
    H, B, steps = 64, 32, 20

    def make(norm):
        return torch.nn.ModuleDict({"l1": torch.nn.Linear(16, H), "norm": norm, "l2": torch.nn.Linear(H, 1)})

    kernel_net = make(rn.RMSNorm(H, dtype=torch.float32)).cuda()
    ref_net = make(torch.nn.RMSNorm(H, eps=1e-6)).double()
    with torch.no_grad():
        for (n1, p1), (n2, p2) in zip(kernel_net.named_parameters(), ref_net.named_parameters()):
            p2.copy_(p1.detach().double().cpu())

    def run(net, xb):
        return net["l2"](torch.nn.functional.silu(net["norm"](net["l1"](xb))))

    opt_k = torch.optim.SGD(kernel_net.parameters(), lr=5e-2)
    opt_r = torch.optim.SGD(ref_net.parameters(), lr=5e-2)
    g = torch.Generator().manual_seed(1)
    calls = rn.CALLS["backward"]
    for _ in range(steps):
        xb = torch.randn(B, 16, generator=g)
        tb = xb[:, :1] * 0.5 - xb[:, 1:2] ** 2
        for net, opt, dev, dt in ((kernel_net, opt_k, "cuda", torch.float32), (ref_net, opt_r, "cpu", torch.float64)):
            opt.zero_grad()
            loss = torch.nn.functional.mse_loss(run(net, xb.to(dev, dt)), tb.to(dev, dt))
            loss.backward()
            opt.step()
    assert rn.CALLS["backward"] == calls + steps
    for (n1, p1), (n2, p2) in zip(kernel_net.named_parameters(), ref_net.named_parameters()):
        diff = (p1.detach().double().cpu() - p2.detach()).abs().max().item()
        assert diff < 1e-4, (n1, diff)


def test_adapters_inside_a_compiled_function():
    """A torch.compile'd function (Dynamo, eager backend) that calls the
    adapters runs them through the library (they are excluded from tracing)
    and matches the uncompiled function bit for bit."""
    torch.manual_seed(1)
    norm = rn.RMSNorm(256, eps=1e-6, dtype=torch.float32, device="cuda")
    lin = torch.nn.Linear(256, 256, device="cuda")
    lw, lb = torch.rand(256, device="cuda"), torch.rand(256, device="cuda")

    def f(x):
        return rn.layernorm(lin(norm(x)), (256,), lw, lb).square().sum()

    x = torch.randn(8, 256, device="cuda")
    eager = f(x)
    before = dict(rn.CALLS)
    compiled = torch.compile(f, backend="eager")(x)
    torch.cuda.synchronize()
    assert rn.CALLS["forward"] == before["forward"] + 1 and rn.CALLS["ln_forward"] == before["ln_forward"] + 1
    assert torch.equal(compiled, eager)
