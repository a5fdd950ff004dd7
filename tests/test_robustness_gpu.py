"""Stream and row independence of the entry points on the GPU.

* Two streams at once: the library keeps no state between calls, so
  RMSNorm and LayerNorm steps issued concurrently on two streams (default
  priority) give results bit-identical to the same calls run alone.
* A non-finite row stays in its row: rows are independent in the forward and
  in dx, so a NaN or an infinity planted in one row of x leaves every other
  row's y, r and dx bit-identical to the run without it (the weight gradient
  sums over rows and does take the non-finite contribution).
* The Python binding rejects per-column vectors, scratch and partials of the
  wrong size, dtype or layout before anything is launched.
* The autograd adapters accept rows spaced apart (a column slice of a wider
  buffer) and give the dense copy's results and gradients.
"""
import pytest
import torch

import row_normalization_amd as rn
import workloads as wl

pytestmark = pytest.mark.gpu


def _case(*what):
    print("case:", *what, flush=True)


def _rms_buffers(w):
    t = wl.make_inputs(w)
    x, g, dy = t["x"].cuda(), t["gamma"].cuda(), t["dy"].cuda()
    return {
        "x": x, "g": g, "dy": dy, "y": torch.empty_like(x), "dx": torch.empty_like(x),
        "rstd": torch.empty(w.M, dtype=torch.float32, device="cuda"),
        "dg": torch.empty(w.N, dtype=torch.float32, device="cuda"),
        "ws": torch.empty(rn.rmsnorm_bwd_workspace_bytes(w.M, w.N, x.dtype) // 4, dtype=torch.float32, device="cuda"),
    }


def _rms_step(b, w, stream=None):
    rn.rmsnorm_fwd(b["x"], b["g"], b["y"], b["rstd"], eps=w.eps, gemma=w.gemma, stream=stream)
    rn.rmsnorm_bwd(b["x"], b["g"], b["dy"], b["rstd"], b["dx"], b["dg"], b["ws"], gemma=w.gemma, stream=stream)


def _ln_buffers(w):
    t = wl.make_inputs(w)
    x, wt, bias, dy = (t[k].cuda() for k in ("x", "gamma", "beta", "dy"))
    return {
        "x": x, "w": wt, "b": bias, "dy": dy, "y": torch.empty_like(x), "dx": torch.empty_like(x),
        "mean": torch.empty(w.M, dtype=torch.float32, device="cuda"),
        "rstd": torch.empty(w.M, dtype=torch.float32, device="cuda"),
        "dw": torch.empty(w.N, dtype=torch.float32, device="cuda"),
        "db": torch.empty(w.N, dtype=torch.float32, device="cuda"),
        "ws": torch.empty(rn.layernorm_bwd_workspace_bytes(w.M, w.N, x.dtype) // 4, dtype=torch.float32, device="cuda"),
    }


def _ln_step(b, w, stream=None):
    rn.layernorm_fwd(b["x"], b["w"], b["b"], b["y"], b["mean"], b["rstd"], eps=w.eps, stream=stream)
    rn.layernorm_bwd(b["x"], b["w"], b["dy"], b["mean"], b["rstd"], b["dx"], b["dw"], b["db"], b["ws"], stream=stream)


def test_two_streams_concurrently():
    wa = wl.C2.scaled(M=3000, N=4096)
    wb = wl.LN1.scaled(M=2500, N=3000)
    _case(wa.name, wa.M, wa.N, "|", wb.name, wb.M, wb.N)
    a, b = _rms_buffers(wa), _ln_buffers(wb)
    _rms_step(a, wa)
    _ln_step(b, wb)
    torch.cuda.synchronize()
    ref_a = {k: a[k].clone() for k in ("y", "rstd", "dx", "dg")}
    ref_b = {k: b[k].clone() for k in ("y", "mean", "rstd", "dx", "dw", "db")}
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        for k in ref_a:
            a[k].fill_(float("nan"))
        for k in ref_b:
            b[k].fill_(float("nan"))
        torch.cuda.synchronize()
        for _ in range(4):  # several steps in flight on each stream
            _rms_step(a, wa, stream=s1)
            _ln_step(b, wb, stream=s2)
        torch.cuda.synchronize()
        for k, v in ref_a.items():
            assert torch.equal(a[k], v), f"RMSNorm {k} differs when run beside another stream"
        for k, v in ref_b.items():
            assert torch.equal(b[k], v), f"LayerNorm {k} differs when run beside another stream"


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
@pytest.mark.parametrize("norm", ["rms", "ln"])
def test_non_finite_row_stays_in_its_row(norm, bad):
    w = (wl.C2 if norm == "rms" else wl.LN1).scaled(M=600, N=3000)
    _case(norm, w.M, w.N, bad)
    make, step = (_rms_buffers, _rms_step) if norm == "rms" else (_ln_buffers, _ln_step)
    clean = make(w)
    step(clean, w)
    dirty = make(w)
    bad_row, col = 257, 1234
    dirty["x"][bad_row, col] = bad
    step(dirty, w)
    torch.cuda.synchronize()
    keep = torch.ones(w.M, dtype=torch.bool, device="cuda")
    keep[bad_row] = False
    for k in ("y", "dx"):
        assert torch.equal(dirty[k][keep], clean[k][keep]), f"{k}: rows other than the planted one changed"
        assert not torch.isfinite(dirty[k][bad_row].float()).all(), f"{k}: the planted row shows no non-finite value"
    assert torch.equal(dirty["rstd"][keep], clean["rstd"][keep])


def test_binding_rejects_malformed_vectors_and_scratch():
    """The Python binding checks what the C ABI cannot (sizes and layouts of the
    per-column vectors, the scratch and the partials it is handed) and raises
    before anything is launched."""
    w = wl.C2.scaled(M=64, N=1024)
    _case(w.name, "malformed arguments")
    b = _rms_buffers(w)
    ln = _ln_buffers(wl.LN1.scaled(M=64, N=1024))
    y0 = b["y"].fill_(3.0).clone()
    bad = {
        "gamma too short": dict(g=b["g"][:-1]),
        "gamma of another dtype": dict(g=b["g"].float()),
        "strided gamma": dict(g=torch.cat([b["g"], b["g"]])[::2]),
        "strided rstd": dict(rstd=torch.empty(2 * w.M, dtype=torch.float32, device="cuda")[::2]),
    }
    for what, repl in bad.items():
        args = {**b, **repl}
        with pytest.raises(ValueError):
            rn.rmsnorm_fwd(args["x"], args["g"], args["y"], args["rstd"], eps=w.eps)
        with pytest.raises(ValueError):
            rn.rmsnorm_bwd(args["x"], args["g"], args["dy"], args["rstd"], args["dx"], args["dg"], args["ws"])
    torch.cuda.synchronize()
    assert torch.equal(b["y"], y0), "a rejected call wrote y"
    with pytest.raises(ValueError):  # scratch given as a strided view
        big = torch.empty(2 * b["ws"].numel(), dtype=torch.float32, device="cuda")
        rn.rmsnorm_bwd(b["x"], b["g"], b["dy"], b["rstd"], b["dx"], b["dg"], big[::2])
    with pytest.raises(ValueError):  # fewer partials than rows * N
        rn.rmsnorm_dgamma_reduce(b["ws"][:100], 8, w.N, b["dg"])
    with pytest.raises(ValueError):
        rn.layernorm_fwd(ln["x"], ln["w"][:-1], ln["b"], ln["y"], ln["mean"], ln["rstd"])
    with pytest.raises(ValueError):
        rn.layernorm_fwd(ln["x"], ln["w"], torch.cat([ln["b"], ln["b"]])[::2], ln["y"], ln["mean"], ln["rstd"])
    with pytest.raises(ValueError):
        rn.layernorm_dwdb_reduce(ln["ws"][:100], 8, 1024, ln["dw"], ln["db"])


def test_adapter_accepts_rows_with_a_row_stride():
    """x given to the autograd adapters as a column slice of a wider buffer
    (rows spaced apart) gives the same results as the dense copy."""
    w = wl.C2.scaled(M=96, N=1000)
    _case(w.name, "adapter on a strided view")
    t = wl.make_inputs(w)
    wide = torch.zeros(w.M, w.N + 40, dtype=t["x"].dtype, device="cuda")
    wide[:, :w.N] = t["x"].cuda()
    xv = wide[:, :w.N]
    xd = t["x"].cuda()
    g = t["gamma"].cuda()
    dy = t["dy"].cuda()
    assert torch.equal(rn.rmsnorm(xv, g, eps=w.eps), rn.rmsnorm(xd, g, eps=w.eps))
    ln_w, ln_b = torch.rand(w.N, device="cuda").to(t["x"].dtype), torch.rand(w.N, device="cuda").to(t["x"].dtype)
    assert torch.equal(rn.layernorm(xv, (w.N,), ln_w, ln_b), rn.layernorm(xd, (w.N,), ln_w, ln_b))
    # gradients through the strided view
    base = wide.clone().requires_grad_(True)
    y = rn.rmsnorm(base[:, :w.N], g, eps=w.eps)
    y.backward(dy)
    ref = xd.clone().requires_grad_(True)
    rn.rmsnorm(ref, g, eps=w.eps).backward(dy)
    assert torch.equal(base.grad[:, :w.N], ref.grad)
    assert torch.all(base.grad[:, w.N:] == 0)
