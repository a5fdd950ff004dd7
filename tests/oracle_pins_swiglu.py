"""Pins for the fp64 SwiGLU oracle, written as functions of the oracle module.

Each ``pin_*`` takes a SwiGLU oracle module (the real one or a broken copy in
``test_oracle_mutants.py``) and checks it against facts fixed independently of
its code:

* library routines: ``torch.nn.functional.silu`` and ``torch.sigmoid`` in
  float64, and float64 autograd of silu(e) * g for the two gradients;
* central finite differences of the oracle's own exact forward;
* limits: silu(0) = 0 with slope 1/2, silu(e) -> e and its slope -> 1 for
  large e, silu(e) -> 0 with slope -> 0 for very negative e;
* the rounding order against torch's own 16-bit arithmetic on the CPU
  (f = silu(e) computed in fp32 and cast, then a bf16/fp16 product with g and
  with the incoming gradient); the oracle must agree bit for bit except
  where fp32 and fp64 evaluations of silu round f differently.
"""
from __future__ import annotations

import numpy as np
import torch


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"{what}: max err {err:.3g} > {tol * scale:.3g}"


def pin_swiglu_silu_matches_torch(orc):
    e = np.linspace(-30, 30, 1201)
    _close(orc.silu(e), torch.nn.functional.silu(torch.from_numpy(e)).numpy(), 1e-14, "silu")
    _close(orc.sigmoid(e), torch.sigmoid(torch.from_numpy(e)).numpy(), 1e-14, "sigmoid")


def pin_swiglu_exact_forward(orc):
    g = _rng(0)
    e, gg = g.standard_normal(500) * 3, g.standard_normal(500)
    want = torch.nn.functional.silu(torch.from_numpy(e)).numpy() * gg
    _close(orc.forward(e, gg, "f64"), want, 1e-14, "h = silu(e) g")


def pin_swiglu_autograd(orc):
    g = _rng(1)
    e, gg, dh = (g.standard_normal(400) * s for s in (3.0, 1.0, 0.5))
    et = torch.from_numpy(e).requires_grad_(True)
    gt = torch.from_numpy(gg).requires_grad_(True)
    (torch.nn.functional.silu(et) * gt).backward(torch.from_numpy(dh))
    h, df, de = orc.backward(dh, e, gg, "f64")
    _close(h, orc.forward(e, gg, "f64"), 0.0, "recomputed h")
    _close(df, gt.grad.numpy(), 1e-14, "df (gradient of g)")
    _close(de, et.grad.numpy(), 1e-13, "de (gradient of e)")


def pin_swiglu_finite_differences(orc):
    g = _rng(2)
    e, gg, dh = (g.standard_normal(12) * s for s in (2.0, 1.0, 1.0))
    hstep = 1e-6
    fde = np.array([(np.sum(orc.forward(e + hstep * np.eye(12)[i], gg, "f64") * dh)
                     - np.sum(orc.forward(e - hstep * np.eye(12)[i], gg, "f64") * dh)) / (2 * hstep) for i in range(12)])
    fdg = np.array([(np.sum(orc.forward(e, gg + hstep * np.eye(12)[i], "f64") * dh)
                     - np.sum(orc.forward(e, gg - hstep * np.eye(12)[i], "f64") * dh)) / (2 * hstep) for i in range(12)])
    _, df, de = orc.backward(dh, e, gg, "f64")
    _close(de, fde, 1e-8, "de vs finite differences")
    _close(df, fdg, 1e-8, "df vs finite differences")


def pin_swiglu_limits(orc):
    one = np.ones(1)
    # e = 0: silu 0, slope 1/2
    h, df, de = orc.backward(one * 3.0, np.zeros(1), one * 2.0, "f64")
    assert h[0] == 0.0 and df[0] == 0.0 and abs(de[0] - 3.0 * 2.0 * 0.5) < 1e-15
    # large e: silu(e) ~ e, slope ~ 1
    h, df, de = orc.backward(one, one * 40.0, one * 0.5, "f64")
    assert abs(h[0] - 20.0) < 1e-12 and abs(df[0] - 40.0) < 1e-12 and abs(de[0] - 0.5) < 1e-12
    # very negative e: silu(e) ~ 0, slope ~ 0 (but silu(-1) is about -0.2689)
    h, _, de = orc.backward(one, one * -40.0, one, "f64")
    assert abs(h[0]) < 1e-15 and abs(de[0]) < 1e-15
    assert abs(orc.silu(np.array([-1.0]))[0] + 0.2689414213699951) < 1e-15


def _torch_16bit(dtype, e, g, dh):
    """torch CPU: f = silu(e) in fp32, cast; h = f * g, df = dh * f in 16-bit."""
    td = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    et, gt, dht = (torch.from_numpy(a).to(td) for a in (e, g, dh))
    f = torch.nn.functional.silu(et.float()).to(td)
    return et, gt, dht, (f * gt).double().numpy(), (dht * f).double().numpy()


def pin_swiglu_rounding_order_vs_torch(orc):
    g = _rng(3)
    for dtype in ("bf16", "f16"):
        e0, g0, dh0 = (g.standard_normal(20000).astype(np.float32) * s for s in (2.0, 1.0, 0.1))
        et, gt, dht, h_t, df_t = _torch_16bit(dtype, e0, g0, dh0)
        # the same (rounded) inputs for both sides
        e, gg, dh = (t.double().numpy() for t in (et, gt, dht))
        h, df, _ = orc.backward(dh, e, gg, dtype)
        for name, mine, theirs in (("h", h, h_t), ("df", df, df_t), ("h (forward)", orc.forward(e, gg, dtype), h_t)):
            diff = mine != theirs
            # the only allowed differences: f rounded differently from an fp32 vs fp64 silu
            assert diff.mean() <= 1e-3, f"{dtype} {name}: {diff.mean():.4f} of elements differ from torch"
            if diff.any():
                ulp = np.abs(theirs[diff]) * (2.0 ** -7 if dtype == "bf16" else 2.0 ** -10)
                assert np.all(np.abs(mine[diff] - theirs[diff]) <= ulp * 1.01), f"{dtype} {name}: more than 1 ulp"


def pin_swiglu_de_rounded_once(orc):
    """de is the exact chain rule (checked against autograd above) rounded once
    to the I/O type, compared with torch's cast of the fp64 value.  torch may
    pass through fp32 on the way (a second rounding), so a difference is
    allowed only as a 1-ulp tie case, in at most 0.1 % of the elements."""
    g = _rng(4)
    e, gg, dh = (g.standard_normal(20000) * s for s in (2.0, 1.0, 0.1))
    for dtype, td, ulp in (("bf16", torch.bfloat16, 2.0 ** -7), ("f16", torch.float16, 2.0 ** -10)):
        _, _, de = orc.backward(dh, e, gg, dtype)
        _, _, exact = orc.backward(dh, e, gg, "f64")
        want = torch.from_numpy(exact).to(td).double().numpy()
        diff = de != want
        assert diff.mean() <= 1e-3, f"{dtype}: {diff.mean():.4f} of de differ from a single rounding"
        assert np.all(np.abs(de[diff] - want[diff]) <= np.abs(want[diff]) * ulp * 1.01)
        # and rounding happened at all
        assert np.mean(de != exact) > 0.9


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
