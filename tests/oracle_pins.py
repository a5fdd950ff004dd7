"""Pins for the fp64 CPU oracle, written as functions of the oracle module.

Each ``pin_*`` takes an oracle module (the real one, or a deliberately broken
copy in ``test_oracle_mutants.py``) and raises ``AssertionError`` when the
module disagrees with something fixed independently of it:

* values printed on the Triton RMSNorm tutorial (partitech.com), kept with
  their citations in ``tests/golden/worked_examples.json``;
* central finite differences of the oracle's own forward (the backward must be
  its derivative);
* closed forms and invariants that follow from the definition (scale
  invariance, the projection identity of dx, the all-zero row, the Gemma
  weight shift);
* an independent formula for dx (the Unsloth closed form from the Unsloth
  kernel walkthrough, section 3) and a library routine
  (``torch.nn.functional.rms_norm`` with CPU float64 autograd).

None of these re-types the oracle's own expressions.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _close_printed(value, printed, decimals, what):
    """``value`` rounds to what the page prints (half a unit in the last place)."""
    value = np.asarray(value, dtype=np.float64)
    printed = np.asarray(printed, dtype=np.float64)
    tol = 0.5 * 10.0 ** (-decimals) + 1e-12
    err = np.max(np.abs(value - printed))
    assert err <= tol, f"{what}: {value} vs printed {printed} (err {err:.3g} > {tol:.3g})"


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# --------------------------------------------------------------------------
# Values printed on the pages
# --------------------------------------------------------------------------

def pin_forward_two_values(orc):
    g = _golden()["forward_two_values"]
    x = np.array([g["x"]])
    r = orc.inverse_rms(x, g["eps"])
    _close_printed(r, [g["r"]], g["decimals"], "r")
    _close_printed(1.0 / r, [g["denominator"]], g["decimals"], "denominator")
    y, r2 = orc.forward(x, np.array(g["gamma"]), g["eps"])
    _close_printed(y[0], g["y"], g["decimals"], "y")
    _close_printed(r2, [g["r"]], g["decimals"], "r from forward")
    # the mean of squares the table prints: 1/r^2 - eps
    assert abs((1.0 / r[0] ** 2 - g["eps"]) - g["mean_of_squares"]) < 1e-9


def pin_forward_two_values_gamma(orc):
    g = _golden()["forward_two_values_gamma"]
    y, _ = orc.forward(np.array([g["x"]]), np.array(g["gamma"]), g["eps"])
    _close_printed(y[0], g["y"], g["decimals"], "y (gamma = [2, 0.5])")


def pin_backward_two_values(orc):
    g = _golden()["backward_two_values"]
    dx, _ = orc.backward(np.array([g["x"]]), np.array(g["gamma"]), np.array([g["dy"]]), g["eps"])
    _close_printed(dx[0], g["dx"], g["decimals"], "dx")
    # the printed u and mean(u*x) feed the page's formula; the first entry of
    # dx is negative although dy is positive.
    assert dx[0, 0] < 0 < dx[0, 1]


def pin_exercise_257_ones(orc):
    g = _golden()["exercise_257_ones"]
    for n in (257, 256):
        x = np.ones((1, n))
        y, r = orc.forward(x, np.full(n, g["gamma"]), g["eps"])
        c = g["correct"]
        _close_printed(y[0], np.full(n, c["y"]), c["decimals"], f"y, {n} ones")
        _close_printed(1.0 / r, [c["denominator"]], c["decimals"], f"denominator, {n} ones")
        # the padded-width bug value must not occur
        assert np.all(np.abs(y - g["padded_bug"]["y"]) > 0.1)


def pin_dgamma_sum_not_mean(orc):
    g = _golden()["dgamma_sum_not_mean"]
    s = orc.dgamma_from_rows(np.array(g["contributions"]))
    assert np.array_equal(s, np.array(g["sum"])), s
    assert not np.allclose(s, g["mean_wrong"])
    # The same table through the full backward: rows x = [1, 1] have
    # r = 1/sqrt(1 + eps), so with eps = 0 each row's contribution dy*x*r is
    # exactly its dy.
    x = np.ones((2, 2))
    dy = np.array(g["contributions"])
    _, dgamma = orc.backward(x, np.ones(2), dy, 0.0)
    assert np.allclose(dgamma, g["sum"], rtol=1e-15, atol=0), dgamma


def pin_dgamma_one_and_seventeen_rows(orc):
    """M=1: dgamma is that row's dy*x*r; M=17 identical rows: 17 times it."""
    g = _golden()["backward_two_values"]
    r_printed = _golden()["forward_two_values"]["r"]
    x1 = np.array([g["x"]])
    dy1 = np.array([g["dy"]])
    _, d1 = orc.backward(x1, np.array(g["gamma"]), dy1, g["eps"])
    # dy*x*r with the page's r: [3 r, 8 r]
    _close_printed(d1, [3 * r_printed, 8 * r_printed], 5, "dgamma, one row")
    _, d17 = orc.backward(np.repeat(x1, 17, 0), np.array(g["gamma"]), np.repeat(dy1, 17, 0), g["eps"])
    assert np.allclose(d17, 17.0 * d1, rtol=1e-14, atol=0), (d17, d1)


# --------------------------------------------------------------------------
# Finite differences of the oracle's forward
# --------------------------------------------------------------------------

def _fd_case(orc, M, N, gemma, seed, eps=1e-6):
    rng = _rng(seed)
    x = rng.standard_normal((M, N))
    gamma = rng.uniform(0.5, 1.5, N) if not gemma else rng.normal(0.0, 0.3, N)
    dy = rng.standard_normal((M, N))

    def loss(xv, gv):
        y, _ = orc.forward(xv, gv, eps, gemma)
        return float(np.sum(dy * y))

    dx_fd = np.empty((M, N))
    for i in range(M):
        for j in range(N):
            h = 1e-5 * max(1.0, abs(x[i, j]))
            xp = x.copy()
            xp[i, j] += h
            xm = x.copy()
            xm[i, j] -= h
            dx_fd[i, j] = (loss(xp, gamma) - loss(xm, gamma)) / (xp[i, j] - xm[i, j])
    dg_fd = np.empty(N)
    for j in range(N):
        h = 1e-5 * max(1.0, abs(gamma[j]))
        gp = gamma.copy()
        gp[j] += h
        gm = gamma.copy()
        gm[j] -= h
        dg_fd[j] = (loss(x, gp) - loss(x, gm)) / (gp[j] - gm[j])
    dx, dg = orc.backward(x, gamma, dy, eps, gemma)
    for name, an, fd in (("dx", dx, dx_fd), ("dgamma", dg, dg_fd)):
        scale = np.abs(an) + np.sqrt(np.mean(an**2))
        err = np.max(np.abs(an - fd) / scale)
        assert err < 1e-7, f"{name} vs central differences (M={M}, N={N}, gemma={gemma}): {err:.3g}"


def pin_finite_differences(orc):
    for k, (M, N) in enumerate([(1, 2), (3, 5), (17, 7), (2, 257)]):
        _fd_case(orc, M, N, gemma=False, seed=100 + k)
    for k, (M, N) in enumerate([(1, 3), (5, 6)]):
        _fd_case(orc, M, N, gemma=True, seed=200 + k)


# --------------------------------------------------------------------------
# Closed forms and invariants
# --------------------------------------------------------------------------

def pin_scale_invariance(orc):
    """With eps = 0: y(c x) = y(x), dx(c x) = dx(x)/c, dgamma(c x) = dgamma(x)."""
    rng = _rng(7)
    x = rng.standard_normal((6, 33))
    gamma = rng.uniform(0.5, 1.5, 33)
    dy = rng.standard_normal((6, 33))
    y0, _ = orc.forward(x, gamma, 0.0)
    dx0, dg0 = orc.backward(x, gamma, dy, 0.0)
    for c in (1e-3, 0.5, 7.0, 1e4):
        y, _ = orc.forward(c * x, gamma, 0.0)
        dx, dg = orc.backward(c * x, gamma, dy, 0.0)
        assert np.allclose(y, y0, rtol=1e-13, atol=0), c
        assert np.allclose(dx * c, dx0, rtol=1e-12, atol=1e-13), c
        assert np.allclose(dg, dg0, rtol=1e-12, atol=1e-13), c
    # with eps > 0 the output shrinks as the row shrinks (eps dominates)
    y_small, _ = orc.forward(1e-6 * x, gamma, 1e-6)
    assert np.all(np.abs(y_small) < np.abs(y0))


def pin_projection_identity(orc):
    """sum_j dx_ij x_ij = N * eps * r_i^3 * mean_j(dy_ij w_j x_ij); zero when eps = 0.

    Follows from the dx formula and r^2 = 1/(mean(x^2) + eps); it holds for
    either weight convention.
    """
    rng = _rng(11)
    M, N = 9, 40
    x = rng.standard_normal((M, N))
    dy = rng.standard_normal((M, N))
    for gemma in (False, True):
        gamma = rng.uniform(0.5, 1.5, N) if not gemma else rng.normal(0, 0.05, N)
        w = gamma + 1.0 if gemma else gamma
        for eps in (1e-6, 0.3):
            dx, _ = orc.backward(x, gamma, dy, eps, gemma)
            lhs = np.sum(dx * x, axis=1)
            s = np.mean(x**2, axis=1)
            rhs = N * eps * (s + eps) ** -1.5 * np.mean(dy * w * x, axis=1)
            assert np.allclose(lhs, rhs, rtol=1e-9, atol=1e-13), (lhs, rhs)
        dx0, _ = orc.backward(x, gamma, dy, 0.0, gemma)
        assert np.max(np.abs(np.sum(dx0 * x, axis=1))) < 1e-12
    # the two-value example: both sides equal 2.4890155675e-7
    g = _golden()["backward_two_values"]
    dx, _ = orc.backward(np.array([g["x"]]), np.array(g["gamma"]), np.array([g["dy"]]), g["eps"])
    assert abs(float(dx[0] @ np.array(g["x"])) - 2.4890155675e-7) < 1e-15


def pin_zero_row(orc):
    """An all-zero row: r = 1/sqrt(eps), y = 0, dx = r*dy*w, no dgamma contribution."""
    rng = _rng(13)
    N = 20
    x = rng.standard_normal((3, N))
    x[1] = 0.0
    gamma = rng.uniform(0.5, 1.5, N)
    dy = rng.standard_normal((3, N))
    eps = 1e-6
    y, r = orc.forward(x, gamma, eps)
    assert abs(r[1] - 1000.0) < 1e-9
    assert np.all(y[1] == 0.0)
    dx, dg = orc.backward(x, gamma, dy, eps)
    assert np.allclose(dx[1], 1000.0 * dy[1] * gamma, rtol=1e-12, atol=0)
    _, dg_without = orc.backward(x[[0, 2]], gamma, dy[[0, 2]], eps)
    assert np.allclose(dg, dg_without, rtol=1e-14, atol=0)


def pin_gemma_is_shifted_weight(orc):
    """Gemma with gamma equals the plain variant with 1 + gamma (exact in fp64)."""
    rng = _rng(17)
    M, N = 5, 24
    x = rng.standard_normal((M, N))
    dy = rng.standard_normal((M, N))
    gamma = np.round(rng.normal(0, 0.2, N) * 256) / 256  # 1 + gamma is exact
    yg, rg = orc.forward(x, gamma, 1e-6, True)
    yp, rp = orc.forward(x, gamma + 1.0, 1e-6, False)
    assert np.array_equal(yg, yp) and np.array_equal(rg, rp)
    dxg, dgg = orc.backward(x, gamma, dy, 1e-6, True)
    dxp, dgp = orc.backward(x, gamma + 1.0, dy, 1e-6, False)
    assert np.array_equal(dxg, dxp) and np.array_equal(dgg, dgp)
    # and it is not the plain variant with gamma itself
    assert not np.allclose(yg, orc.forward(x, gamma, 1e-6, False)[0])


def pin_unsloth_form(orc):
    """dx against the Unsloth closed form (kernel walkthrough, section 3):
    dX = r/n * (n * dY_W - normed * sum(dY_W * normed)), normed = x*r, dY_W = dy*W."""
    rng = _rng(19)
    M, N = 7, 65
    x = rng.standard_normal((M, N))
    dy = rng.standard_normal((M, N))
    for gemma in (False, True):
        gamma = rng.uniform(0.5, 1.5, N) if not gemma else rng.normal(0, 0.1, N)
        W = 1.0 + gamma if gemma else gamma
        r = orc.inverse_rms(x, 1e-6)[:, None]
        normed = x * r
        dYW = dy * W
        dX = r / N * (N * dYW - normed * np.sum(dYW * normed, axis=1, keepdims=True))
        dx, _ = orc.backward(x, gamma, dy, 1e-6, gemma)
        assert np.allclose(dx, dX, rtol=1e-12, atol=1e-14)


def pin_torch_library(orc):
    """Forward, dx and dgamma against torch.nn.functional.rms_norm (CPU fp64 autograd)."""
    import torch

    rng = _rng(23)
    for M, N, gemma in ((4, 257, False), (6, 64, True), (1, 3, False)):
        x = rng.standard_normal((M, N))
        dy = rng.standard_normal((M, N))
        gamma = rng.uniform(0.5, 1.5, N) if not gemma else rng.normal(0, 0.1, N)
        xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
        gt = torch.tensor(gamma, dtype=torch.float64, requires_grad=True)
        wt = 1.0 + gt if gemma else gt
        yt = torch.nn.functional.rms_norm(xt, (N,), weight=wt, eps=1e-6)
        yt.backward(torch.tensor(dy, dtype=torch.float64))
        y, _ = orc.forward(x, gamma, 1e-6, gemma)
        dx, dg = orc.backward(x, gamma, dy, 1e-6, gemma)
        assert np.allclose(y, yt.detach().numpy(), rtol=1e-13, atol=1e-15)
        assert np.allclose(dx, xt.grad.numpy(), rtol=1e-11, atol=1e-13)
        assert np.allclose(dg, gt.grad.numpy(), rtol=1e-11, atol=1e-13)


# --------------------------------------------------------------------------
# Rounding to the 16-bit I/O types and the rounded-normalised forward
# --------------------------------------------------------------------------

def pin_quantize_against_torch_casts(orc):
    """fp32 values rounded by the oracle equal torch's round-to-nearest-even casts."""
    import torch

    rng = _rng(29)
    v = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 1.0, 37.0, 1e3)]).astype(np.float32)
    for dtype, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        ref = torch.from_numpy(v).to(tdt).double().numpy()
        got = orc.quantize(v.astype(np.float64), dtype)
        assert np.array_equal(got, ref), (dtype, np.flatnonzero(got != ref)[:5])


def pin_quantize_ties_to_even(orc):
    """Halfway cases round to the even neighbour (hand-checked against the bit layouts)."""
    bf = orc.quantize(np.array([1 + 2.0**-8, 1 + 3 * 2.0**-8, -(1 + 2.0**-8), 2 + 2.0**-7, 1 + 2.0**-9]), "bf16")
    assert np.array_equal(bf, [1.0, 1 + 2.0**-6, -1.0, 2.0, 1.0]), bf
    hf = orc.quantize(np.array([1 + 2.0**-11, 1 + 3 * 2.0**-11, 1 + 2.0**-12, 65504.0]), "f16")
    assert np.array_equal(hf, [1.0, 1 + 2.0**-9, 1.0, 65504.0]), hf


def pin_normed_rounded_unit_weight(orc):
    """With w = 1 the two roundings collapse to one: T(T(x r) * 1) = T(x r)."""
    rng = _rng(31)
    x = rng.standard_normal((9, 70))
    for dtype in ("bf16", "f16"):
        y1, r1 = orc.forward_normed_rounded(x, np.ones(70), 1e-6, False, dtype)
        y0, r0 = orc.forward(x, np.ones(70), 1e-6)
        assert np.array_equal(y1, orc.quantize(y0, dtype)) and np.array_equal(r1, r0)
        # Gemma with gamma = 0 is the same unit weight
        y2, _ = orc.forward_normed_rounded(x, np.zeros(70), 1e-6, True, dtype)
        assert np.array_equal(y2, y1)


def pin_normed_rounded_against_torch(orc):
    """The Hugging Face order computed with torch on the CPU: normed (fp64 -> fp32 -> T), times the
    weight in T (torch multiplies 16-bit tensors in fp32 and rounds once).  Equal everywhere except
    where torch's fp32 intermediate lands exactly on a tie of T (double rounding; about one element
    in 2^16 for bf16, 2^13 for fp16), where the oracle rounds the exact value once."""
    import torch

    rng = _rng(37)
    x = rng.standard_normal((64, 512))
    bits = {"bf16": 8, "f16": 11}
    for dtype, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        gamma = torch.from_numpy(rng.uniform(0.5, 1.5, 512)).to(tdt)
        xt = torch.from_numpy(x)
        normed32 = (xt * torch.rsqrt(xt.square().mean(-1, keepdim=True) + 1e-6)).to(torch.float32)
        ref = (normed32.to(tdt) * gamma).double().numpy()
        got, _ = orc.forward_normed_rounded(x, gamma.double().numpy(), 1e-6, False, dtype)
        bad = np.flatnonzero(got != ref)
        m, _ = np.frexp(normed32.double().numpy().ravel()[bad])
        frac = np.abs(m) * 2.0 ** bits[dtype]
        assert np.all(frac - np.floor(frac) == 0.5), (dtype, bad)  # every mismatch is a tie in fp32
        assert len(bad) <= 8, (dtype, len(bad))
        # and it is a different function from one rounding of x r w
        single = orc.quantize(orc.forward(x, gamma.double().numpy(), 1e-6)[0], dtype)
        assert np.mean(single != got) > 0.05


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
