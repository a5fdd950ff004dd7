"""Pins for the fp64 LayerNorm oracle, written as functions of the oracle module.

Each ``pin_*`` takes a LayerNorm oracle module (the real one, or a broken copy
in ``test_oracle_mutants.py``) and raises ``AssertionError`` when the module
disagrees with something fixed independently of it:

* a library routine: ``torch.nn.functional.layer_norm`` in CPU float64, its
  forward and its autograd gradients;
* central finite differences of the oracle's own forward;
* exact rational arithmetic (``fractions.Fraction``) for the row moments;
* properties that follow from the definition: invariance under a per-row
  shift (so each row of dx sums to zero), two-element rows (whose normalised
  value is +-1 whatever x is, so dx vanishes), constant rows (y = b), rows of
  zero mean (where LayerNorm with b = 0 is RMSNorm), and the weight and bias
  gradients being sums over rows, not means.

The page on LayerNorm (the Triton LayerNorm tutorial chapter on
chuoer47.github.io) prints no numeric example, so there is no golden file for
it; none of these pins re-types the oracle's own expressions.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _case(seed, M, N, offset=-2.3, scale=0.5):
    """x ~ offset + scale * N(0,1), w, b ~ U(0,1), dy ~ 0.1 N(0,1): the page's test distributions."""
    g = _rng(seed)
    x = offset + scale * g.standard_normal((M, N))
    w = g.random(N)
    b = g.random(N)
    dy = 0.1 * g.standard_normal((M, N))
    return x, w, b, dy


def _assert_close(a, b, rtol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rtol * scale, f"{what}: max err {err:.3g} > {rtol * scale:.3g}"


# --------------------------------------------------------------------------
# Library routine (torch CPU float64)
# --------------------------------------------------------------------------

def pin_ln_torch_forward(orc):
    for seed, (M, N), eps in ((0, (7, 33), 1e-5), (1, (4, 512), 1e-6), (2, (3, 1), 1e-5)):
        x, w, b, _ = _case(seed, M, N)
        y, mean, rstd = orc.forward(x, w, b, eps)
        xt = torch.from_numpy(x)
        ref = torch.nn.functional.layer_norm(xt, (N,), torch.from_numpy(w), torch.from_numpy(b), eps)
        _assert_close(y, ref.numpy(), 1e-12, "y vs torch layer_norm")
        var_t, mean_t = torch.var_mean(xt, dim=1, unbiased=False)
        _assert_close(mean, mean_t.numpy(), 1e-13, "mean vs torch var_mean")
        _assert_close(rstd, (1.0 / torch.sqrt(var_t + eps)).numpy(), 1e-12, "rstd vs torch var")


def pin_ln_torch_autograd(orc):
    for seed, (M, N), eps in ((3, (5, 48), 1e-5), (4, (2, 7), 1e-3)):
        x, w, b, dy = _case(seed, M, N)
        dx, dw, db = orc.backward(x, w, dy, eps)
        xt = torch.from_numpy(x).requires_grad_(True)
        wt = torch.from_numpy(w).requires_grad_(True)
        bt = torch.from_numpy(b).requires_grad_(True)
        y = torch.nn.functional.layer_norm(xt, (N,), wt, bt, eps)
        y.backward(torch.from_numpy(dy))
        _assert_close(dx, xt.grad.numpy(), 1e-11, "dx vs torch autograd")
        _assert_close(dw, wt.grad.numpy(), 1e-11, "dw vs torch autograd")
        _assert_close(db, bt.grad.numpy(), 1e-11, "db vs torch autograd")


# --------------------------------------------------------------------------
# Derivatives of the oracle's own forward
# --------------------------------------------------------------------------

def pin_ln_finite_differences(orc):
    M, N, eps, h = 3, 6, 1e-2, 1e-6
    x, w, b, dy = _case(5, M, N, offset=0.7, scale=1.3)

    def loss(x_, w_, b_):
        return float(np.sum(orc.forward(x_, w_, b_, eps)[0] * dy))

    dx, dw, db = orc.backward(x, w, dy, eps)
    fdx = np.zeros_like(x)
    for i in range(M):
        for j in range(N):
            e = np.zeros_like(x)
            e[i, j] = h
            fdx[i, j] = (loss(x + e, w, b) - loss(x - e, w, b)) / (2 * h)
    fdw = np.array([(loss(x, w + h * np.eye(N)[j], b) - loss(x, w - h * np.eye(N)[j], b)) / (2 * h) for j in range(N)])
    fdb = np.array([(loss(x, w, b + h * np.eye(N)[j]) - loss(x, w, b - h * np.eye(N)[j])) / (2 * h) for j in range(N)])
    _assert_close(dx, fdx, 1e-7, "dx vs finite differences")
    _assert_close(dw, fdw, 1e-7, "dw vs finite differences")
    _assert_close(db, fdb, 1e-7, "db vs finite differences")


# --------------------------------------------------------------------------
# Exact arithmetic and closed forms
# --------------------------------------------------------------------------

def pin_ln_exact_moments(orc):
    """Mean and variance against exact rationals, on rows with a large offset
    (where E[x^2] - mean^2 in float64 would lose most of the variance)."""
    g = _rng(6)
    rows = [[10**8 + int(v) for v in g.integers(-3, 4, size=9)] for _ in range(4)]
    rows.append([1, 2, 3, 4, 5, 6, 7, 8, 9])
    mean, var = orc.moments(np.array(rows, dtype=np.float64))
    for i, r in enumerate(rows):
        n = len(r)
        m = Fraction(sum(r), n)
        v = sum((Fraction(t) - m) ** 2 for t in r) / n
        assert abs(mean[i] - float(m)) <= 1e-15 * abs(float(m)), f"row {i}: mean {mean[i]} vs {float(m)}"
        assert abs(var[i] - float(v)) <= 1e-12 * max(1.0, float(v)), f"row {i}: var {var[i]} vs exact {float(v)}"


def pin_ln_two_element_rows(orc):
    """N = 2, eps = 0: x_hat is (+1, -1) or (-1, +1) for any distinct pair, so
    y = w * x_hat + b and the input gradient vanishes."""
    x = np.array([[3.0, -1.0], [-0.25, 7.5], [1e-3, 2e-3]])
    w = np.array([1.5, -0.5])
    b = np.array([0.25, 2.0])
    y, mean, rstd = orc.forward(x, w, b, 0.0)
    s = np.sign(x[:, 0] - x[:, 1])
    want = np.stack([s * w[0] + b[0], -s * w[1] + b[1]], axis=1)
    _assert_close(y, want, 1e-12, "two-element y")
    _assert_close(mean, x.mean(axis=1), 1e-15, "two-element mean")
    _assert_close(rstd, 2.0 / np.abs(x[:, 0] - x[:, 1]), 1e-12, "two-element rstd")
    dy = np.array([[0.3, -2.0], [1.0, 1.0], [-4.0, 0.5]])
    dx, dw, db = orc.backward(x, w, dy, 0.0)
    _assert_close(dx, np.zeros_like(dx), 1e-9, "two-element dx")
    _assert_close(db, dy.sum(axis=0), 1e-15, "two-element db")
    _assert_close(dw, np.array([np.sum(dy[:, 0] * s), np.sum(-dy[:, 1] * s)]), 1e-12, "two-element dw")


def pin_ln_constant_row(orc):
    """A constant row has zero variance: y = b, rstd = 1/sqrt(eps).  A small
    perturbation d changes y by (d - mean(d)) * rstd * w to first order (the
    variance changes only at second order), so dx = rstd * (g - mean(g))."""
    N, eps = 8, 1e-4
    x = np.full((2, N), 3.25)
    x[1] = -1.0
    g = _rng(7)
    w = g.random(N) + 0.5
    b = g.standard_normal(N)
    dy = g.standard_normal((2, N))
    y, mean, rstd = orc.forward(x, w, b, eps)
    _assert_close(y, np.broadcast_to(b, (2, N)), 1e-15, "constant-row y")
    _assert_close(mean, [3.25, -1.0], 0.0, "constant-row mean")
    _assert_close(rstd, np.full(2, 1.0 / np.sqrt(eps)), 1e-12, "constant-row rstd")
    dx, dw, db = orc.backward(x, w, dy, eps)
    gw = dy * w
    _assert_close(dx, (gw - gw.mean(axis=1, keepdims=True)) / np.sqrt(eps), 1e-10, "constant-row dx")
    _assert_close(dw, np.zeros(N), 0.0, "constant-row dw")


def pin_ln_shift_invariance(orc):
    """y(x + c) = y(x) for any per-row shift c, so every row of dx sums to zero."""
    x, w, b, dy = _case(8, 6, 40)
    c = np.array([-5.0, 0.5, 3.0, 100.0, -0.01, 7.0])[:, None]
    y0, m0, r0 = orc.forward(x, w, b, 1e-5)
    y1, m1, r1 = orc.forward(x + c, w, b, 1e-5)
    _assert_close(y1, y0, 1e-11, "shifted y")
    _assert_close(m1 - m0, c[:, 0], 1e-11, "shifted mean")
    _assert_close(r1, r0, 1e-9, "shifted rstd")
    dx, _, _ = orc.backward(x, w, dy, 1e-5)
    scale = np.max(np.abs(dx))
    assert np.max(np.abs(dx.sum(axis=1))) <= 1e-12 * scale * x.shape[1], "rows of dx must sum to zero"


def pin_ln_zero_mean_rows_are_rmsnorm(orc):
    """On rows of mean zero the variance is the mean of squares, so LayerNorm
    with b = 0 is RMSNorm: y = x / sqrt(mean(x^2) + eps) * w, written here
    from that definition."""
    g = _rng(9)
    half = g.standard_normal((5, 16))
    x = np.concatenate([half, -half], axis=1)  # every row sums to zero exactly
    w = g.random(32)
    eps = 1e-5
    y, mean, _ = orc.forward(x, w, np.zeros(32), eps)
    assert np.all(np.abs(mean) <= 1e-15)
    ms = np.einsum("ij,ij->i", x, x) / 32
    _assert_close(y, x / np.sqrt(ms + eps)[:, None] * w, 1e-12, "zero-mean rows vs RMSNorm")


def pin_ln_gradients_sum_not_mean(orc):
    """dw and db are sums over rows: 17 copies of a row give 17 times one row's."""
    x, w, _, dy = _case(10, 1, 24)
    _, dw1, db1 = orc.backward(x, w, dy, 1e-5)
    _, dw17, db17 = orc.backward(np.repeat(x, 17, axis=0), w, np.repeat(dy, 17, axis=0), 1e-5)
    _assert_close(db1, dy[0], 1e-15, "one-row db")
    _assert_close(dw17, 17 * dw1, 1e-12, "17-row dw")
    _assert_close(db17, 17 * db1, 1e-12, "17-row db")


def pin_ln_column_sums(orc):
    _assert_close(orc.column_sums([[1.0, 2.0], [3.0, 4.0]]), [4.0, 6.0], 0.0, "column sums")
    _assert_close(orc.column_sums([[1.0, -2.0, 0.5]]), [1.0, -2.0, 0.5], 0.0, "one row")
    assert orc.column_sums(np.zeros((0, 3))).shape == (3,)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
