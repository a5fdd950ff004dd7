"""Plain float64 CPU oracle for LayerNorm forward and backward.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  The HIP
library in ``row_normalization_amd`` never imports it and has no CPU fallback;
the two share no code (only the seeded input generators in ``workloads.py``
feed both).

Source: [P4] "第 07 章:LayerNorm——反向传播与原子锁" (chuoer47.github.io, a
chapter on the Triton LayerNorm tutorial):

* section 1 ("前向内核 _layernorm_forward") and its forward kernel: per row the
  mean over the N columns, then the variance as the mean of the squared
  differences from that mean (a second pass), rstd = 1/sqrt(var + eps), and
  y = (x - mean) * rstd * w + b; mean and rstd are kept for the backward;
* section 3.0 (the chain-rule derivation) and the dLdx kernel of section 3.3:
  x_hat = (x - mean) * rstd, g = w * dy, c1 = sum(x_hat * g) / N,
  c2 = sum(g) / N, dx = (g - (x_hat * c1 + c2)) * rstd;
* sections 3.3-3.5: each row contributes dy * x_hat to dw and dy to db, and
  the weight and bias gradients are the sums of those contributions over all
  M rows.

Every value is computed in float64 from the exact float64 upcast of the
(quantised) inputs; mean and rstd are recomputed here and never taken from
the GPU.  Each function writes the page's steps out with whole-array numpy
operations: no blocking, fusion or reordering.

Readings of points the page leaves open:

* The variance is the biased one (divided by N, not N - 1), as the page's
  forward kernel divides the sum of squared differences by N.
* The page rounds each row's dw/db contribution to the weight's dtype and
  accumulates in that dtype; the oracle keeps every contribution and the sum
  exact in float64 (the rounding is an artefact of the page's lock scheme,
  not part of the gradient).

Every function here is pinned by ``tests/test_oracle.py`` (library forward
and autograd in float64, finite differences, exact rational moments, the
shift invariance of LayerNorm, closed forms for two-element and constant
rows); none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def moments(x) -> tuple[np.ndarray, np.ndarray]:
    """Per-row mean and biased variance, in the page's two passes [P4 section 1].

    mean_i = sum_j x_ij / N;  var_i = sum_j (x_ij - mean_i)^2 / N.
    """
    x = _f64(x)
    n = x.shape[1]
    mean = np.sum(x, axis=1) / n
    diff = x - mean[:, None]
    var = np.sum(diff * diff, axis=1) / n
    return mean, var


def forward(x, w, b, eps: float):
    """y = (x - mean) * rstd * w + b; returns (y [M,N], mean [M], rstd [M]) [P4 section 1]."""
    x = _f64(x)
    mean, var = moments(x)
    rstd = 1.0 / np.sqrt(var + eps)
    x_hat = (x - mean[:, None]) * rstd[:, None]
    y = x_hat * _f64(w)[None, :] + _f64(b)[None, :]
    return y, mean, rstd


def backward(x, w, dy, eps: float):
    """dx, dw and db of LayerNorm [P4 sections 3.0 and 3.3].

    x_hat = (x - mean) * rstd;  g = w * dy;  c1 = sum_j(x_hat * g) / N;
    c2 = sum_j(g) / N;  dx = (g - (x_hat * c1 + c2)) * rstd;
    dw = sum over rows of dy * x_hat;  db = sum over rows of dy.
    Returns (dx [M,N], dw [N], db [N]).
    """
    x = _f64(x)
    dy = _f64(dy)
    n = x.shape[1]
    mean, var = moments(x)
    rstd = 1.0 / np.sqrt(var + eps)
    x_hat = (x - mean[:, None]) * rstd[:, None]
    g = _f64(w)[None, :] * dy
    c1 = np.sum(x_hat * g, axis=1) / n
    c2 = np.sum(g, axis=1) / n
    dx = (g - (x_hat * c1[:, None] + c2[:, None])) * rstd[:, None]
    dw = column_sums(dy * x_hat)
    db = column_sums(dy)
    return dx, dw, db


def column_sums(contributions) -> np.ndarray:
    """Sum over rows of per-row contributions to a weight or bias gradient
    [P4 sections 3.4-3.5].  Also the oracle of the second-stage reduction when
    fed a table of partial rows directly."""
    return np.sum(_f64(contributions), axis=0)
