"""Plain float64 CPU oracle for the elementwise SwiGLU forward and backward.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module; the HIP
library never imports it and the two share no code.

Source: [P1] "02 · 手写 Triton kernel:RMSNorm / RoPE / SwiGLU", section 5
(SwiGLU): the MLP is h = silu(X@G) * (X@U); the GEMMs stay with the BLAS
library and only the elementwise part is fused.  Forward: read e and g,
compute f = e * sigmoid(e) in fp32, cast f, then h = f * g.  Backward: one
kernel reads the incoming gradient DW (of h), e and g and writes, in place
over those three buffers, h (recomputed, for the next weight gradient),
df = DW * f (the gradient of g) and de (DW * g through the derivative of
silu).

Readings of points the page leaves open:

* "cast, then h = f * g": f is rounded to the I/O type before the product,
  so h = T(T(f) * g) with T round-to-nearest-even to the I/O type; the same
  T(f) enters df = T(DW * T(f)).
* de is the exact chain rule, rounded once: silu'(e) = s (1 + e (1 - s))
  with s = sigmoid(e), de = T(DW * g * silu'(e)).
* For fp32 I/O, T rounds to fp32; ``dtype="f64"`` disables rounding (the
  exact mathematics, used by the pins).

Every function is pinned by ``tests/test_oracle.py`` (torch's silu and fp64
autograd, finite differences, limits, the rounding order against torch's
bf16 arithmetic); none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

from .rmsnorm_oracle import quantize as _quantize_io


def _t(v, dtype: str) -> np.ndarray:
    """Round to the I/O type (identity for "f64")."""
    if dtype == "f64":
        return np.asarray(v, dtype=np.float64)
    return _quantize_io(v, dtype)


def sigmoid(e) -> np.ndarray:
    e = np.asarray(e, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-e))


def silu(e) -> np.ndarray:
    """f = e * sigmoid(e) [P1 section 5]."""
    e = np.asarray(e, dtype=np.float64)
    return e * sigmoid(e)


def forward(e, g, dtype: str) -> np.ndarray:
    """h = T(T(f) * g) with f = silu(e) [P1 section 5]."""
    f = _t(silu(e), dtype)
    return _t(f * np.asarray(g, dtype=np.float64), dtype)


def backward(dh, e, g, dtype: str):
    """(h, df, de) of the fused backward [P1 section 5]:
    h = T(T(f) g), df = T(dh T(f)) (the gradient of g),
    de = T(dh g sigmoid(e) (1 + e (1 - sigmoid(e)))) (the gradient of e)."""
    dh = np.asarray(dh, dtype=np.float64)
    e = np.asarray(e, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    s = sigmoid(e)
    f = _t(e * s, dtype)
    h = _t(f * g, dtype)
    df = _t(dh * f, dtype)
    de = _t(dh * g * s * (1.0 + e * (1.0 - s)), dtype)
    return h, df, de
