"""Plain float64 CPU oracle for RMSNorm forward and backward.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  The HIP
library in ``row_normalization_amd`` never imports it and has no CPU fallback;
the two share no code (only the seeded input generators in ``workloads.py``
feed both).

Sources (pages on RMSNorm; cited by title and section):

* [P2] "Hướng dẫn Triton RMSNorm: kernel, backward và…" (partitech.com):
  section "Vấn đề và công thức tham chiếu" (the reference formula: per-row
  inverse RMS with epsilon added under the root, output x*r*gamma); section
  "Vì sao cần một lượt đi và một lượt về?" (the backward formulas for dx and
  dgamma, mean over the N columns, sum over the M rows); section "Lập phương
  của r từ đâu?" (the derivative of r, which gives the r^3 term); section
  "Tổng không phải trung bình" (dgamma is a sum over rows, not a mean).
* [P1] "02 · 手写 Triton kernel:RMSNorm / RoPE / SwiGLU", section 3 (RMSNorm):
  the Gemma variant applies the weight as (1 + W).

Every value is computed in float64 from the exact float64 upcast of the
(quantised) inputs; r is recomputed here and never taken from the GPU.  Each
function is the definition written out with whole-array numpy operations: no
blocking, fusion or reordering.

Readings of points the pages leave open:

* Gemma weight: w = 1 + gamma, formed in float64.  The pages do not give the
  Gemma dgamma; by the chain rule d(1+gamma)/dgamma = 1, so it is the same
  sum of dy*x*r as the plain variant.
* The mean in r and in the dx projection divides by the true column count N.

* The rounding order of [P1] ("normed.to(W.dtype)" before "* W", the
  Hugging Face order) is ``forward_normed_rounded``: y = T(T(x*r) * w) with T
  round-to-nearest-even to the I/O type, x*r taken exactly (fp64) before its
  rounding.  ``forward`` is the single-rounding definition y = x*r*w.

Every function here is pinned by ``tests/test_oracle.py`` (worked values
printed on [P2], finite differences, closed-form identities, library
cross-checks); none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def weight(gamma, gemma: bool = False) -> np.ndarray:
    """Per-column weight: gamma, or (1 + gamma) for the Gemma variant [P1 §3]."""
    g = _f64(gamma)
    if gemma:
        return 1.0 + g
    return g


def inverse_rms(x, eps: float) -> np.ndarray:
    """r_i = 1 / sqrt(mean_j x_ij^2 + eps), one value per row [P2 reference formula]."""
    x = _f64(x)
    n = x.shape[1]
    mean_sq = np.sum(x * x, axis=1) / n
    return 1.0 / np.sqrt(mean_sq + eps)


def forward(x, gamma, eps: float, gemma: bool = False):
    """y_ij = x_ij * r_i * w_j; returns (y [M,N], r [M]) [P2 reference formula]."""
    x = _f64(x)
    r = inverse_rms(x, eps)
    w = weight(gamma, gemma)
    y = x * r[:, None] * w[None, :]
    return y, r


def backward(x, gamma, dy, eps: float, gemma: bool = False):
    """dx and dgamma of RMSNorm [P2 "Vì sao cần một lượt đi và một lượt về?"].

    u = dy * w;  m_i = mean_j(u_ij * x_ij)  (over the N columns);
    dx = r * u - x * r^3 * m;  dgamma_j = sum_i dy_ij * x_ij * r_i (over the M rows).
    Returns (dx [M,N], dgamma [N]).
    """
    x = _f64(x)
    dy = _f64(dy)
    n = x.shape[1]
    r = inverse_rms(x, eps)
    w = weight(gamma, gemma)
    u = dy * w[None, :]
    m = np.sum(u * x, axis=1) / n
    dx = r[:, None] * u - x * (r**3 * m)[:, None]
    dgamma = dgamma_from_rows(dy * x * r[:, None])
    return dx, dgamma


def dgamma_from_rows(contributions) -> np.ndarray:
    """Column sums of per-row dgamma contributions [P2 "Tổng không phải trung bình"].

    The weight gradient is the sum over rows of each row's contribution,
    never their mean.  Used both by ``backward`` and, fed a table of partial
    rows directly, as the oracle of the second-stage reduction.
    """
    return np.sum(_f64(contributions), axis=0)


# Significand bits (with the implicit one) of the 16-bit I/O types.
_SIGNIFICAND_BITS = {"bf16": 8, "f16": 11}


def quantize(v, dtype: str) -> np.ndarray:
    """v rounded to nearest (ties to even) in the I/O type, returned as float64.

    fp16 uses numpy's float16 conversion (correctly rounded, subnormals
    included); bf16 keeps 8 significant bits of the fp64 value (frexp gives
    m in [0.5, 1); m * 2^8 rounded half-to-even by ``np.round``).  bf16 has
    fp32's exponent range, far from anything these values reach.
    """
    v = _f64(v)
    if dtype == "f32":
        return v.astype(np.float32).astype(np.float64)
    if dtype == "f16":
        return v.astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        m, e = np.frexp(v)
        p = _SIGNIFICAND_BITS["bf16"]
        return np.ldexp(np.round(m * 2.0**p), e - p)
    raise ValueError(f"unknown dtype {dtype!r}")


def forward_normed_rounded(x, gamma, eps: float, gemma: bool, dtype: str):
    """y = T(T(x * r) * w): the normalised row rounded to the I/O type before
    the weight multiply, then the product rounded again [P1 §3].  Returns
    (y [M,N], r [M])."""
    x = _f64(x)
    r = inverse_rms(x, eps)
    normed = quantize(x * r[:, None], dtype)
    w = weight(gamma, gemma)
    return quantize(normed * w[None, :], dtype), r
