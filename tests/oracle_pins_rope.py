"""Pins for the fp64 RoPE oracle, written as functions of the oracle module.

Each ``pin_*`` takes a RoPE oracle module (the real one or a broken copy in
``test_oracle_mutants.py``) and checks it against facts fixed independently of
its code:

* complex multiplication: with z = q1 + i q2 and the unit phasor c + i s,
  the rotated pair is z (c + i s) (numpy complex arithmetic);
* a rotation preserves each pair's norm and, for true cos/sin tables, the
  dot product of a rotated query and key depends only on the difference of
  their positions (the property rotary embeddings are built for);
* the backward is both the inverse of the forward and its transpose: the
  gradient of sum(forward(q) * dy) with respect to q, by finite differences;
* a quarter turn (c = 0, s = 1) maps (q1, q2) to (-q2, q1); position 0 with
  angle zero is the identity; positions default to t mod seq_len.
"""
from __future__ import annotations

import numpy as np


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _tables(P, D, base=10000.0):
    """True cos/sin tables: angle p * base^(-2i/D) for pair i."""
    inv = base ** (-np.arange(0, D, 2, dtype=np.float64) / D)
    ang = np.arange(P, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max err {err:.3g} > {tol:.3g}"


def pin_rope_complex_multiplication(orc):
    g = _rng(0)
    T, H, D, P = 6, 3, 16, 10
    q = g.standard_normal((T, H, D))
    cos, sin = g.standard_normal((P, D // 2)), g.standard_normal((P, D // 2))  # any tables, not only unit phasors
    pos = g.integers(0, P, size=T)
    out = orc.forward(q, cos, sin, pos)
    z = (q[..., : D // 2] + 1j * q[..., D // 2:]) * (cos[pos] + 1j * sin[pos])[:, None, :]
    _close(out, np.concatenate([z.real, z.imag], axis=-1), 1e-12, "forward vs complex product")
    zb = (q[..., : D // 2] + 1j * q[..., D // 2:]) * (cos[pos] - 1j * sin[pos])[:, None, :]
    _close(orc.backward(q, cos, sin, pos), np.concatenate([zb.real, zb.imag], axis=-1), 1e-12,
           "backward vs conjugate product")


def pin_rope_preserves_pair_norms(orc):
    g = _rng(1)
    T, H, D = 9, 4, 32
    cos, sin = _tables(64, D)
    q = g.standard_normal((T, H, D))
    pos = g.integers(0, 64, size=T)
    out = orc.forward(q, cos, sin, pos)
    h = D // 2
    _close(out[..., :h] ** 2 + out[..., h:] ** 2, q[..., :h] ** 2 + q[..., h:] ** 2, 1e-12, "pair norms")


def pin_rope_relative_position(orc):
    """<R(p) q, R(p') k> depends only on p - p'."""
    g = _rng(2)
    D = 64
    cos, sin = _tables(512, D)
    q = g.standard_normal((1, 1, D))
    k = g.standard_normal((1, 1, D))
    dots = []
    for p, pk in ((10, 3), (107, 100), (407, 400)):
        rq = orc.forward(q, cos, sin, np.array([p]))
        rk = orc.forward(k, cos, sin, np.array([pk]))
        dots.append(float(np.sum(rq * rk)))
    assert max(dots) - min(dots) <= 1e-10 * max(1.0, abs(dots[0])), dots
    # and it does change with the offset
    r0 = float(np.sum(orc.forward(q, cos, sin, np.array([0])) * orc.forward(k, cos, sin, np.array([0]))))
    assert abs(r0 - dots[0]) > 1e-6


def pin_rope_backward_is_inverse(orc):
    g = _rng(3)
    T, H, D = 5, 2, 8
    cos, sin = _tables(16, D)
    q = g.standard_normal((T, H, D))
    pos = g.integers(0, 16, size=T)
    _close(orc.backward(orc.forward(q, cos, sin, pos), cos, sin, pos), q, 1e-12, "backward(forward(q))")


def pin_rope_backward_is_transpose(orc):
    """The gradient of L = sum(forward(q) * dy) w.r.t. q, by central differences,
    equals backward(dy) (any tables: this does not rely on orthogonality)."""
    g = _rng(4)
    T, H, D, P = 3, 2, 6, 5
    cos, sin = g.standard_normal((P, D // 2)), g.standard_normal((P, D // 2))
    q = g.standard_normal((T, H, D))
    dy = g.standard_normal((T, H, D))
    pos = g.integers(0, P, size=T)
    # the transpose of a rotation by (c, s) is the rotation by (c, -s) only
    # when it is applied with the same tables, which is what backward does
    fd = np.zeros_like(q)
    h = 1e-6
    for idx in np.ndindex(q.shape):
        e = np.zeros_like(q)
        e[idx] = h
        fd[idx] = (np.sum(orc.forward(q + e, cos, sin, pos) * dy) - np.sum(orc.forward(q - e, cos, sin, pos) * dy)) / (2 * h)
    _close(orc.backward(dy, cos, sin, pos), fd, 1e-7, "backward vs finite-difference gradient")


def pin_rope_quarter_turn_and_identity(orc):
    D = 4
    q = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    cos = np.array([[1.0, 1.0], [0.0, 0.0]])
    sin = np.array([[0.0, 0.0], [1.0, 1.0]])
    _close(orc.forward(q, cos, sin, np.array([0])), q, 0.0, "angle zero")
    _close(orc.forward(q, cos, sin, np.array([1])), [[[-3.0, -4.0, 1.0, 2.0]]], 0.0, "quarter turn")
    _close(orc.backward(q, cos, sin, np.array([1])), [[[3.0, 4.0, -1.0, -2.0]]], 0.0, "inverse quarter turn")
    assert D == 4


def pin_rope_positions(orc):
    assert list(orc.token_positions(7, 3)) == [0, 1, 2, 0, 1, 2, 0]
    assert list(orc.token_positions(3, 3, positions=[5, 0, 2])) == [5, 0, 2]


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
