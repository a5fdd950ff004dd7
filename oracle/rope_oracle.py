"""Plain float64 CPU oracle for the rotary position embedding (RoPE) and its
backward.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module; the HIP
library never imports it and the two share no code.

Source: [P1] "02 · 手写 Triton kernel:RMSNorm / RoPE / SwiGLU", section 4
(RoPE): each pair of dimensions (Q1, Q2) is rotated by its position's angle,
Q1' = Q1 cos - Q2 sin and Q2' = Q2 cos + Q1 sin; the rotation is invertible,
so the backward applies the same rotation with sin negated to the incoming
gradient and saves no activation.

Readings of points the page leaves open:

* The pairs are the two halves of a head, (d, d + D/2) for d < D/2 (the
  half-split pairing of the Hugging Face Llama implementation the walkthrough
  patches): Q1 = q[..., :D/2], Q2 = q[..., D/2:].
* cos and sin are inputs: tables [P, D/2] indexed by a token's position, in
  float64 here (their fp32 values on the GPU side are exact in float64).
* A token's position is positions[t] when given, else t mod seq_len.

Every function is pinned by ``tests/test_oracle.py`` (complex multiplication,
norm preservation, the relative-position property, inverse and transpose
checks by finite differences, quarter turns); none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np


def token_positions(n_tokens: int, seq_len: int, positions=None) -> np.ndarray:
    """Position of each token: the given positions, or t mod seq_len."""
    if positions is not None:
        return np.asarray(positions, dtype=np.int64)
    return np.arange(n_tokens, dtype=np.int64) % seq_len


def rotate(q, cos, sin, pos) -> np.ndarray:
    """q [T, H, D] rotated pairwise: (q1, q2) -> (q1 c - q2 s, q2 c + q1 s) with
    c = cos[pos[t]], s = sin[pos[t]] per token [P1 section 4]."""
    q = np.asarray(q, dtype=np.float64)
    half = q.shape[-1] // 2
    c = np.asarray(cos, dtype=np.float64)[pos][:, None, :]
    s = np.asarray(sin, dtype=np.float64)[pos][:, None, :]
    q1 = q[..., :half]
    q2 = q[..., half:]
    return np.concatenate([q1 * c - q2 * s, q2 * c + q1 * s], axis=-1)


def forward(q, cos, sin, pos) -> np.ndarray:
    """The forward rotation [P1 section 4]."""
    return rotate(q, cos, sin, pos)


def backward(dq, cos, sin, pos) -> np.ndarray:
    """The backward: the same rotation with sin negated, applied to the
    gradient [P1 section 4]."""
    return rotate(dq, cos, -np.asarray(sin, dtype=np.float64), pos)
