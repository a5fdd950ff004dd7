"""Seeded random shapes for RoPE and SwiGLU against the oracles.

Drawn once from fixed seeds (a failure names a reproducible case).  RoPE:
tokens in [1, 600], heads in [1, 16], an even head_dim in [2, 256], table
positions by token index or drawn at random, table length in [1, 300], both
directions.  SwiGLU: M in [1, 400], N in [1, 20000], each operand a view with
its own padded row stride of one shared value (the ABI takes one stride), the
forward and the backward.  Same checks as the fixed-shape tests: the
per-dtype tolerance, and for 16-bit outputs at least 99.5 % of the elements
bit-identical to the oracle rounded to the I/O type.
"""
import numpy as np
import pytest
import torch

import row_normalization_amd as rn
import workloads as wl
from tests.parity import check_close
from tests.test_elementwise_gpu import _exact_fraction, _rope_oracle, _rope_run, _swiglu_check

pytestmark = pytest.mark.gpu


def _rope_cases(seed, n):
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(n):
        T = int(rng.integers(1, 601))
        H = int(rng.integers(1, 17))
        D = 2 * int(rng.integers(1, 129))
        out.append((str(rng.choice(["f32", "bf16", "f16"])), T, H, D, str(rng.choice(["mod", "random"])),
                    int(rng.integers(1, 301))))
    return out


def _swiglu_cases(seed, n):
    rng = np.random.Generator(np.random.PCG64(seed))
    return [(str(rng.choice(["f32", "bf16", "f16"])), int(rng.integers(1, 401)), int(rng.integers(1, 20001)),
             int(rng.choice([0, 0, 1, 8, 100]))) for _ in range(n)]


ROPE_CASES = _rope_cases(42, 14)
SWIGLU_CASES = _swiglu_cases(43, 14)


@pytest.mark.parametrize("case", ROPE_CASES, ids=[f"{a}-{b}x{c}x{d}-{e}-P{f}" for a, b, c, d, e, f in ROPE_CASES])
def test_rope_random_case(case):
    dtype, T, H, D, positions, seq_len = case
    w = wl.RopeWorkload(f"rope_{dtype}_{T}x{H}x{D}", dtype, T, H, D, seq_len=seq_len, positions=positions,
                        seed=T * 31 + H * 7 + D)
    for direction in ("fwd", "bwd"):
        print("case:", w.name, positions, seq_len, direction, flush=True)
        t, q = _rope_run(w, direction, positions=(positions == "random"))
        o = _rope_oracle(w, t, direction, positions=(positions == "random"))
        g = wl.to_f64(q)
        check_close(f"{w.name} {direction}", g.reshape(T, -1), o.reshape(T, -1), dtype, "y")
        _exact_fraction(f"{w.name} {direction}", g, o, dtype)


def _view(t, pad, fill):
    M, N = t.shape
    buf = torch.full((M, N + pad), fill, dtype=t.dtype, device="cuda")
    v = buf[:, :N]
    v.copy_(t.cuda())
    return v, buf


@pytest.mark.parametrize("case", SWIGLU_CASES, ids=[f"{a}-{b}x{c}-pad{d}" for a, b, c, d in SWIGLU_CASES])
def test_swiglu_random_case(case):
    dtype, M, N, pad = case
    w = wl.SwigluWorkload(f"swiglu_{dtype}_{M}x{N}", dtype, M, N, dh=("normal", 0.0, 1.0), seed=M * 13 + N)
    print("case:", w.name, "pad", pad, flush=True)
    t = wl.make_swiglu_inputs(w)
    (e, _), (g, _), (dh, _) = (_view(t[k], pad, 5.0) for k in ("e", "g", "dh"))
    (h, hbuf), (hb, _), (df, _), (de, _) = (_view(torch.zeros_like(t["e"]), pad, -3.0) for _ in range(4))
    rn.swiglu_fwd(e, g, h)
    rn.swiglu_bwd(dh, e, g, hb, df, de)
    torch.cuda.synchronize()
    _swiglu_check(w.name + " fwd", w, t, h)
    _swiglu_check(w.name + " bwd", w, t, hb, df, de)
    if pad:
        assert torch.all(hbuf[:, N:] == -3.0), "a store landed in the row padding"
