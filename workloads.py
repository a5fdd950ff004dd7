"""Seeded synthetic inputs for the RMSNorm and LayerNorm forward/backward paths.

This module is shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()``:
it feeds the same quantised inputs to the fp64 CPU oracle and to the HIP
library.  It holds only random-number generation and dtype quantisation, none
of the normalisation arithmetic, so that the oracle and the GPU path share no
code that computes the method.

Recipe (the same for every workload):

* ``numpy.random.SeedSequence(seed).spawn(4)`` gives four independent PCG64
  streams, one each for x, gamma, dy and the choice of special rows.
* Values are drawn in float32 (``standard_normal``/``random`` with
  ``dtype=float32``), then shifted and scaled in float32.
* LayerNorm workloads also draw a bias from a fifth stream
  (``spawn(5)[4]``; the first four children of ``spawn(5)`` are those of
  ``spawn(4)``, so adding it changes no other input).
* Special rows (scaled by 100 / set to zero) are chosen from one permutation
  of the row indices: the first ``n_scaled`` rows of it are multiplied by 100
  (in float32, before quantisation), the next ``n_zero`` rows are zeroed, so
  the two sets are disjoint and their sizes exact.
* Quantisation to bf16 or fp16 uses torch's round-to-nearest-even cast on
  the CPU.
  The quantised tensors are the canonical inputs: the oracle upcasts them
  exactly to float64, the GPU receives the same bits.

"N(0, 1e-2)" for dy is read as a standard deviation of 1e-2.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclass(frozen=True)
class Workload:
    """One synthetic problem: shape, dtype and input distributions.

    ``x``, ``gamma`` (the weight), ``dy`` and ``beta`` (the LayerNorm bias;
    None for RMSNorm) are ``("normal", mean, std)`` or ``("uniform", low,
    high)``.
    """

    name: str
    dtype: str
    M: int
    N: int
    x: tuple = ("normal", 0.0, 1.0)
    gamma: tuple = ("normal", 1.0, 0.1)
    dy: tuple = ("normal", 0.0, 1e-2)
    eps: float = 1e-6
    gemma: bool = False
    dx_in_place: bool = False
    scaled_row_frac: float = 0.0
    zero_row_frac: float = 0.0
    seed: int = 0
    beta: tuple | None = None
    note: str = field(default="", compare=False)

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    @property
    def elsize(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def n_scaled(self) -> int:
        return int(round(self.scaled_row_frac * self.M))

    @property
    def n_zero(self) -> int:
        return int(round(self.zero_row_frac * self.M))

    def scaled(self, M: int | None = None, N: int | None = None, **kw) -> "Workload":
        """The same distributions at another shape (for small parity cases)."""
        return replace(self, M=self.M if M is None else M, N=self.N if N is None else N, **kw)


# The five workloads the method is measured on.  C3 is the headline one:
# Gemma weight (1 + gamma), dx written in place into dy's buffer.
C1 = Workload("c1_f32_64x128", "f32", 64, 128, gamma=("uniform", 0.5, 1.5), dy=("normal", 0.0, 1.0),
              note="fp32 parity case, seed 0")
C2 = Workload("c2_bf16_4096x4096", "bf16", 4096, 4096, gamma=("normal", 1.0, 0.1),
              note="batch 2 x seq 2048 tokens, hidden 4096")
C3 = Workload("c3_bf16_16384x8192_gemma_inplace", "bf16", 16384, 8192, gamma=("normal", 0.0, 0.02),
              gemma=True, dx_in_place=True, note="Gemma (1+gamma) weight, dx in place into dy")
C4 = Workload("c4_bf16_32768x5120_special_rows", "bf16", 32768, 5120, gamma=("uniform", 0.5, 1.5),
              scaled_row_frac=0.01, zero_row_frac=0.001,
              note="non-power-of-two N; 1% rows x100, 0.1% rows all zero")
C5 = Workload("c5_bf16_8192x16384", "bf16", 8192, 16384, gamma=("normal", 1.0, 0.1),
              note="wide rows spanning several wavefronts")

RMS_WORKLOADS = {"c1": C1, "c2": C2, "c3": C3, "c4": C4, "c5": C5}
HEADLINE = C3

# LayerNorm workloads, with the distributions of the LayerNorm chapter's unit
# test and benchmark: x = -2.3 + 0.5 N(0,1), weight and bias U(0,1),
# dy = 0.1 N(0,1), eps 1e-5, fp16.
_LN = dict(x=("normal", -2.3, 0.5), gamma=("uniform", 0.0, 1.0), beta=("uniform", 0.0, 1.0),
           dy=("normal", 0.0, 0.1), eps=1e-5)
LN1 = Workload("ln1_f16_1151x8192", "f16", 1151, 8192, note="the chapter's unit-test shape", **_LN)
# its GB/s sweep: M = 4096, N = 512 * i for i = 2 .. 31
LN_SWEEP_M = 4096
LN_SWEEP_NS = tuple(512 * i for i in range(2, 32))


def ln_sweep(N: int) -> Workload:
    """One point of the LayerNorm bandwidth sweep (M = 4096, fp16)."""
    return Workload(f"ln_f16_{LN_SWEEP_M}x{N}", "f16", LN_SWEEP_M, N, note="GB/s sweep point", **_LN)


LN_WORKLOADS = {"ln1": LN1, "ln_sweep_8192": ln_sweep(8192)}


def _draw(rng: np.random.Generator, spec: tuple, shape) -> np.ndarray:
    kind, a, b = spec
    if kind == "normal":
        out = rng.standard_normal(size=shape, dtype=np.float32)
        out *= np.float32(b)
        out += np.float32(a)
    elif kind == "uniform":
        out = rng.random(size=shape, dtype=np.float32)
        out *= np.float32(b - a)
        out += np.float32(a)
    else:
        raise ValueError(f"unknown distribution {kind!r}")
    return out


def special_rows(w: Workload) -> tuple[np.ndarray, np.ndarray]:
    """Row indices scaled by 100 and rows set to zero (disjoint, sorted)."""
    ss = np.random.SeedSequence(w.seed).spawn(4)[3]
    rng = np.random.Generator(np.random.PCG64(ss))
    if w.n_scaled + w.n_zero == 0:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    perm = rng.permutation(w.M)
    scaled = np.sort(perm[: w.n_scaled])
    zero = np.sort(perm[w.n_scaled : w.n_scaled + w.n_zero])
    return scaled, zero


def make_inputs(w: Workload) -> dict[str, torch.Tensor]:
    """Quantised CPU tensors ``x [M,N]``, ``gamma [N]``, ``dy [M,N]`` (and
    ``beta [N]`` for a LayerNorm workload) in ``w.dtype``."""
    ss = np.random.SeedSequence(w.seed).spawn(5)
    rx, rg, rdy = (np.random.Generator(np.random.PCG64(s)) for s in ss[:3])
    x = _draw(rx, w.x, (w.M, w.N))
    gamma = _draw(rg, w.gamma, (w.N,))
    dy = _draw(rdy, w.dy, (w.M, w.N))
    scaled, zero = special_rows(w)
    if scaled.size:
        x[scaled] *= np.float32(100.0)
    if zero.size:
        x[zero] = 0.0
    arrays = [("x", x), ("gamma", gamma), ("dy", dy)]
    if w.beta is not None:
        arrays.append(("beta", _draw(np.random.Generator(np.random.PCG64(ss[4])), w.beta, (w.N,))))
    out = {}
    for k, a in arrays:
        t = torch.from_numpy(a)
        out[k] = t if w.dtype == "f32" else t.to(w.torch_dtype)
    return out


# ---------------------------------------------------------------------------
# RoPE and SwiGLU (the other row/elementwise ops of the Unsloth walkthrough)
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class RopeWorkload:
    """q [tokens, heads, head_dim] rotated in place; cos/sin tables [seq_len, head_dim/2].

    positions: "mod" (token t at position t mod seq_len, i.e. a batch of
    sequences laid out one after another) or "random" (a seeded draw in
    [0, seq_len), as for packed sequences of mixed lengths)."""

    name: str
    dtype: str
    tokens: int
    heads: int
    head_dim: int
    seq_len: int
    base: float = 10000.0
    positions: str = "mod"
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    @property
    def elsize(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def scaled(self, **kw) -> "RopeWorkload":
        return replace(self, **kw)


def make_rope_inputs(w: RopeWorkload) -> dict[str, torch.Tensor]:
    """q and dq ~ N(0, 1) in ``w.dtype`` [T, H, D]; cos/sin fp32 [seq_len, D/2]
    from the usual frequency recipe (angle p * base^(-2i/D), computed in
    float64, stored as fp32); positions int32 [T]."""
    ss = np.random.SeedSequence(w.seed).spawn(3)
    rq, rd, rp = (np.random.Generator(np.random.PCG64(s)) for s in ss)
    shape = (w.tokens, w.heads, w.head_dim)
    q = rq.standard_normal(size=shape, dtype=np.float32)
    dq = rd.standard_normal(size=shape, dtype=np.float32)
    inv = w.base ** (-np.arange(0, w.head_dim, 2, dtype=np.float64) / w.head_dim)
    ang = np.arange(w.seq_len, dtype=np.float64)[:, None] * inv[None, :]
    if w.positions == "mod":
        pos = np.arange(w.tokens, dtype=np.int64) % w.seq_len
    else:
        pos = rp.integers(0, w.seq_len, size=w.tokens)
    out = {"cos": torch.from_numpy(np.cos(ang).astype(np.float32)),
           "sin": torch.from_numpy(np.sin(ang).astype(np.float32)),
           "positions": torch.from_numpy(pos.astype(np.int32))}
    for k, a in (("q", q), ("dq", dq)):
        t = torch.from_numpy(a)
        out[k] = t if w.dtype == "f32" else t.to(w.torch_dtype)
    return out


# Llama-7B/8B attention geometry: a batch of 4 sequences of 2048 tokens,
# 32 query heads of 128 dimensions.
ROPE1 = RopeWorkload("rope_bf16_8192tok_32x128", "bf16", 4 * 2048, 32, 128, 2048,
                     note="batch 4 x seq 2048, 32 heads x 128")


@dataclass(frozen=True)
class SwigluWorkload:
    """e (gate pre-activation), g (up projection) and dh [M, N]."""

    name: str
    dtype: str
    M: int
    N: int
    e: tuple = ("normal", 0.0, 1.0)
    g: tuple = ("normal", 0.0, 1.0)
    dh: tuple = ("normal", 0.0, 1e-2)
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    @property
    def elsize(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def scaled(self, **kw) -> "SwigluWorkload":
        return replace(self, **kw)


def make_swiglu_inputs(w: SwigluWorkload) -> dict[str, torch.Tensor]:
    ss = np.random.SeedSequence(w.seed).spawn(3)
    out = {}
    for k, spec, s in (("e", w.e, ss[0]), ("g", w.g, ss[1]), ("dh", w.dh, ss[2])):
        a = _draw(np.random.Generator(np.random.PCG64(s)), spec, (w.M, w.N))
        t = torch.from_numpy(a)
        out[k] = t if w.dtype == "f32" else t.to(w.torch_dtype)
    return out


# The token count and MLP width of the SwiGLU workload quoted in the packed
# SwiGLU note ([M, K, N] = [11136, 3584, 14336]): e and g are [11136, 14336].
SWIGLU1 = SwigluWorkload("swiglu_bf16_11136x14336", "bf16", 11136, 14336, note="M tokens x MLP width 14336")


def rope_algorithmic_bytes(tokens: int, heads: int, head_dim: int, elsize: int, seq_len: int) -> int:
    """One rotation pass: q read and written once, plus the two fp32 tables
    and (when given) the int32 positions.  Forward and backward are equal."""
    return 2 * tokens * heads * head_dim * elsize + 2 * seq_len * (head_dim // 2) * 4 + 4 * tokens


def swiglu_algorithmic_bytes(M: int, N: int, elsize: int) -> dict[str, int]:
    """fwd reads e and g and writes h; bwd reads dh, e and g and writes h, df and de."""
    return {"fwd": 3 * M * N * elsize, "bwd": 6 * M * N * elsize}


def algorithmic_bytes(M: int, N: int, elsize: int) -> dict[str, int]:
    """Bytes the method itself must move (no scratch): per pass and in total.

    fwd reads x and gamma, writes y and r (fp32 per row); bwd reads x, dy,
    gamma and r, writes dx and dgamma (fp32 per column).  The backward row
    kernel alone does everything but the dgamma write.
    """
    fwd = 2 * M * N * elsize + N * elsize + 4 * M
    bwd_rows = 3 * M * N * elsize + N * elsize + 4 * M
    bwd = bwd_rows + 4 * N
    return {"fwd": fwd, "bwd_rows": bwd_rows, "bwd": bwd, "fwd_bwd": fwd + bwd}


def ln_algorithmic_bytes(M: int, N: int, elsize: int) -> dict[str, int]:
    """LayerNorm's algorithmic bytes.  fwd reads x, weight and bias, writes y,
    mean and rstd (fp32 per row); bwd reads x, dy, weight, mean and rstd,
    writes dx and the fp32 dw and db.  (The chapter's own GB/s figures count
    2 * numel * elsize for the forward and 3 * numel * elsize for the
    backward: the same up to the O(M + N) terms.)"""
    fwd = 2 * M * N * elsize + 2 * N * elsize + 8 * M
    bwd_rows = 3 * M * N * elsize + N * elsize + 8 * M
    bwd = bwd_rows + 8 * N
    return {"fwd": fwd, "bwd_rows": bwd_rows, "bwd": bwd, "fwd_bwd": fwd + bwd}


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a (CPU or GPU) fp32/bf16 tensor to a float64 numpy array."""
    return t.detach().to("cpu", torch.float64).numpy()


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


assert math.isclose(algorithmic_bytes(16384, 8192, 2)["fwd_bwd"], 1_342_373_888)
