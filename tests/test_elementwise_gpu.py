"""RoPE and SwiGLU parity on the GPU: the HIP path through the C ABI against
the fp64 oracles on seeded inputs.

Tolerances: outputs are compared with ``tests.parity.check_close`` in the
form for their I/O dtype (fp32: 1e-5 relative against |o| + rms(o); bf16:
2e-2 + 1.6e-2 |o| and 4e-3 norm-wise; fp16: 3e-3 + 3e-3 |o| and 4e-3
norm-wise).  Both ops round each output once (SwiGLU's f once more, before
its products, in both the kernel and the oracle), so for 16-bit I/O nearly
every element must also be bit-identical to the oracle: at least 99.5 % of
them (a differing element comes from fp32 evaluation landing on the other
side of a rounding boundary than the fp64 value, about 1e-4 of them).  That
makes a dropped or misplaced rounding step visible even where it stays
inside the tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import row_normalization_amd as rn
import workloads as wl
from oracle import rope_oracle as ro
from oracle import swiglu_oracle as so
from tests.parity import check_close

pytestmark = pytest.mark.gpu


def _case(*what):
    print("case:", *what, flush=True)


def _exact_fraction(name, g, o, dtype, minimum=0.995):
    """Share of elements equal to the oracle's value rounded to the I/O type
    (SwiGLU's oracle already returns rounded values; rounding them again is
    the identity)."""
    if dtype == "f32":
        return 1.0
    frac = float(np.mean(g == oracle.quantize(o, dtype)))
    assert frac >= minimum, f"{name}: only {frac:.5f} of elements bit-identical to the oracle"
    return frac


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------

def _rope_run(w, direction="fwd", q_view=None, positions=True, seq_len=None):
    t = wl.make_rope_inputs(w)
    q = (t["q"] if direction == "fwd" else t["dq"]).cuda() if q_view is None else q_view
    cos, sin = t["cos"].cuda(), t["sin"].cuda()
    pos = t["positions"].cuda() if positions else None
    fn = rn.rope_fwd if direction == "fwd" else rn.rope_bwd
    fn(q, cos, sin, pos, seq_len)
    torch.cuda.synchronize()
    return t, q


def _rope_oracle(w, t, direction, positions=True, seq_len=None):
    src = t["q"] if direction == "fwd" else t["dq"]
    pos = ro.token_positions(w.tokens, seq_len or w.seq_len, t["positions"].numpy() if positions else None)
    f = ro.forward if direction == "fwd" else ro.backward
    return f(wl.to_f64(src), wl.to_f64(t["cos"]), wl.to_f64(t["sin"]), pos)


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_rope_full_size(direction):
    w = wl.ROPE1
    _case(w.name, direction)
    t, q = _rope_run(w, direction)
    o = _rope_oracle(w, t, direction)
    g = wl.to_f64(q)
    check_close(f"rope {direction}", g.reshape(w.tokens, -1), o.reshape(w.tokens, -1), w.dtype, "y")
    _exact_fraction(f"rope {direction}", g, o, w.dtype)


ROPE_SMALL = [
    ("f32", 7, 3, 8, "mod"), ("f32", 33, 5, 64, "random"), ("f32", 2, 1, 2, "mod"),
    ("bf16", 100, 8, 128, "random"), ("bf16", 17, 7, 6, "mod"), ("bf16", 1, 1, 256, "mod"),
    ("f16", 300, 4, 96, "random"), ("f16", 64, 9, 128, "mod"), ("f16", 5, 2, 1024, "random"),
]


@pytest.mark.parametrize("dtype,T,H,D,positions", ROPE_SMALL, ids=[f"{a}-{b}x{c}x{d}-{e}" for a, b, c, d, e in ROPE_SMALL])
def test_rope_small_shapes(dtype, T, H, D, positions):
    w = wl.RopeWorkload(f"rope_{dtype}_{T}x{H}x{D}", dtype, T, H, D, seq_len=50, positions=positions, seed=T + H + D)
    for direction in ("fwd", "bwd"):
        _case(w.name, positions, direction)
        t, q = _rope_run(w, direction, positions=(positions == "random"))
        o = _rope_oracle(w, t, direction, positions=(positions == "random"))
        g = wl.to_f64(q)
        check_close(f"{w.name} {direction}", g.reshape(T, -1), o.reshape(T, -1), dtype, "y")
        _exact_fraction(f"{w.name} {direction}", g, o, dtype)


def test_rope_strided_view_of_a_fused_qkv_buffer():
    """q is the first H*D columns of a [tokens, 3*H*D] buffer: the rest is untouched."""
    w = wl.RopeWorkload("rope_qkv_view", "bf16", 64, 4, 128, seq_len=64, seed=3)
    _case(w.name)
    t = wl.make_rope_inputs(w)
    buf = torch.full((64, 3 * 4 * 128), 7.0, dtype=torch.bfloat16, device="cuda")
    q = buf[:, : 4 * 128].view(64, 4, 128)
    q.copy_(t["q"].cuda())
    rn.rope_fwd(q, t["cos"].cuda(), t["sin"].cuda(), None, 64)
    torch.cuda.synchronize()
    o = ro.forward(wl.to_f64(t["q"]), wl.to_f64(t["cos"]), wl.to_f64(t["sin"]), ro.token_positions(64, 64))
    check_close("qkv view", wl.to_f64(q).reshape(64, -1), o.reshape(64, -1), "bf16", "y")
    assert torch.all(buf[:, 4 * 128:] == 7.0)


def test_rope_round_trip_and_out_of_table_positions():
    w = wl.RopeWorkload("rope_round_trip", "f32", 40, 6, 64, seq_len=32, positions="random", seed=9)
    _case(w.name)
    t = wl.make_rope_inputs(w)
    q = t["q"].cuda()
    cos, sin, pos = t["cos"].cuda(), t["sin"].cuda(), t["positions"].cuda()
    rn.rope_fwd(q, cos, sin, pos)
    rn.rope_bwd(q, cos, sin, pos)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(q.cpu() - t["q"])) < 1e-5
    # a position outside the table reads cos = sin = 0: that token becomes zeros, the others are rotated
    bad = pos.clone()
    bad[3] = 32
    bad[5] = -1
    q2 = t["q"].cuda()
    rn.rope_fwd(q2, cos, sin, bad)
    torch.cuda.synchronize()
    assert torch.all(q2[3] == 0) and torch.all(q2[5] == 0)
    assert torch.all(q2[4] != 0)


def test_rope_autograd():
    w = wl.RopeWorkload("rope_autograd", "bf16", 24, 4, 64, seq_len=24, seed=4)
    _case(w.name)
    t = wl.make_rope_inputs(w)
    leaf = t["q"].cuda().requires_grad_(True)
    before = dict(rn.CALLS)
    y = rn.rope_embedding(leaf * 1, t["cos"].cuda(), t["sin"].cuda(), None, 24)  # a non-leaf, rotated in place
    y.backward(t["dq"].cuda())
    assert rn.CALLS["rope_forward"] == before["rope_forward"] + 1 and rn.CALLS["rope_backward"] == before["rope_backward"] + 1
    pos = ro.token_positions(24, 24)
    c, s = wl.to_f64(t["cos"]), wl.to_f64(t["sin"])
    check_close("rope y", wl.to_f64(y).reshape(24, -1), ro.forward(wl.to_f64(t["q"]), c, s, pos).reshape(24, -1), "bf16", "y")
    check_close("rope grad", wl.to_f64(leaf.grad).reshape(24, -1),
                ro.backward(wl.to_f64(t["dq"]), c, s, pos).reshape(24, -1), "bf16", "y")


# --------------------------------------------------------------------------
# SwiGLU
# --------------------------------------------------------------------------

def _swiglu_check(name, w, t, h, df=None, de=None, rows=None):
    e, g, dh = (wl.to_f64(t[k]) for k in ("e", "g", "dh"))
    sel = slice(None) if rows is None else rows
    if df is None:
        ho = so.forward(e[sel], g[sel], w.dtype)
        hg = wl.to_f64(h)[sel]
        check_close(f"{name} h", hg, ho, w.dtype, "y")
        _exact_fraction(f"{name} h", hg, ho, w.dtype)
        return
    ho, dfo, deo = so.backward(dh[sel], e[sel], g[sel], w.dtype)
    for out, gpu, ref in (("h", h, ho), ("df", df, dfo), ("de", de, deo)):
        gg = wl.to_f64(gpu)[sel]
        check_close(f"{name} {out}", gg, ref, w.dtype, "y")
        _exact_fraction(f"{name} {out}", gg, ref, w.dtype)


def test_swiglu_full_size_sampled_rows():
    """11136 x 14336 bf16; every output row computed, 192 seeded rows compared
    in full (the op is elementwise, so rows are independent)."""
    w = wl.SWIGLU1
    _case(w.name)
    t = wl.make_swiglu_inputs(w)
    e, g, dh = (t[k].cuda() for k in ("e", "g", "dh"))
    h = torch.empty_like(e)
    rn.swiglu_fwd(e, g, h)
    hb, dfb, deb = torch.empty_like(e), torch.empty_like(e), torch.empty_like(e)
    rn.swiglu_bwd(dh, e, g, hb, dfb, deb)
    torch.cuda.synchronize()
    rows = np.sort(np.random.Generator(np.random.PCG64(1)).choice(w.M, 192, replace=False))
    rows = np.concatenate([rows, [0, w.M - 1]])
    _swiglu_check(w.name + " fwd", w, t, h, rows=rows)
    _swiglu_check(w.name + " bwd", w, t, hb, dfb, deb, rows=rows)
    assert torch.equal(h, hb)  # the recomputed h is the forward's h


SWIGLU_SMALL = [("f32", 5, 7), ("f32", 64, 1000), ("bf16", 1, 1), ("bf16", 33, 513), ("bf16", 128, 14336),
                ("f16", 3, 5), ("f16", 77, 4096), ("f16", 9, 70000)]


@pytest.mark.parametrize("dtype,M,N", SWIGLU_SMALL, ids=[f"{a}-{b}x{c}" for a, b, c in SWIGLU_SMALL])
def test_swiglu_small_shapes(dtype, M, N):
    w = wl.SwigluWorkload(f"swiglu_{dtype}_{M}x{N}", dtype, M, N, dh=("normal", 0.0, 1.0), seed=M + N)
    _case(w.name)
    t = wl.make_swiglu_inputs(w)
    e, g, dh = (t[k].cuda() for k in ("e", "g", "dh"))
    h = torch.empty_like(e)
    rn.swiglu_fwd(e, g, h)
    outs = [torch.empty_like(e) for _ in range(3)]
    rn.swiglu_bwd(dh, e, g, *outs)
    torch.cuda.synchronize()
    _swiglu_check(w.name + " fwd", w, t, h)
    _swiglu_check(w.name + " bwd", w, t, *outs)


def test_swiglu_in_place_over_inputs_on_a_fused_gate_up_buffer():
    """e and g are the two halves of one [M, 2N] buffer (row stride 2N); the
    backward writes h over dh, df over e and de over g, as on the page."""
    M, N = 50, 3000
    w = wl.SwigluWorkload("swiglu_inplace", "bf16", M, N, seed=5)
    _case(w.name)
    t = wl.make_swiglu_inputs(w)
    gu = torch.empty(M, 2 * N, dtype=torch.bfloat16, device="cuda")
    e, g = gu[:, :N], gu[:, N:]
    e.copy_(t["e"].cuda())
    g.copy_(t["g"].cuda())
    dh_buf = torch.empty(M, 2 * N, dtype=torch.bfloat16, device="cuda")
    dh = dh_buf[:, :N]
    dh.copy_(t["dh"].cuda())
    dh_buf[:, N:] = 3.0
    h = torch.empty(M, 2 * N, dtype=torch.bfloat16, device="cuda")[:, :N]
    rn.swiglu_fwd(e, g, h)
    torch.cuda.synchronize()
    _swiglu_check("fwd on views", w, t, h)
    rn.swiglu_bwd(dh, e, g, dh, e, g)
    torch.cuda.synchronize()
    _swiglu_check("in place", w, t, dh, e, g)
    assert torch.all(dh_buf[:, N:] == 3.0)


def test_swiglu_autograd():
    w = wl.SwigluWorkload("swiglu_autograd", "f32", 6, 40, dh=("normal", 0.0, 1.0), seed=8)
    _case(w.name)
    t = wl.make_swiglu_inputs(w)
    e = t["e"].cuda().view(2, 3, 40).requires_grad_(True)
    g = t["g"].cuda().view(2, 3, 40).requires_grad_(True)
    before = dict(rn.CALLS)
    h = rn.swiglu(e, g)
    h.backward(t["dh"].cuda().view(2, 3, 40))
    assert rn.CALLS["swiglu_backward"] == before["swiglu_backward"] + 1
    ho, dfo, deo = so.backward(*(wl.to_f64(t[k]) for k in ("dh", "e", "g")), "f32")
    check_close("h", wl.to_f64(h).reshape(6, 40), ho, "f32", "y")
    check_close("de", wl.to_f64(e.grad).reshape(6, 40), deo, "f32", "y")
    check_close("dg", wl.to_f64(g.grad).reshape(6, 40), dfo, "f32", "y")
