"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Every test here runs the gfx950 kernels (the library must load; there is no
fallback) on seeded inputs from ``workloads`` and compares every output with
``oracle`` under the tolerances written in ``tests/parity.py``.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import row_normalization_amd as rn
import workloads as wl
from tests.parity import Run, check_close, compare_with_oracle

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _name_the_case(request):
    _say(f"\n[gpu] {request.node.name}")
    yield


# ---------------------------------------------------------------------------
# The five workloads at their full sizes, in the launch sequence bench.py times
# (fwd, bwd row pass, dgamma reduction; C3 in place).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4", "c5"])
def test_workload_full_size(key):
    w = wl.RMS_WORKLOADS[key]
    run = Run(w)
    diag = compare_with_oracle(run)
    _say(f"{w.name}: partial rows {run.partial_rows}, {diag}")
    if w.dx_in_place:
        assert run.dx.data_ptr() != run.y.data_ptr()


def test_c4_special_rows():
    """Rows x100 and all-zero rows of C4: zero rows give r = 1/sqrt(eps), y = 0, dx = r*dy*w."""
    w = wl.C4.scaled(M=2000)  # 20 scaled rows, 2 zero rows
    run = Run(w)
    compare_with_oracle(run)
    scaled, zero = wl.special_rows(w)
    y, r, dx, _ = run.host()
    gamma = wl.to_f64(run.inputs["gamma"])
    dy = wl.to_f64(run.inputs["dy"])
    assert np.allclose(r[zero], 1000.0, rtol=2e-6)
    assert np.all(y[zero] == 0)
    check_close("zero rows dx", dx[zero], 1000.0 * dy[zero] * gamma, "bf16", "dx")


# ---------------------------------------------------------------------------
# Small and ragged shapes, several tiles each, every code path of the plan
# (16/8/4/2-byte vectors, 1..16 waves per row, persistent row loops).
# ---------------------------------------------------------------------------
SMALL = [
    # (dtype, M, N, gemma, in_place)
    ("f32", 17, 257, False, False),     # N=257: one-element vectors; the pages' denominator case
    ("bf16", 17, 257, False, False),
    ("f32", 17, 256, True, True),
    ("bf16", 33, 1000, False, False),   # 125 16-byte vectors: ragged last vector column
    ("bf16", 300, 5120, False, True),
    ("bf16", 257, 8192, True, True),    # the headline shape, fewer rows
    ("bf16", 100, 16384, False, False), # 8 waves per row in the backward
    ("f32", 40, 16384, True, False),
    ("f32", 64, 128, False, False),
    ("bf16", 1, 4096, False, False),    # M = 1
    ("f32", 1, 3, False, False),
    ("bf16", 5, 1, True, False),        # N = 1: dx is pure cancellation
    ("f32", 6, 1, False, True),
    ("bf16", 7, 2, False, True),
    ("bf16", 5000, 512, False, False),  # many rows per workgroup in the persistent backward
    ("f32", 3001, 96, True, True),
    ("bf16", 2, 12288, False, False),
    ("bf16", 9, 6, False, False),       # 4-byte vectors (3 per row)
    ("f32", 11, 10, False, False),      # 8-byte fp32 vectors
    ("f16", 17, 257, False, False),     # fp16 I/O
    ("f16", 33, 1000, True, False),
    ("f16", 257, 8192, True, True),
    ("f16", 100, 16384, False, False),
    ("f16", 4096, 4096, False, False),
    ("f16", 7, 12, False, True),
    # shapes whose last wave is partly empty by the planner's choice
    ("bf16", 67, 7680, True, True),     # 8 waves x 2 vectors, 64 of 1024 vectors empty
    ("f16", 45, 2560, False, False),    # 3 x 2, two row groups per workgroup
    ("bf16", 300, 3584, True, False),   # 4 x 2
    ("bf16", 129, 13312, False, False), # forward 7 x 4 (128 empty), backward 13 x 2
    ("f32", 23, 3328, False, False),    # fp32 7 x 2 rather than 13 x 1
    # one workgroup per CU: the backward keeps the next row's loads in flight
    # (odd and even numbers of rows per workgroup, in place)
    ("bf16", 600, 12288, True, True),   # 3 rows per workgroup
    ("f16", 1100, 9216, False, False),  # 5
    ("f32", 513, 8192, False, True),    # 3, fp32 16 x 2
    ("bf16", 1024, 10240, False, True), # 4
    # persistent forward with 7-wave rows of four vectors; the last of its 9
    # row steps holds rows for only some workgroups
    ("f32", 4100, 7168, False, True),
    ("bf16", 4097, 12800, True, False),
    # forward rows of three waves' width run as one wave of 4 or 5 vectors
    # (the last vectors of the lane partly or wholly past N)
    ("bf16", 700, 1232, False, True),
    ("f16", 300, 2504, True, False),
    # two or four vectors per lane with more than a quarter of the row's
    # vectors empty, rather than one vector per lane over 3-7 waves
    ("bf16", 300, 3200, False, True),   # 4 x 2 both ways
    ("f16", 200, 2304, True, False),    # backward 3 x 2
    ("f32", 150, 704, False, False),    # 2 x 2
    ("f32", 90, 1600, True, True),      # 4 x 2
    ("bf16", 129, 1096, False, False),  # forward one wave of 4
    # forward rows of 2-7 KiB dividing evenly into two row steps of a
    # persistent grid of 768 workgroups (four 2-wave rows, two 3-wave rows)
    ("bf16", 6144, 1792, True, True),
    ("f16", 3072, 2816, False, False),
    # backward rows of 5-8 waves where the partial rows would be a large share
    # of the traffic: one workgroup of two or three row groups per CU, the
    # next row's loads in flight (odd numbers of row steps: the loop runs one
    # step past the last, on rows past M)
    ("bf16", 2050, 8192, True, True),   # 8 x 2, 5 row steps
    ("f16", 3001, 6144, False, False),  # 6 x 2
    ("f32", 2000, 4096, False, True),   # fp32 8 x 2
    ("bf16", 1500, 5120, True, False),  # 5 x 2, three row groups (15 waves)
    # persistent forward of 4-wave rows, two row groups per workgroup
    ("bf16", 8200, 4096, False, True),
    # rows of 1-4 waves where the partial rows would be a large share: one
    # workgroup of the row shape per CU, at least four row steps each where
    # the grid keeps 8 waves per CU, the next row's loads in flight (2, 4, 5
    # and 6 row steps, the odd counts with a ragged last step)
    ("bf16", 4100, 2048, False, True),  # 2 x 2, four row groups per workgroup
    ("f16", 4096, 1024, True, False),   # 1 x 2, eight row groups
    ("bf16", 3000, 3072, False, False), # 3 x 2, two row groups (6 waves)
    ("f32", 4097, 1024, False, True),   # fp32 4 x 1 x 2
    ("bf16", 1151, 8192, True, True),   # 8 x 2 rows, 16-wave workgroups, 144 of them, 4 steps
    # forward of 3-4 row steps: 1024 persistent workgroups of one row group
    ("bf16", 4096, 4096, False, True),  # 4 x 2, 4 steps
    ("f16", 3500, 5120, True, False),   # 5 x 2, 4 steps, the last ragged
    ("bf16", 2049, 3584, False, False), # 4 x 2, 3 steps, one row in the last
]


@pytest.mark.parametrize("dtype,M,N,gemma,in_place", SMALL)
def test_small_shapes(dtype, M, N, gemma, in_place):
    base = wl.C3 if gemma else wl.C2
    w = base.scaled(M=M, N=N, dtype=dtype, gemma=gemma, dx_in_place=in_place, seed=M * 100003 + N)
    if dtype == "f32":
        w = w.scaled(dy=("normal", 0.0, 1.0))
    for split in (True, False):
        compare_with_oracle(Run(w, split_bwd=split))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("pad,offset", [(64, 0), (3, 0), (0, 1), (5, 3)])
def test_strided_and_misaligned(dtype, pad, offset):
    """Row stride > N and base pointers off the 16-byte grid; padding is never written."""
    w = wl.C2.scaled(M=70, N=1000, dtype=dtype, seed=pad * 10 + offset)
    run = Run(w, row_stride=1000 + pad, offset=offset)
    compare_with_oracle(run)
    if pad:
        for t in (run.y, run.dx):
            full = t.as_strided((70, 1000 + pad), (1000 + pad, 1))
            assert torch.all(full[:, 1000:].float() == -7.0)


@pytest.mark.parametrize("dtype,M,N,pad,in_place", [("bf16", 4096, 3072, 64, True), ("f16", 6144, 2304, 8, False)])
def test_strided_persistent_forward(dtype, M, N, pad, in_place):
    """Row stride > N on persistent forward grids of two row steps whose
    workgroups load their first row before unpacking the weight (two 3-wave
    rows per workgroup; four 1-wave rows), and the backward of the same rows;
    padding is never written (dx over dy keeps dy's NaN padding)."""
    w = wl.C3.scaled(M=M, N=N, dtype=dtype, gemma=True, dx_in_place=in_place, seed=M + N + pad)
    run = Run(w, row_stride=N + pad)
    compare_with_oracle(run)
    for t, fill in ((run.y, -7.0), (run.dx, float("nan") if in_place else -7.0)):
        pad_vals = t.as_strided((M, N + pad), (N + pad, 1))[:, N:].float()
        assert torch.all(torch.isnan(pad_vals)) if in_place and t is run.dx else torch.all(pad_vals == fill)


def test_inputs_untouched_and_outputs_complete():
    w = wl.C2.scaled(M=64, N=768)
    inputs = wl.make_inputs(w)
    run = Run(w, inputs=inputs)
    assert torch.equal(run.x_gpu.cpu().view(torch.int16), inputs["x"].view(torch.int16))
    y, r, dx, dg = run.host()
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(r)) and np.all(np.isfinite(dx)) and np.all(np.isfinite(dg))


# ---------------------------------------------------------------------------
# Determinism and the second stage on its own.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("key", ["c2", "c5"])
def test_bitwise_deterministic(key):
    w = wl.RMS_WORKLOADS[key].scaled(M=2048)
    inputs = wl.make_inputs(w)
    a, b = Run(w, inputs=inputs), Run(w, inputs=inputs)
    for ta, tb in ((a.y, b.y), (a.rstd, b.rstd), (a.dx, b.dx), (a.dgamma, b.dgamma)):
        assert torch.equal(ta.view(torch.int16) if ta.dtype == torch.bfloat16 else ta.view(torch.int32),
                           tb.view(torch.int16) if tb.dtype == torch.bfloat16 else tb.view(torch.int32))
    c = Run(w, inputs=inputs, split_bwd=False)
    assert torch.equal(a.dgamma.view(torch.int32), c.dgamma.view(torch.int32))


def test_dgamma_reduce_sum_not_mean():
    """The page's two-row table: column sums [4, 6], not means [2, 3]."""
    partials = torch.tensor([[1.0, 2.0], [3.0, 4.0]], device="cuda")
    out = torch.full((2,), float("nan"), device="cuda")
    rn.rmsnorm_dgamma_reduce(partials, 2, 2, out)
    torch.cuda.synchronize()
    assert out.tolist() == [4.0, 6.0]
    rn.rmsnorm_dgamma_reduce(partials, 1, 2, out)
    torch.cuda.synchronize()
    assert out.tolist() == [1.0, 2.0]


@pytest.mark.parametrize("rows,N", [(0, 8), (1, 1), (17, 3), (256, 8192), (300, 1001), (1024, 16384)])
def test_dgamma_reduce_against_oracle(rows, N):
    g = np.random.Generator(np.random.PCG64(rows * 7 + N))
    p = g.standard_normal((rows, N)).astype(np.float32)
    partials = torch.from_numpy(p).cuda() if rows else None
    out = torch.full((N,), float("nan"), device="cuda")
    rn.rmsnorm_dgamma_reduce(partials, rows, N, out)
    torch.cuda.synchronize()
    ref = oracle.dgamma_from_rows(p.astype(np.float64)) if rows else np.zeros(N)
    got = out.double().cpu().numpy()
    if rows == 0:
        assert np.all(got == 0)
    else:
        # fp32 sums of `rows` terms in a fixed order: error <= rows * 2^-24 * sum|terms|
        bound = rows * 2.0**-24 * np.sum(np.abs(p.astype(np.float64)), axis=0) + 1e-30
        assert np.all(np.abs(got - ref) <= bound)


def test_bwd_with_zero_rows_zeroes_dgamma():
    N = 40
    dg = torch.full((N,), float("nan"), device="cuda")
    e = torch.empty(0, N, dtype=torch.bfloat16, device="cuda")
    r = torch.empty(0, dtype=torch.float32, device="cuda")
    rn.rmsnorm_bwd(e, torch.ones(N, dtype=torch.bfloat16, device="cuda"), e, r, e, dg, None)
    rn.rmsnorm_fwd(e, torch.ones(N, dtype=torch.bfloat16, device="cuda"), e.clone(), r)
    torch.cuda.synchronize()
    assert torch.all(dg == 0)


def test_rejections_do_not_write():
    """A rejected call launches nothing: outputs keep their sentinel values."""
    w = wl.C2.scaled(M=16, N=256)
    t = wl.make_inputs(w)
    x, g = t["x"].cuda(), t["gamma"].cuda()
    y = torch.full_like(x, 3.0)
    r = torch.full((16,), 5.0, device="cuda")
    with pytest.raises(ValueError, match="E_EPS"):
        rn.rmsnorm_fwd(x, g, y, r, eps=0.0)
    with pytest.raises(ValueError, match="E_ALIAS"):
        rn.rmsnorm_fwd(x, g, x, r)
    torch.cuda.synchronize()
    assert torch.all(y == 3.0) and torch.all(r == 5.0)


# ---------------------------------------------------------------------------
# The Hugging Face rounding order (normalised value rounded before the weight
# multiply), against oracle.forward_normed_rounded.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,M,N,gemma", [("bf16", 300, 1000, False), ("f16", 300, 1000, False),
                                             ("bf16", 64, 8192, True), ("f16", 33, 257, False),
                                             ("bf16", 4096, 3072, True)])
def test_round_normed_order(dtype, M, N, gemma):
    w = (wl.C3 if gemma else wl.C2).scaled(M=M, N=N, dtype=dtype, gemma=gemma, seed=7 * M + N)
    t = wl.make_inputs(w)
    x, g = t["x"].cuda(), t["gamma"].cuda()
    outs = {}
    for rn_flag in (True, False):
        y = torch.empty_like(x)
        r = torch.empty(M, dtype=torch.float32, device="cuda")
        rn.rmsnorm_fwd(x, g, y, r, eps=w.eps, gemma=gemma, round_normed=rn_flag)
        torch.cuda.synchronize()
        outs[rn_flag] = wl.to_f64(y)
    xs, gs = wl.to_f64(t["x"]), wl.to_f64(t["gamma"])
    hf, r64 = oracle.forward_normed_rounded(xs, gs, w.eps, gemma, dtype)
    single = oracle.quantize(oracle.forward(xs, gs, w.eps, gemma)[0], dtype)
    # Exact except where the kernel's fp32 r flips the inner rounding T(x*r)
    # by one unit u_n of the normalised value: the products then differ by
    # |w| * u_n before the outer rounding, and the two outer roundings add up
    # to one unit u_y of y (so two units of y where |w| > 1 and the two
    # products straddle a rounding boundary: bf16 4096 x 3072 Gemma has one
    # such element in 12.6 million, and the kernel's value equals its fp32
    # arithmetic evaluated on the CPU).  Units are the spacing of the dtype's
    # grid in the binade of the value.
    mant = {"bf16": 7, "f16": 10}[dtype]
    unit = lambda v: np.ldexp(1.0, np.frexp(np.abs(v))[1] - 1 - mant)
    normed = oracle.quantize(xs * r64[:, None], dtype)
    bound = np.abs(oracle.weight(gs, gemma))[None, :] * unit(normed) + unit(hf)
    assert np.mean(outs[True] == hf) >= 0.999, np.mean(outs[True] == hf)
    assert np.all(np.abs(outs[True] - hf) <= bound)
    assert np.mean(outs[False] == single) >= 0.999
    assert np.mean(outs[True] != outs[False]) > 0.02  # the flag changes the result
