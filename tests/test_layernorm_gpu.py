"""LayerNorm parity on the GPU: the HIP path through the C ABI against the fp64
oracle on seeded inputs (the tolerance rules are in ``tests/parity_ln.py``)."""
import numpy as np
import pytest
import torch

import row_normalization_amd as rn
import workloads as wl
from oracle import layernorm_oracle as lo
from tests.parity_ln import LnRun, compare_ln_with_oracle

pytestmark = pytest.mark.gpu


def _print_case(*what):
    print("case:", *what, flush=True)


def test_unit_test_shape_1151x8192_fp16():
    """The LayerNorm chapter's unit-test shape and distributions, against the
    oracle in full, and against the chapter's own rule (atol 1e-2, rtol 0)."""
    w = wl.LN1
    _print_case(w.name)
    run = LnRun(w)
    compare_ln_with_oracle(run)
    x, wt, b, dy = (wl.to_f64(run.inputs[k]) for k in ("x", "gamma", "beta", "dy"))
    y_o, _, _ = lo.forward(x, wt, b, w.eps)
    dx_o, dw_o, db_o = lo.backward(x, wt, dy, w.eps)
    y_g, _, _, dx_g, dw_g, db_g = run.host()
    # the chapter rounds dw and db to fp16 before comparing; rounding the fp32
    # sums here as well keeps its rule meaningful
    dw16 = run.dw.to(torch.float16).double().cpu().numpy()
    db16 = run.db.to(torch.float16).double().cpu().numpy()
    for name, g, o in (("y", y_g, y_o), ("dx", dx_g, dx_o), ("dw", dw16, dw_o), ("db", db16, db_o)):
        err = np.max(np.abs(g - o))
        assert err <= 1e-2, f"{name}: max abs err {err:.3g} > 1e-2 (the chapter's rule)"


SMALL = [
    ("f32", 1, 1), ("f32", 3, 7), ("f32", 17, 33), ("f32", 64, 128), ("f32", 130, 1000), ("f32", 9, 16384),
    ("bf16", 1, 1), ("bf16", 5, 2), ("bf16", 33, 5120), ("bf16", 257, 4096), ("bf16", 20, 12288),
    ("f16", 2, 3), ("f16", 31, 96), ("f16", 100, 1024), ("f16", 1030, 1536), ("f16", 7, 15872), ("f16", 5, 16384),
    # partly empty last waves (planner's choice)
    ("f16", 67, 7680), ("bf16", 45, 2560), ("f16", 300, 3584), ("f16", 29, 13312), ("f32", 23, 3328),
    # one workgroup per CU, next row's loads in flight (3, 5, 3, 4 rows per workgroup)
    ("f16", 600, 12288), ("bf16", 1100, 9216), ("f32", 513, 8192), ("f16", 1024, 10240),
    # persistent forward with 7-wave rows of four vectors, ragged last row step
    ("bf16", 4100, 14336), ("f16", 4100, 11264), ("f32", 4100, 6144),   # and 6-wave rows (12 waves per CU)
    # forward rows of three waves' width run as one wave of 4 or 5 vectors
    ("f16", 300, 1232), ("bf16", 129, 2504),
    # more than a quarter of the vectors empty rather than one vector per lane
    ("f16", 100, 3200), ("bf16", 77, 2304), ("f32", 100, 1100), ("f32", 65, 704),
]


@pytest.mark.parametrize("dtype,M,N", SMALL, ids=[f"{d}-{m}x{n}" for d, m, n in SMALL])
def test_small_shapes(dtype, M, N):
    w = wl.Workload(f"ln_{dtype}_{M}x{N}", dtype, M, N, x=wl.LN1.x, gamma=wl.LN1.gamma, beta=wl.LN1.beta,
                    dy=wl.LN1.dy, eps=1e-5, seed=M * 7 + N)
    _print_case(w.name)
    compare_ln_with_oracle(LnRun(w))


# Forward shapes the planner gives four or five vectors per lane, at row
# counts where the forward grid is persistent with two multi-wave row groups
# per workgroup (the last row step ragged for 8195 and 8200 rows); and
# backward rows of 5-8 waves run as one workgroup of two or three row groups
# per CU with the next row's loads in flight; rows of 1-4 waves where the
# partial rows are a large share run one workgroup of their own shape per CU,
# pipelined, as well; forwards of 3-6 row steps run as 1024 persistent
# workgroups of one row group, and forwards of shorter rows as persistent
# grids of two to four row groups per workgroup where the rows divide
# evenly.  Each in place and not, with the split and the fused backward.
LARGE = [("f16", 8200, 5264), ("bf16", 16384, 6432), ("f16", 8195, 9216), ("f16", 4100, 6144), ("f32", 3000, 4096),
         ("f16", 4097, 8192), ("bf16", 4100, 8192), ("f16", 2049, 5120),
         # rows of 1-4 waves, one workgroup per CU, next row's loads in flight
         ("f16", 4100, 1024), ("f16", 4096, 2048), ("f16", 4096, 3072), ("f32", 4096, 2048), ("f16", 1000, 8192),
         # bf16 rows of 4-8 waves, not pipelined: one 16-wave workgroup per CU
         ("bf16", 4096, 4096), ("bf16", 1151, 8192), ("bf16", 4097, 6144),
         # forward of 3-6 row steps: 1024 persistent workgroups of one row group
         ("f16", 6000, 5632), ("bf16", 5000, 3584), ("f16", 2100, 7168),
         # rows of 2-7 KiB dividing evenly into row steps of a persistent grid
         # (4096 x 3072 above: 1024 workgroups of two 3-wave rows, two steps;
         # 768 workgroups of four 1-wave rows, and of two 4-wave rows, two steps)
         ("bf16", 6144, 2304), ("f16", 3072, 3328),
         # bf16 backward pipelined in its build for workgroups of at most 512
         # threads: rows of 1-4 waves, and of 8 waves where the partial rows are light
         ("bf16", 4100, 1024), ("bf16", 3000, 3072), ("bf16", 9000, 8192)]


@pytest.mark.parametrize("dtype,M,N", LARGE, ids=[f"{d}-{m}x{n}" for d, m, n in LARGE])
def test_persistent_and_wide_workgroup_shapes(dtype, M, N):
    w = wl.Workload(f"ln_{dtype}_{M}x{N}", dtype, M, N, x=wl.LN1.x, gamma=wl.LN1.gamma, beta=wl.LN1.beta,
                    dy=wl.LN1.dy, eps=1e-5, seed=M * 11 + N)
    for split, in_place in ((True, False), (False, True)):
        _print_case(w.name, "split" if split else "fused", "in place" if in_place else "")
        compare_ln_with_oracle(LnRun(w, split_bwd=split, in_place=in_place))


# 16-bit rows beyond 16384 elements, up to the chapter's 64 KB per row: the
# wide kernels (one 1024-thread workgroup per row; 16-byte vectors held in
# registers between the backward's passes, narrower ones read again; 32767
# takes the most chunks, 32 one-element vectors per lane), and for the
# forward of rows of at most 8 waves (11 with narrower vectors) the register
# plans (16392: 7 waves x 5 vectors; 20002: 2-element vectors; 20480 at 4100
# rows: 8 x 5, persistent).  More rows than the backward's 256 workgroups,
# so they loop; in place and not, split and fused.  The backward over 16-byte
# vectors loads each workgroup's next row during a row's second pass: three
# chunks with a ragged last step (300, 257 and 4100 rows: 44, 1 and 4 rows
# in it), four chunks over three steps (513 rows) and in one (33).
WIDE = [("f16", 300, 16392), ("bf16", 257, 24576), ("f16", 33, 32768), ("bf16", 20, 32767), ("f16", 600, 20002),
        ("bf16", 5, 16385), ("bf16", 513, 32768), ("f16", 4100, 20480)]


@pytest.mark.parametrize("dtype,M,N", WIDE, ids=[f"{d}-{m}x{n}" for d, m, n in WIDE])
def test_wide_rows(dtype, M, N):
    w = wl.Workload(f"ln_{dtype}_{M}x{N}", dtype, M, N, x=wl.LN1.x, gamma=wl.LN1.gamma, beta=wl.LN1.beta,
                    dy=wl.LN1.dy, eps=1e-5, seed=M * 13 + N)
    for split, in_place in ((True, False), (False, True)):
        _print_case(w.name, "split" if split else "fused", "in place" if in_place else "")
        compare_ln_with_oracle(LnRun(w, split_bwd=split, in_place=in_place))


def test_wide_rows_strided_and_misaligned():
    for N, stride, offset in ((32768, 32800, 0), (20000, 20003, 1), (16400, 16408, 4)):
        w = wl.LN1.scaled(M=40, N=N, dtype="bf16", seed=stride)
        _print_case(w.name, "stride", stride, "offset", offset)
        run = LnRun(w, row_stride=stride, offset=offset)
        compare_ln_with_oracle(run)
        pad = run.y.as_strided((w.M, stride - w.N), (stride, 1), run.y.storage_offset() + w.N)
        assert torch.all(pad == -7.0)


@pytest.mark.parametrize("N", [1024, 8192, 13312, 15872])
def test_sweep_points(N):
    """Points of the chapter's bandwidth sweep (M = 4096, fp16) in full."""
    w = wl.ln_sweep(N)
    _print_case(w.name)
    compare_ln_with_oracle(LnRun(w))


def test_in_place_dx_and_split_vs_fused_bitwise():
    w = wl.LN1.scaled(M=300, N=2048)
    _print_case(w.name, "in place / split / fused")
    a = LnRun(w, split_bwd=True, in_place=False)
    b = LnRun(w, split_bwd=False, in_place=True)
    compare_ln_with_oracle(b)
    for t in ("y", "mean", "rstd", "dx", "dw", "db"):
        assert torch.equal(getattr(a, t), getattr(b, t)), t


def test_strided_and_misaligned_views():
    for stride, offset in ((1000, 0), (1003, 1), (1024, 3)):
        w = wl.LN1.scaled(M=70, N=999 if offset else 1000, seed=stride)
        _print_case(w.name, "stride", stride, "offset", offset)
        run = LnRun(w, row_stride=stride, offset=offset)
        compare_ln_with_oracle(run)
        # padding between rows is never written
        pad = run.y.as_strided((w.M, stride - w.N), (stride, 1), run.y.storage_offset() + w.N)
        assert torch.all(pad == -7.0)


def test_deterministic():
    w = wl.LN1.scaled(M=2000, N=4096)
    _print_case(w.name, "determinism")
    a, b = LnRun(w), LnRun(w)
    for t in ("y", "mean", "rstd", "dx", "dw", "db"):
        assert torch.equal(getattr(a, t), getattr(b, t)), t


def test_inputs_untouched():
    w = wl.LN1.scaled(M=64, N=512)
    run = LnRun(w)
    assert torch.equal(run.x_gpu.cpu(), run.inputs["x"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [2, 3, 64, 1000])
def test_near_constant_rows(N, dtype):
    """Rows whose spread is near or below sqrt(eps) next to their values
    (x = 5 + 1e-3 z): the variance is about eps / 10, so eps decides rstd, and
    in fp32 the centering x - mean is what limits y and dx (the centering
    allowance of tests.parity_ln)."""
    w = wl.Workload(f"ln_near_const_{dtype}_{N}", dtype, 300, N, x=("normal", 5.0, 1e-3), gamma=wl.LN1.gamma,
                    beta=wl.LN1.beta, dy=wl.LN1.dy, eps=1e-5, seed=N)
    _print_case(w.name)
    compare_ln_with_oracle(LnRun(w))


def test_zero_rows_gives_zero_gradients():
    w = wl.LN1.scaled(M=0, N=256)
    _print_case(w.name)
    dw = torch.full((256,), float("nan"), device="cuda")
    db = torch.full((256,), float("nan"), device="cuda")
    x = torch.empty(0, 256, dtype=torch.float16, device="cuda")
    wt = torch.ones(256, dtype=torch.float16, device="cuda")
    m = torch.empty(0, device="cuda")
    rn.layernorm_bwd(x, wt, x, m, m, x, dw, db, torch.empty(1, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(dw == 0) and torch.all(db == 0)


def test_dwdb_reduce_against_oracle():
    rng = np.random.Generator(np.random.PCG64(5))
    for rows, N in ((1, 8), (37, 1000), (1024, 4096), (3, 5)):
        _print_case("dwdb reduce", rows, N)
        p = rng.standard_normal((2 * rows, N)).astype(np.float32)
        dw = torch.full((N,), float("nan"), device="cuda")
        db = torch.full((N,), float("nan"), device="cuda")
        rn.layernorm_dwdb_reduce(torch.from_numpy(p).cuda(), rows, N, dw, db)
        torch.cuda.synchronize()
        for got, want in ((dw, lo.column_sums(p[:rows])), (db, lo.column_sums(p[rows:]))):
            err = np.abs(wl.to_f64(got) - want) / (np.abs(want) + np.sqrt(np.mean(want ** 2)))
            assert err.max() <= 1e-5


def test_rejections_write_nothing():
    w = wl.LN1.scaled(M=8, N=64)
    t = wl.make_inputs(w)
    x = t["x"].cuda()
    wt = t["gamma"].cuda()
    y = torch.full_like(x, -3.0)
    mean = torch.full((8,), -3.0, device="cuda")
    with pytest.raises(ValueError):
        rn.layernorm_fwd(x, wt, wt, y, mean, mean, eps=1e-5)  # mean and rstd alias
    with pytest.raises(ValueError):
        rn.layernorm_fwd(x, wt, wt, y, mean, torch.empty(8, device="cuda"), eps=0.0)
    torch.cuda.synchronize()
    assert torch.all(y == -3.0) and torch.all(mean == -3.0)


# --------------------------------------------------------------------------
# autograd adapter
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_autograd_gradients(dtype):
    w = wl.LN1.scaled(M=48, N=768, dtype=dtype, seed=11)
    _print_case("autograd", w.name)
    t = wl.make_inputs(w)
    x = t["x"].cuda().view(4, 12, 768).requires_grad_(True)
    wt = t["gamma"].cuda().requires_grad_(True)
    b = t["beta"].cuda().requires_grad_(True)
    before = dict(rn.CALLS)
    y = rn.layernorm(x, (768,), wt, b, 1e-5)
    y.backward(t["dy"].cuda().view(4, 12, 768))
    assert rn.CALLS["ln_forward"] == before["ln_forward"] + 1
    assert rn.CALLS["ln_backward"] == before["ln_backward"] + 1
    xo, wo, bo, dyo = (wl.to_f64(t[k]) for k in ("x", "gamma", "beta", "dy"))
    y_o, _, r_o = lo.forward(xo, wo, bo, 1e-5)
    dx_o, dw_o, db_o = lo.backward(xo, wo, dyo, 1e-5)
    from tests.parity import check_close

    check_close("y", wl.to_f64(y).reshape(48, 768), y_o, dtype, "y")
    check_close("dx", wl.to_f64(x.grad).reshape(48, 768), dx_o, dtype, "dx", direct=wo * dyo * r_o[:, None])
    # the adapter returns dw and db in the parameters' dtype: compare after that rounding
    tol = {"f32": 1e-4, "bf16": 8e-3, "f16": 1e-3}[dtype]
    for name, g, o in (("dw", wt.grad, dw_o), ("db", b.grad, db_o)):
        err = np.abs(wl.to_f64(g) - o) / (np.abs(o) + np.sqrt(np.mean(o ** 2)))
        assert err.max() <= tol, (name, err.max())


@pytest.mark.parametrize("dtype,N", [("bf16", 20000), ("f16", 32768)])
def test_autograd_wide_rows(dtype, N):
    """The adapter on rows beyond 16384 elements (the wide kernels)."""
    w = wl.LN1.scaled(M=6, N=N, dtype=dtype, seed=13)
    _print_case("autograd wide", w.name)
    t = wl.make_inputs(w)
    x = t["x"].cuda().view(2, 3, N).requires_grad_(True)
    wt = t["gamma"].cuda().requires_grad_(True)
    b = t["beta"].cuda().requires_grad_(True)
    y = rn.layernorm(x, (N,), wt, b, 1e-5)
    y.backward(t["dy"].cuda().view(2, 3, N))
    xo, wo, bo, dyo = (wl.to_f64(t[k]) for k in ("x", "gamma", "beta", "dy"))
    y_o, _, r_o = lo.forward(xo, wo, bo, 1e-5)
    dx_o, dw_o, db_o = lo.backward(xo, wo, dyo, 1e-5)
    from tests.parity import check_close

    check_close("y", wl.to_f64(y).reshape(6, N), y_o, dtype, "y")
    check_close("dx", wl.to_f64(x.grad).reshape(6, N), dx_o, dtype, "dx", direct=wo * dyo * r_o[:, None])
    tol = {"bf16": 8e-3, "f16": 1e-3}[dtype]
    for name, g, o in (("dw", wt.grad, dw_o), ("db", b.grad, db_o)):
        err = np.abs(wl.to_f64(g) - o) / (np.abs(o) + np.sqrt(np.mean(o ** 2)))
        assert err.max() <= tol, (name, err.max())


def test_zero_rows_wide():
    """M = 0 with a wide row: a no-op forward, zero weight gradients."""
    N = 20000
    dw = torch.full((N,), float("nan"), device="cuda")
    db = torch.full((N,), float("nan"), device="cuda")
    x, y = (torch.empty(0, N, dtype=torch.bfloat16, device="cuda") for _ in range(2))
    wt, bias = (torch.ones(N, dtype=torch.bfloat16, device="cuda") for _ in range(2))
    mean, rstd = (torch.empty(0, device="cuda") for _ in range(2))
    rn.layernorm_fwd(x, wt, bias, y, mean, rstd, eps=1e-5)
    rn.layernorm_bwd(x, wt, x, mean, rstd, x, dw, db, torch.empty(1, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(dw == 0) and torch.all(db == 0)


def test_module_training_matches_fp64_reference():
    """A few SGD steps through the LayerNorm module on fp32 data track the same
    steps through torch's LayerNorm in CPU float64."""
    torch.manual_seed(0)
    N = 256
    mod = rn.LayerNorm(N, dtype=torch.float32, device="cuda")
    ref = torch.nn.LayerNorm(N, eps=1e-5, dtype=torch.float64)
    x = (-2.3 + 0.5 * torch.randn(64, N)).float()
    target = torch.randn(64, N).float()
    for _ in range(10):
        for m, dev, dt in ((mod, "cuda", torch.float32), (ref, "cpu", torch.float64)):
            out = m(x.to(dev, dt))
            loss = ((out - target.to(dev, dt)) ** 2).mean()
            m.zero_grad()
            loss.backward()
            with torch.no_grad():
                for p in m.parameters():
                    p -= 0.5 * p.grad
    for a, b in ((mod.weight, ref.weight), (mod.bias, ref.bias)):
        assert torch.max(torch.abs(a.detach().cpu().double() - b.detach())) < 1e-4
