"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects every contract violation before launching anything.

No call here reaches a kernel launch: each argument set is invalid (or M == 0,
a documented no-op), so validation returns first.  The "device pointers" are
fake addresses that are never dereferenced.
"""
import ctypes
import subprocess

import pytest

import row_normalization_amd as rn
from row_normalization_amd import _lib

OK, E_NULL, E_SHAPE, E_STRIDE, E_ALIGN, E_DTYPE, E_EPS, E_ALIAS, E_WS, E_FLAG, E_HIP = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10
F32, BF16 = 0, 1
GiB = 1 << 30

# fake, well-separated, 256-byte-aligned device addresses
X, G, Y, R, DY, DX, WS, DG = (0x7F0000000000 + i * 4 * GiB for i in range(8))


@pytest.fixture(scope="module")
def L():
    # These calls pass fake device addresses and rely on validation failing
    # before any launch.  Where a GPU is visible, a mistake in an argument set
    # would launch a kernel on those addresses, so the fake-pointer tests run
    # only where there is no GPU (validation with real buffers is covered by
    # the GPU tests).
    import torch

    if torch.cuda.is_available():
        pytest.skip("fake-pointer validation tests run only without a GPU")
    return rn.lib()


def test_library_exports_every_declared_symbol(L):
    names = rn.header_functions()
    assert set(names) == {"rmsnorm_fwd", "rmsnorm_bwd_workspace_bytes", "rmsnorm_bwd_rows", "rmsnorm_dgamma_reduce",
                          "rmsnorm_bwd", "rmsnorm_bwd_noalloc", "rmsnorm_status_string", "layernorm_fwd", "layernorm_bwd_workspace_bytes",
                          "layernorm_bwd_rows", "layernorm_dwdb_reduce", "layernorm_bwd", "rope_fwd", "rope_bwd",
                          "swiglu_fwd", "swiglu_bwd"}
    for n in names:
        assert hasattr(L, n), n
    dyn = subprocess.run(["nm", "-D", "--defined-only", rn.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in dyn.splitlines() if " T " in line}
    assert set(names) <= exported


def test_library_has_gfx950_code_only():
    # the offload bundle ids name each code object's target
    import re

    with open(rn.LIB_PATH, "rb") as f:
        blob = f.read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa-[-\w:+]*", blob))
    assert targets == {b"amdgcn-amd-amdhsa--gfx950"}, targets


def test_status_strings(L):
    for code in range(-11, 1):
        assert rn.rmsnorm_status_string(code) not in ("", "unknown status")
    assert rn.rmsnorm_status_string(-99) == "unknown status"


def fwd(L, x=X, g=G, y=Y, r=R, M=4, N=8, stride=None, eps=1e-6, dtype=BF16, gemma=0):
    return L.rmsnorm_fwd(x, g, y, r, M, N, N if stride is None else stride, eps, dtype, gemma, None)


def test_fwd_rejections(L):
    assert fwd(L, dtype=7) == E_DTYPE
    assert fwd(L, dtype=-1) == E_DTYPE
    assert fwd(L, gemma=4) == E_FLAG
    assert fwd(L, M=-1) == E_SHAPE
    assert fwd(L, N=0) == E_SHAPE
    assert fwd(L, N=16385) == E_SHAPE
    assert fwd(L, stride=7) == E_STRIDE
    for eps in (0.0, -1e-6, float("inf"), float("nan")):
        assert fwd(L, eps=eps) == E_EPS
    for kw in ("x", "g", "y", "r"):
        assert fwd(L, **{kw: None}) == E_NULL
    assert fwd(L, x=X + 1) == E_ALIGN            # bf16 needs 2-byte alignment
    assert fwd(L, r=R + 2) == E_ALIGN            # rstd is fp32
    assert fwd(L, dtype=F32, g=G + 2) == E_ALIGN
    assert fwd(L, y=X) == E_ALIAS                # in-place forward is not offered
    assert fwd(L, y=X + 2 * 8 * 3) == E_ALIAS    # y overlaps the last row of x
    assert fwd(L, r=Y + 4) == E_ALIAS
    assert fwd(L, g=Y + 16) == E_ALIAS


def test_fwd_zero_rows_is_a_noop(L):
    # M == 0 returns before any HIP call, whatever the pointers
    assert L.rmsnorm_fwd(None, None, None, None, 0, 8, 8, 1e-6, BF16, 0, None) == OK
    # ... but the other arguments are still checked
    assert L.rmsnorm_fwd(None, None, None, None, 0, 0, 8, 1e-6, BF16, 0, None) == E_SHAPE
    assert L.rmsnorm_fwd(None, None, None, None, 0, 8, 8, 0.0, BF16, 0, None) == E_EPS


def test_workspace_query(L):
    out = ctypes.c_size_t(123)
    assert L.rmsnorm_bwd_workspace_bytes(0, 8, BF16, ctypes.byref(out)) == OK and out.value == 0
    assert L.rmsnorm_bwd_workspace_bytes(16384, 8192, BF16, ctypes.byref(out)) == OK
    assert out.value == 1024 * 8192 * 4  # at most 1024 fp32 partial rows
    assert L.rmsnorm_bwd_workspace_bytes(17, 257, F32, ctypes.byref(out)) == OK and out.value == 17 * 257 * 4
    assert L.rmsnorm_bwd_workspace_bytes(17, 0, F32, ctypes.byref(out)) == E_SHAPE
    assert L.rmsnorm_bwd_workspace_bytes(17, 8, 7, ctypes.byref(out)) == E_DTYPE
    assert L.rmsnorm_bwd_workspace_bytes(17, 8, F32, None) == E_NULL
    assert rn.rmsnorm_bwd_workspace_bytes(64, 128, 0) == 64 * 128 * 4


def bwd(L, x=X, g=G, dy=DY, r=R, dx=DX, dg=DG, ws=WS, wsb=None, M=4, N=8, stride=None, dtype=BF16, gemma=0):
    if wsb is None:
        wsb = M * N * 4
    return L.rmsnorm_bwd(x, g, dy, r, dx, dg, ws, wsb, M, N, N if stride is None else stride, dtype, gemma, None)


def bwd_rows(L, x=X, g=G, dy=DY, r=R, dx=DX, ws=WS, wsb=None, M=4, N=8, stride=None, dtype=BF16, gemma=0, rows=True):
    if wsb is None:
        wsb = M * N * 4
    out = ctypes.c_int64(-5)
    st = L.rmsnorm_bwd_rows(x, g, dy, r, dx, ws, wsb, M, N, N if stride is None else stride, dtype, gemma,
                            ctypes.byref(out) if rows else None, None)
    return st


@pytest.mark.parametrize("call", [bwd, bwd_rows])
def test_bwd_rejections(L, call):
    assert call(L, dtype=3) == E_DTYPE
    assert call(L, gemma=-1) == E_FLAG
    assert call(L, N=0) == E_SHAPE
    assert call(L, N=20000) == E_SHAPE
    assert call(L, M=-2) == E_SHAPE
    assert call(L, stride=4) == E_STRIDE
    for kw in ("x", "g", "dy", "r", "dx", "ws"):
        assert call(L, **{kw: None}) == E_NULL, kw
    assert call(L, dy=DY + 1) == E_ALIGN
    assert call(L, ws=WS + 2) == E_ALIGN
    assert call(L, wsb=4 * 8 * 4 - 1) == E_WS
    assert call(L, dx=X) == E_ALIAS              # dx over x
    assert call(L, dx=DY + 2) == E_ALIAS         # dx overlapping dy but not equal to it
    assert call(L, dx=R) == E_ALIAS
    assert call(L, ws=DY + 8) == E_ALIAS         # workspace inside dy
    assert call(L, ws=X) == E_ALIAS
    assert call(L, g=DX + 4) == E_ALIAS


def test_bwd_specific_rejections(L):
    assert bwd(L, dg=None) == E_NULL
    assert bwd(L, dg=DG + 2) == E_ALIGN
    assert bwd(L, dg=DX) == E_ALIAS
    assert bwd(L, dg=WS + 16) == E_ALIAS
    assert bwd(L, dg=G) == E_ALIAS
    assert bwd_rows(L, rows=False) == E_NULL
    # dgamma is checked even when M == 0 (it is written with zeros then)
    assert L.rmsnorm_bwd(None, None, None, None, None, None, None, 0, 0, 8, 8, BF16, 0, None) == E_NULL
    # the row pass alone with M == 0 is a no-op
    out = ctypes.c_int64(-5)
    assert L.rmsnorm_bwd_rows(None, None, None, None, None, None, 0, 0, 8, 8, BF16, 0, ctypes.byref(out), None) == OK
    assert out.value == 0


def noalloc(L, x=X, g=G, dy=DY, r=R, dx=DX, dg=DG, M=4, N=8, stride=None, dtype=BF16, gemma=0):
    return L.rmsnorm_bwd_noalloc(x, g, dy, r, dx, dg, M, N, N if stride is None else stride, dtype, gemma, None)


def test_bwd_noalloc_rejections(L):
    # the same validation as rmsnorm_bwd, before anything touches the GPU
    # (the static scratch is not even looked up on an invalid call)
    assert noalloc(L, dtype=3) == E_DTYPE
    assert noalloc(L, gemma=8) == E_FLAG
    assert noalloc(L, N=0) == E_SHAPE
    assert noalloc(L, N=16385) == E_SHAPE
    assert noalloc(L, M=-1) == E_SHAPE
    assert noalloc(L, M=(1 << 29) + 1) == E_SHAPE
    assert noalloc(L, stride=7) == E_STRIDE
    for kw in ("x", "g", "dy", "r", "dx", "dg"):
        assert noalloc(L, **{kw: None}) == E_NULL, kw
    assert noalloc(L, dy=DY + 1) == E_ALIGN
    assert noalloc(L, dg=DG + 2) == E_ALIGN
    assert noalloc(L, dx=X) == E_ALIAS
    assert noalloc(L, dx=DY + 2) == E_ALIAS
    assert noalloc(L, dg=DX) == E_ALIAS
    assert noalloc(L, g=DX + 4) == E_ALIAS
    assert noalloc(L, M=0, x=None, g=None, dy=None, r=None, dx=None, dg=None) == E_NULL  # dgamma still required
    assert rn.rmsnorm_status_string(-11).startswith("the launch plan needs more partial rows")


def test_dgamma_reduce_rejections(L):
    assert L.rmsnorm_dgamma_reduce(WS, -1, 8, DG, None) == E_SHAPE
    assert L.rmsnorm_dgamma_reduce(WS, 4, 0, DG, None) == E_SHAPE
    assert L.rmsnorm_dgamma_reduce(WS, 4, 16385, DG, None) == E_SHAPE
    # tables beyond RMSNORM_PARTIALS_MAX floats, including row counts whose
    # product with N wraps around int64 (1 << 62 rows x 4 columns wraps to 0)
    assert L.rmsnorm_dgamma_reduce(WS, (1 << 29) // 8 + 1, 8, DG, None) == E_SHAPE
    assert L.rmsnorm_dgamma_reduce(WS, 1 << 62, 4, DG, None) == E_SHAPE
    assert L.rmsnorm_dgamma_reduce(WS, 1 << 61, 8, DG, None) == E_SHAPE
    assert L.rmsnorm_dgamma_reduce(WS, (1 << 63) - 1, 16384, DG, None) == E_SHAPE
    assert L.rmsnorm_dgamma_reduce(WS, 4, 8, None, None) == E_NULL
    assert L.rmsnorm_dgamma_reduce(None, 4, 8, DG, None) == E_NULL
    assert L.rmsnorm_dgamma_reduce(WS + 1, 4, 8, DG, None) == E_ALIGN
    assert L.rmsnorm_dgamma_reduce(WS, 4, 8, WS + 32, None) == E_ALIAS


def test_python_binding_refuses_cpu_tensors():
    import torch

    x = torch.zeros(4, 8)
    with pytest.raises(ValueError, match="GPU tensors only"):
        rn.rmsnorm_fwd(x, torch.ones(8), torch.empty_like(x), torch.empty(4))
    with pytest.raises(ValueError):
        _lib._check(E_ALIAS, "probe")
    with pytest.raises(rn.RMSNormError):
        _lib._check(E_HIP, "probe")


def test_autograd_adapter_refuses_cpu_tensors():
    import torch

    x = torch.randn(4, 8, requires_grad=True)
    with pytest.raises(ValueError, match="GPU tensors only"):
        rn.rmsnorm(x, torch.ones(8))
    assert rn.RMSNorm(8, gemma=True).weight.detach().abs().sum() == 0


def test_flags_and_fp16_validation(L):
    assert fwd(L, gemma=4) == E_FLAG          # unknown flag bit
    assert fwd(L, gemma=-1) == E_FLAG
    assert bwd(L, gemma=8) == E_FLAG
    assert fwd(L, dtype=3) == E_DTYPE
    assert fwd(L, dtype=2, x=X + 1) == E_ALIGN  # fp16 needs 2-byte alignment
    # fp16, Gemma and the rounding-order flag are all accepted (M = 0: nothing is launched)
    assert L.rmsnorm_fwd(None, None, None, None, 0, 8, 8, 1e-6, 2, 3, None) == OK
    out = ctypes.c_size_t(0)
    assert L.rmsnorm_bwd_workspace_bytes(4, 8, 2, ctypes.byref(out)) == OK and out.value == 4 * 8 * 4
