"""The LayerNorm C ABI on the CPU: every contract violation is rejected before
anything is launched.

As in ``test_abi.py``, each argument set is invalid (or M == 0, a documented
no-op), so validation returns first, and the "device pointers" are fake
addresses that are never dereferenced; the tests run only where no GPU is
visible.
"""
import ctypes

import pytest

import row_normalization_amd as rn

OK, E_NULL, E_SHAPE, E_STRIDE, E_ALIGN, E_DTYPE, E_EPS, E_ALIAS, E_WS = 0, -1, -2, -3, -4, -5, -6, -7, -8
F32, BF16, F16 = 0, 1, 2
GiB = 1 << 30

X, W, B, Y, MU, R, DY, DX, WS, DW, DB = (0x7F0000000000 + i * 4 * GiB for i in range(11))


@pytest.fixture(scope="module")
def L():
    import torch

    if torch.cuda.is_available():
        pytest.skip("fake-pointer validation tests run only without a GPU")
    return rn.lib()


def fwd(L, x=X, w=W, b=B, y=Y, mu=MU, r=R, M=4, N=8, stride=None, eps=1e-5, dtype=F16):
    return L.layernorm_fwd(x, w, b, y, mu, r, M, N, N if stride is None else stride, eps, dtype, None)


def test_fwd_rejections(L):
    assert fwd(L, dtype=3) == E_DTYPE
    assert fwd(L, M=-1) == E_SHAPE
    assert fwd(L, N=0) == E_SHAPE
    # 16-bit rows up to 32768 elements (the wide kernels), fp32 rows up to 16384
    assert fwd(L, N=32769) == E_SHAPE
    assert fwd(L, N=32769, dtype=BF16) == E_SHAPE
    assert fwd(L, N=16385, dtype=F32) == E_SHAPE
    assert fwd(L, stride=7) == E_STRIDE
    for eps in (0.0, -1e-5, float("inf"), float("nan")):
        assert fwd(L, eps=eps) == E_EPS
    for kw in ("x", "w", "b", "y", "mu", "r"):
        assert fwd(L, **{kw: None}) == E_NULL, kw
    assert fwd(L, x=X + 1) == E_ALIGN
    assert fwd(L, b=B + 1) == E_ALIGN
    assert fwd(L, mu=MU + 2) == E_ALIGN
    assert fwd(L, dtype=F32, w=W + 2) == E_ALIGN
    assert fwd(L, y=X) == E_ALIAS
    assert fwd(L, y=X + 2 * 8 * 3) == E_ALIAS     # y overlaps x's last row
    assert fwd(L, mu=R) == E_ALIAS                # mean and rstd share memory
    assert fwd(L, r=Y + 4) == E_ALIAS
    assert fwd(L, b=Y + 16) == E_ALIAS
    assert fwd(L, mu=W) == E_ALIAS


def test_fwd_zero_rows_is_a_noop(L):
    assert L.layernorm_fwd(None, None, None, None, None, None, 0, 8, 8, 1e-5, F16, None) == OK
    assert L.layernorm_fwd(None, None, None, None, None, None, 0, 0, 8, 1e-5, F16, None) == E_SHAPE
    assert L.layernorm_fwd(None, None, None, None, None, None, 0, 8, 8, 0.0, F16, None) == E_EPS


def test_workspace_query(L):
    out = ctypes.c_size_t(7)
    assert L.layernorm_bwd_workspace_bytes(0, 8, F16, ctypes.byref(out)) == OK and out.value == 0
    assert L.layernorm_bwd_workspace_bytes(4096, 8192, F16, ctypes.byref(out)) == OK
    assert out.value == 2 * 1024 * 8192 * 4  # two tables of at most 1024 fp32 partial rows
    assert L.layernorm_bwd_workspace_bytes(17, 257, F32, ctypes.byref(out)) == OK and out.value == 2 * 17 * 257 * 4
    assert L.layernorm_bwd_workspace_bytes(17, 0, F32, ctypes.byref(out)) == E_SHAPE
    assert L.layernorm_bwd_workspace_bytes(17, 16385, F32, ctypes.byref(out)) == E_SHAPE
    assert L.layernorm_bwd_workspace_bytes(17, 32769, F16, ctypes.byref(out)) == E_SHAPE
    assert L.layernorm_bwd_workspace_bytes(300, 32768, BF16, ctypes.byref(out)) == OK
    assert out.value == 2 * 256 * 32768 * 4  # wide rows: at most one partial row per CU
    assert L.layernorm_bwd_workspace_bytes(100, 20000, F16, ctypes.byref(out)) == OK and out.value == 2 * 100 * 20000 * 4
    assert L.layernorm_bwd_workspace_bytes(17, 8, 9, ctypes.byref(out)) == E_DTYPE
    assert L.layernorm_bwd_workspace_bytes(17, 8, F32, None) == E_NULL
    assert rn.layernorm_bwd_workspace_bytes(64, 128, 2) == 2 * 64 * 128 * 4


def bwd(L, x=X, w=W, dy=DY, mu=MU, r=R, dx=DX, dw=DW, db=DB, ws=WS, wsb=None, M=4, N=8, stride=None, dtype=F16):
    if wsb is None:
        wsb = 2 * M * N * 4
    return L.layernorm_bwd(x, w, dy, mu, r, dx, dw, db, ws, wsb, M, N, N if stride is None else stride, dtype, None)


def bwd_rows(L, x=X, w=W, dy=DY, mu=MU, r=R, dx=DX, ws=WS, wsb=None, M=4, N=8, stride=None, dtype=F16, rows=True):
    if wsb is None:
        wsb = 2 * M * N * 4
    out = ctypes.c_int64(-5)
    return L.layernorm_bwd_rows(x, w, dy, mu, r, dx, ws, wsb, M, N, N if stride is None else stride, dtype,
                                ctypes.byref(out) if rows else None, None)


@pytest.mark.parametrize("call", [bwd, bwd_rows])
def test_bwd_rejections(L, call):
    assert call(L, dtype=-1) == E_DTYPE
    assert call(L, N=0) == E_SHAPE
    assert call(L, N=32769) == E_SHAPE
    assert call(L, N=16385, dtype=F32) == E_SHAPE
    assert call(L, M=-2) == E_SHAPE
    assert call(L, stride=4) == E_STRIDE
    for kw in ("x", "w", "dy", "mu", "r", "dx", "ws"):
        assert call(L, **{kw: None}) == E_NULL, kw
    assert call(L, dy=DY + 1) == E_ALIGN
    assert call(L, mu=MU + 1) == E_ALIGN
    assert call(L, ws=WS + 2) == E_ALIGN
    assert call(L, wsb=2 * 4 * 8 * 4 - 1) == E_WS   # room for one table is not enough
    assert call(L, dx=X) == E_ALIAS
    assert call(L, dx=DY + 2) == E_ALIAS            # overlapping dy without being dy
    assert call(L, dx=MU) == E_ALIAS
    assert call(L, ws=DY + 8) == E_ALIAS
    assert call(L, ws=R) == E_ALIAS
    assert call(L, w=DX + 4) == E_ALIAS


def test_bwd_specific_rejections(L):
    assert bwd(L, dw=None) == E_NULL
    assert bwd(L, db=None) == E_NULL
    assert bwd(L, db=DB + 2) == E_ALIGN
    assert bwd(L, db=DW + 8) == E_ALIAS              # dw and db overlap
    assert bwd(L, dw=DX) == E_ALIAS
    assert bwd(L, db=WS + 16) == E_ALIAS
    assert bwd(L, dw=W) == E_ALIAS
    assert bwd_rows(L, rows=False) == E_NULL
    # dw and db are checked even when M == 0 (they are zeroed then)
    assert L.layernorm_bwd(None, None, None, None, None, None, None, None, None, 0, 0, 8, 8, F16, None) == E_NULL
    out = ctypes.c_int64(-5)
    assert L.layernorm_bwd_rows(None, None, None, None, None, None, None, 0, 0, 8, 8, F16, ctypes.byref(out),
                                None) == OK
    assert out.value == 0


def test_dwdb_reduce_rejections(L):
    assert L.layernorm_dwdb_reduce(WS, -1, 8, DW, DB, None) == E_SHAPE
    assert L.layernorm_dwdb_reduce(WS, 4, 0, DW, DB, None) == E_SHAPE
    assert L.layernorm_dwdb_reduce(WS, 4, 32769, DW, DB, None) == E_SHAPE
    assert L.layernorm_dwdb_reduce(WS, 1 << 15, 1 << 14, DW, DB, None) == E_SHAPE  # 2 * rows * N > 2^29
    # row counts whose 2 * rows * N wraps around int64 (to 0 for 1 << 61 rows x 4)
    assert L.layernorm_dwdb_reduce(WS, 1 << 61, 4, DW, DB, None) == E_SHAPE
    assert L.layernorm_dwdb_reduce(WS, 1 << 62, 4, DW, DB, None) == E_SHAPE
    assert L.layernorm_dwdb_reduce(WS, (1 << 63) - 1, 16384, DW, DB, None) == E_SHAPE
    assert L.layernorm_dwdb_reduce(WS, 4, 8, None, DB, None) == E_NULL
    assert L.layernorm_dwdb_reduce(WS, 4, 8, DW, None, None) == E_NULL
    assert L.layernorm_dwdb_reduce(None, 4, 8, DW, DB, None) == E_NULL
    assert L.layernorm_dwdb_reduce(WS + 1, 4, 8, DW, DB, None) == E_ALIGN
    assert L.layernorm_dwdb_reduce(WS, 4, 8, DW, DW + 16, None) == E_ALIAS
    assert L.layernorm_dwdb_reduce(WS, 4, 8, WS + 4 * 8 * 4 + 4, DB, None) == E_ALIAS  # inside the db table


def test_python_layernorm_refuses_cpu_tensors():
    import torch

    x = torch.zeros(4, 8, dtype=torch.float16)
    w = torch.ones(8, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU tensors only"):
        rn.layernorm_fwd(x, w, w, torch.empty_like(x), torch.empty(4), torch.empty(4))
    with pytest.raises(ValueError, match="GPU tensors only"):
        rn.layernorm(x.requires_grad_(), (8,), w, w)
    m = rn.LayerNorm(8)
    assert m.weight.detach().float().sum() == 8 and m.bias.detach().float().abs().sum() == 0
