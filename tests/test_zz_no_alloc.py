"""The allocation-free backward, rmsnorm_bwd_noalloc, through the C ABI.

Its dx and dgamma must equal rmsnorm_bwd's bit for bit: the same kernels
run with the same launch plan and summation order, only the partial rows
live in the library's static scratch instead of a caller's workspace.  Two
calls in a row, the second on a smaller problem, so that the scratch still
holds more partial rows from the first call than the second one writes (the
column sum must read only its own); then M = 0, which must give dgamma = 0.
"""
import pytest
import torch

import row_normalization_amd as rn
import workloads as wl

pytestmark = pytest.mark.gpu

CODES = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}


def _inputs(w):
    t = wl.make_inputs(w)
    x, g, dy = (t[k].cuda() for k in ("x", "gamma", "dy"))
    M, N = x.shape
    L = rn.lib()
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream().cuda_stream
    assert L.rmsnorm_fwd(x.data_ptr(), g.data_ptr(), y.data_ptr(), rstd.data_ptr(), M, N, N, w.eps, CODES[x.dtype],
                         int(w.gemma), stream) == 0
    return x, g, dy, rstd


def _both(w):
    """(dx, dgamma) from rmsnorm_bwd with a workspace and from rmsnorm_bwd_noalloc."""
    x, g, dy, rstd = _inputs(w)
    M, N = x.shape
    L = rn.lib()
    stream = torch.cuda.current_stream().cuda_stream
    code, flags = CODES[x.dtype], int(w.gemma)
    out = []
    for noalloc in (False, True):
        dy_k = dy.clone()
        dx = dy_k if w.dx_in_place else torch.empty_like(dy)
        dg = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            st = L.rmsnorm_bwd_noalloc(x.data_ptr(), g.data_ptr(), dy_k.data_ptr(), rstd.data_ptr(), dx.data_ptr(),
                                       dg.data_ptr(), M, N, N, code, flags, stream)
        else:
            nbytes = rn.rmsnorm_bwd_workspace_bytes(M, N, x.dtype)
            ws = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device="cuda")
            st = L.rmsnorm_bwd(x.data_ptr(), g.data_ptr(), dy_k.data_ptr(), rstd.data_ptr(), dx.data_ptr(),
                               dg.data_ptr(), ws.data_ptr(), nbytes, M, N, N, code, flags, stream)
        assert st == 0, rn.rmsnorm_status_string(st)
        torch.cuda.synchronize()
        out.append((dx, dg))
    return out


def test_noalloc_matches_workspace_entry_point_twice():
    torch.cuda.set_device(0)
    # first call: the headline layout (bf16, Gemma weight, dx over dy), 512
    # partial rows of 8192 columns (16 MiB of the scratch)
    big = wl.C3.scaled(M=3000)
    # second call: smaller, fp32, dx in its own buffer, fewer partial rows
    # and columns than the first call left in the scratch
    small = wl.C1.scaled(M=300)
    for w in (big, small):
        (dx_ref, dg_ref), (dx, dg) = _both(w)
        assert torch.isfinite(dg_ref).all()
        assert torch.equal(dx, dx_ref), w.name
        assert torch.equal(dg, dg_ref), w.name


def test_noalloc_zero_rows_zeroes_dgamma():
    torch.cuda.set_device(0)
    L = rn.lib()
    dg = torch.full((257,), float("nan"), dtype=torch.float32, device="cuda")
    st = L.rmsnorm_bwd_noalloc(None, None, None, None, None, dg.data_ptr(), 0, 257, 257, 1, 0,
                               torch.cuda.current_stream().cuda_stream)
    assert st == 0, rn.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(dg, torch.zeros_like(dg))
