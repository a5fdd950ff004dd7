"""GPU parity at the limits of the launch plans and of the ABI.

* More row groups than the forward's grid holds (2^20 workgroups): the forward
  then takes several steps per workgroup; checked in full against the oracle,
  for RMSNorm and LayerNorm.
* The largest row count the ABI accepts (M = 2^29, one column, bf16): every
  row is computed; y, r and dx are compared on a seeded sample of rows plus
  the first and last, and the weight gradient — a sum over all 2^29 rows — in
  full, with the oracle's own definition evaluated chunk by chunk (the same
  arithmetic, only split so the fp64 temporaries stay small).
"""
import numpy as np
import pytest
import torch

import oracle
import row_normalization_amd as rn
import workloads as wl
from oracle import layernorm_oracle as lo
from tests.parity import Run, check_close, check_rstd, compare_with_oracle
from tests.parity_ln import LnRun, check_mean_rstd, compare_ln_with_oracle

pytestmark = pytest.mark.gpu

GRID_MAX_FWD = 1 << 20


def _case(*what):
    print("case:", *what, flush=True)


def test_rmsnorm_forward_takes_several_steps():
    # N = 8 bf16: one 16-byte vector per row, 8 rows per workgroup, so
    # 2^23 + 37 rows make 2^20 + 5 row groups: two forward steps.
    w = wl.C2.scaled(M=8 * GRID_MAX_FWD + 37, N=8)
    _case(w.name, w.M, w.N)
    compare_with_oracle(Run(w))


def test_layernorm_forward_takes_several_steps():
    w = wl.LN1.scaled(M=8 * GRID_MAX_FWD + 37, N=8)
    _case(w.name, w.M, w.N)
    compare_ln_with_oracle(LnRun(w))


def _sample_rows(M, k, seed):
    rows = np.random.Generator(np.random.PCG64(seed)).choice(M, k, replace=False)
    return np.unique(np.concatenate([rows, [0, 1, M - 2, M - 1]]))


def test_rmsnorm_max_rows():
    M = 1 << 29
    w = wl.C2.scaled(M=M, N=1)
    _case(w.name, "M = 2^29")
    t = wl.make_inputs(w)
    x, g, dy = t["x"].cuda(), t["gamma"].cuda(), t["dy"].cuda()
    y = torch.empty_like(x)
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    dx = torch.empty_like(x)
    dgamma = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(rn.rmsnorm_bwd_workspace_bytes(M, 1, torch.bfloat16) // 4, dtype=torch.float32, device="cuda")
    rn.rmsnorm_fwd(x, g, y, rstd, eps=w.eps)
    rn.rmsnorm_bwd(x, g, dy, rstd, dx, dgamma, ws)
    torch.cuda.synchronize()
    del ws
    rows = _sample_rows(M, 100_000, 1)
    xs, dys = wl.to_f64(t["x"][rows]), wl.to_f64(t["dy"][rows])
    gam = wl.to_f64(t["gamma"])
    y_o, r_o = oracle.forward(xs, gam, w.eps)
    dx_o, _ = oracle.backward(xs, gam, dys, w.eps)
    idx = torch.from_numpy(rows).cuda()
    check_close("max rows y", wl.to_f64(y[idx]), y_o, "bf16", "y")
    check_rstd("max rows rstd", wl.to_f64(rstd[idx]), r_o)
    check_close("max rows dx", wl.to_f64(dx[idx]), dx_o, "bf16", "dx", direct=r_o[:, None] * dys * gam)
    # the weight gradient over all rows: the oracle's row contributions, summed chunk by chunk
    total = 0.0
    chunk = 1 << 25
    for s in range(0, M, chunk):
        xc, dyc = wl.to_f64(t["x"][s:s + chunk]), wl.to_f64(t["dy"][s:s + chunk])
        r = oracle.inverse_rms(xc, w.eps)
        total += float(oracle.dgamma_from_rows(dyc * xc * r[:, None])[0])
    check_close("max rows dgamma", wl.to_f64(dgamma), np.array([total]), "bf16", "dgamma")


def test_layernorm_max_rows():
    M = 1 << 29
    w = wl.LN1.scaled(M=M, N=2, dtype="bf16")
    _case(w.name, "M = 2^29")
    t = wl.make_inputs(w)
    x, wt, b, dy = (t[k].cuda() for k in ("x", "gamma", "beta", "dy"))
    y = torch.empty_like(x)
    mean = torch.empty(M, dtype=torch.float32, device="cuda")
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    dx = torch.empty_like(x)
    dw = torch.empty(2, dtype=torch.float32, device="cuda")
    db = torch.empty(2, dtype=torch.float32, device="cuda")
    ws = torch.empty(rn.layernorm_bwd_workspace_bytes(M, 2, torch.bfloat16) // 4, dtype=torch.float32, device="cuda")
    rn.layernorm_fwd(x, wt, b, y, mean, rstd, eps=w.eps)
    rn.layernorm_bwd(x, wt, dy, mean, rstd, dx, dw, db, ws)
    torch.cuda.synchronize()
    del ws
    rows = _sample_rows(M, 100_000, 2)
    idx = torch.from_numpy(rows).cuda()
    xs, dys = wl.to_f64(t["x"][rows]), wl.to_f64(t["dy"][rows])
    ww, bb = wl.to_f64(t["gamma"]), wl.to_f64(t["beta"])
    y_o, m_o, r_o = lo.forward(xs, ww, bb, w.eps)
    dx_o, _, _ = lo.backward(xs, ww, dys, w.eps)
    check_close("max rows y", wl.to_f64(y[idx]), y_o, "bf16", "y")
    check_mean_rstd("max rows", wl.to_f64(mean[idx]), wl.to_f64(rstd[idx]), m_o, r_o)
    check_close("max rows dx", wl.to_f64(dx[idx]), dx_o, "bf16", "dx", direct=ww * dys * r_o[:, None])
    # dw and db over all rows, chunk by chunk with the oracle's own backward
    dw_o = np.zeros(2)
    db_o = np.zeros(2)
    chunk = 1 << 24
    for s in range(0, M, chunk):
        _, dwc, dbc = lo.backward(wl.to_f64(t["x"][s:s + chunk]), ww, wl.to_f64(t["dy"][s:s + chunk]), w.eps)
        dw_o += dwc
        db_o += dbc
    check_close("max rows dw", wl.to_f64(dw), dw_o, "bf16", "dgamma")
    check_close("max rows db", wl.to_f64(db), db_o, "bf16", "dgamma")
