"""Helpers of the LayerNorm GPU parity tests: run the HIP path through the C
ABI on seeded inputs and compare it with the fp64 LayerNorm oracle.

Tolerances (per element unless stated; the forms are those of
``tests/parity.py``):

* y, dx: ``check_close`` of ``tests/parity.py`` for the I/O dtype (fp32:
  1e-5 relative against |o| + rms(o); bf16: 2e-2 + 1.6e-2 |o|; fp16:
  3e-3 + 3e-3 |o|; 16-bit outputs also within 4e-3 norm-wise).  dx is a
  difference of g * rstd and (x_hat c1 + c2) * rstd, so its fp32 allowance
  scales with the oracle's direct term |w dy rstd|, as for RMSNorm, plus the
  centering term: fp32 x - mean is off by about one ulp of max|x| of the
  row, which reaches x_hat scaled by rstd and dx through c1 and x_hat c1,
  so the allowance adds max|x| rstd^2 (|c1| + |x_hat| mean|g|); y = x_hat w + b
  gets the matching fp32 allowance max|x| rstd |w|, and dw (a column sum of
  dy x_hat) 4 sqrt(sum over rows of (dy max|x| rstd)^2), the rows' centering
  errors being independent.  It matters
  only for rows whose spread is close to sqrt(eps) next to their values (a
  two-column row of -2.0045 and -2.0117: var 1.3e-5, dx off by 8.5e-5
  relative, and an fp32 evaluation in the kernel's order on the CPU gives
  the GPU's value); for rows of unit spread it is below 1e-6 of |dx|.
* dw, db (fp32 accumulators): 1e-4 (fp32 I/O) or 1e-3 (16-bit I/O) relative
  against |o| + rms(o).
* mean: |g - o| <= 2e-6 (|o| + sqrt(var)), i.e. fp32 rounding of a sum of N
  terms relative to the row's spread; rstd: relative error <= 4e-6 (the
  variance is a second fp32 sum, over the squared differences).
* For 16-bit dx, the shift invariance of LayerNorm gives a row invariant:
  every row of dx sums to zero; the median over rows of
  |sum_j dx_ij| / (||dx_i|| sqrt(N)) must stay <= 1e-3 (a kernel that drops
  the c2 term fails it by orders of magnitude).
* The LayerNorm chapter's own test rule (torch.testing.assert_close with
  atol = 1e-2, rtol = 0 for y, dx, dw and db in fp16) is checked as well on
  its unit-test shape.
"""
from __future__ import annotations

import numpy as np
import torch

import row_normalization_amd as rn
import workloads as wl
from oracle import layernorm_oracle as lo
from tests.parity import check_close, padded

# The LayerNorm-specific bounds (y, dx, dw, db otherwise take check_close's
# per-dtype rules), each with its source; frozen like those of
# tests/parity.py (tests/test_tolerances.py pins them).
TOL_LN = {
    # mean: fp32 rounding of a sum of N values, relative to |mean| + the
    # row's spread (sqrt(var + eps)); sums of 16384 unit-spread values in fp32
    # on the CPU stay below 3e-7
    "mean_rel": 2e-6,
    # rstd: a second fp32 sum, over the squared differences from the fp32
    # mean, then rsqrt within one ulp
    "rstd_rel": 4e-6,
    # 16-bit dx rows sum to zero (LayerNorm's shift invariance): median over
    # rows of |sum_j dx_ij| / (||dx_i|| sqrt(N)); a dropped c2 term fails it
    # by orders of magnitude
    "row_sums": 1e-3,
    # dw's centering allowance: the rows' fp32 centering errors (one ulp of
    # max|x| of the row, times rstd) reach dw through dy; independent between
    # rows, so they add as a root sum of squares, allowed four fp32 ulps of it
    # (2^-20 with check_close's 2^-22 units).  Near-constant rows x = 5 +
    # 1e-3 z (|mean| / sigma = 5000) need it: at N = 2 dw was off by 1.5e-4
    # relative on the GPU, and an fp32 evaluation in the kernel's order on the
    # CPU gave the same value
    "dw_center_factor": 4.0,
}


def check_mean_rstd(name: str, mean_g, rstd_g, mean_o, rstd_o) -> None:
    sd = 1.0 / rstd_o  # sqrt(var + eps) >= sqrt(var)
    err_m = np.abs(mean_g - mean_o) / (np.abs(mean_o) + sd)
    assert err_m.max() <= TOL_LN["mean_rel"], f"{name}: mean err {err_m.max():.3g} at row {int(np.argmax(err_m))}"
    rel = np.abs(rstd_g - rstd_o) / rstd_o
    assert rel.max() <= TOL_LN["rstd_rel"], f"{name}: rstd rel err {rel.max():.3g} at row {int(np.argmax(rel))}"


def check_row_sums_vanish(name: str, dx: np.ndarray) -> float:
    nd = np.linalg.norm(dx, axis=1)
    ok = nd > 0
    if not ok.any() or dx.shape[1] < 64:
        return 0.0
    res = np.abs(dx.sum(axis=1))[ok] / (nd[ok] * np.sqrt(dx.shape[1]))
    med = float(np.median(res))
    assert med <= TOL_LN["row_sums"], f"{name}: row sums of dx: median residual {med:.3g} > {TOL_LN['row_sums']}"
    return med


class LnRun:
    """Outputs of one LayerNorm fwd + bwd pass of the HIP path."""

    def __init__(self, w: wl.Workload, inputs=None, row_stride: int | None = None, offset: int = 0,
                 split_bwd: bool = True, in_place: bool = False):
        self.w = w
        self.inputs = inputs if inputs is not None else wl.make_inputs(w)
        stride = w.N if row_stride is None else row_stride
        x = padded(self.inputs["x"], stride, float("nan"), offset)
        dy = padded(self.inputs["dy"], stride, float("nan"), offset)
        weight = self.inputs["gamma"].to("cuda")
        bias = self.inputs["beta"].to("cuda")
        y = padded(torch.zeros_like(self.inputs["x"]), stride, -7.0, offset)
        mean = torch.full((w.M,), float("nan"), dtype=torch.float32, device="cuda")
        rstd = torch.full((w.M,), float("nan"), dtype=torch.float32, device="cuda")
        dx = dy if in_place else padded(torch.zeros_like(self.inputs["x"]), stride, -7.0, offset)
        dw = torch.full((w.N,), float("nan"), dtype=torch.float32, device="cuda")
        db = torch.full((w.N,), float("nan"), dtype=torch.float32, device="cuda")
        ws_bytes = rn.layernorm_bwd_workspace_bytes(w.M, w.N, w.torch_dtype)
        ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device="cuda")

        rn.layernorm_fwd(x, weight, bias, y, mean, rstd, eps=w.eps)
        if split_bwd:
            self.partial_rows = rn.layernorm_bwd_rows(x, weight, dy, mean, rstd, dx, ws)
            rn.layernorm_dwdb_reduce(ws, self.partial_rows, w.N, dw, db)
        else:
            rn.layernorm_bwd(x, weight, dy, mean, rstd, dx, dw, db, ws)
        torch.cuda.synchronize()
        self.y, self.mean, self.rstd, self.dx, self.dw, self.db = y, mean, rstd, dx, dw, db
        self.x_gpu, self.ws = x, ws

    def host(self):
        return tuple(wl.to_f64(t) for t in (self.y, self.mean, self.rstd, self.dx, self.dw, self.db))


def compare_ln_with_oracle(run: LnRun, rows: np.ndarray | None = None) -> dict:
    """Every output of ``run`` against the oracle (y, mean, rstd, dx on ``rows``
    or all rows; dw and db need every row, so they are compared in full)."""
    w = run.w
    x = wl.to_f64(run.inputs["x"])
    wt = wl.to_f64(run.inputs["gamma"])
    b = wl.to_f64(run.inputs["beta"])
    dy = wl.to_f64(run.inputs["dy"])
    y_g, m_g, r_g, dx_g, dw_g, db_g = run.host()
    diag = {}
    if w.M:
        sel = np.arange(w.M) if rows is None else rows
        y_o, m_o, r_o = lo.forward(x[sel], wt, b, w.eps)
        dx_o, _, _ = lo.backward(x[sel], wt, dy[sel], w.eps)
        # fp32 centering: x - mean off by about one ulp of max|x|, scaled by rstd and w
        y_center = (np.max(np.abs(x[sel]), axis=1) * r_o)[:, None] * np.abs(wt)[None, :] if w.dtype == "f32" else None
        diag["y"] = check_close(f"{w.name} y", y_g[sel], y_o, w.dtype, "y", direct=y_center)
        check_mean_rstd(w.name, m_g[sel], r_g[sel], m_o, r_o)
        g_o = wt[None, :] * dy[sel]
        direct = np.abs(g_o * r_o[:, None])
        if w.dtype == "f32":
            xh = (x[sel] - m_o[:, None]) * r_o[:, None]
            c1 = np.mean(g_o * xh, axis=1)
            center = (np.max(np.abs(x[sel]), axis=1) * r_o ** 2)[:, None] * (
                np.abs(c1)[:, None] + np.abs(xh) * np.mean(np.abs(g_o), axis=1)[:, None])
            direct = direct + center
        diag["dx"] = check_close(f"{w.name} dx", dx_g[sel], dx_o, w.dtype, "dx", direct=direct)
        if w.dtype != "f32":
            diag["dx_row_sums"] = check_row_sums_vanish(f"{w.name} dx", dx_g[sel])
    _, dw_o, db_o = lo.backward(x, wt, dy, w.eps) if w.M else (None, np.zeros(w.N), np.zeros(w.N))
    dw_center = None
    if w.dtype == "f32" and w.M:
        # each row's fp32 centering error, carried by dy * x_hat into the column
        # sums; independent between rows, so combined as a root sum of squares
        _, _, r_all = lo.forward(x, wt, b, w.eps)
        dw_center = TOL_LN["dw_center_factor"] * np.sqrt(
            np.sum((dy * (np.max(np.abs(x), axis=1) * r_all)[:, None]) ** 2, axis=0))
    diag["dw"] = check_close(f"{w.name} dw", dw_g, dw_o, w.dtype, "dgamma", direct=dw_center)
    diag["db"] = check_close(f"{w.name} db", db_g, db_o, w.dtype, "dgamma")
    return diag
