"""Every row shape the launch planner can emit, run against the oracle.

``tests/native/bin/plan_check --widths`` (built with the library) lists, for
every distinct plan of the four row operations (element size, vector width,
waves per row, vectors per lane) over N <= 16384, the smallest and the
largest N that get it.  Each listed width runs here through the forward and
the backward of its norm on 33 rows (several row groups, a ragged last
workgroup) and is compared with the oracle under the usual per-dtype rule.
16-bit widths alternate between bf16 and fp16, and the RMSNorm cases
alternate Gemma's weight and the in-place backward, so that both of each
show up across the shapes.
"""
import os
import subprocess

import pytest

import workloads as wl
from tests.parity import Run, compare_with_oracle
from tests.parity_ln import LnRun, compare_ln_with_oracle

pytestmark = pytest.mark.gpu

PLAN_CHECK = os.path.join(os.path.dirname(__file__), "native", "bin", "plan_check")
M = 33


def _widths():
    if not os.path.exists(PLAN_CHECK):
        return []
    out = subprocess.run([PLAN_CHECK, "--widths"], capture_output=True, text=True, check=True).stdout
    cases = []
    for k, line in enumerate(out.split("\n")):
        if not line.strip():
            continue
        norm, es, n = line.split()
        dtype = "f32" if es == "4" else ("bf16" if k % 2 == 0 else "f16")
        cases.append((norm, dtype, int(n), k))
    return cases


CASES = _widths()


@pytest.mark.skipif(not CASES, reason="tests/native/bin/plan_check is not built")
@pytest.mark.parametrize("norm,dtype,N,k", CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}" for c in CASES])
def test_planner_shape(norm, dtype, N, k):
    print("case:", norm, dtype, M, N, flush=True)
    if norm == "rms":
        gemma, in_place = bool(k & 2), bool(k & 4)
        base = wl.C3 if gemma else wl.C2
        w = base.scaled(M=M, N=N, dtype=dtype, gemma=gemma, dx_in_place=in_place, seed=N * 7 + k)
        if dtype == "f32":
            w = w.scaled(dy=("normal", 0.0, 1.0))
        compare_with_oracle(Run(w))
    else:
        w = wl.Workload(f"ln_{dtype}_{M}x{N}", dtype, M, N, x=wl.LN1.x, gamma=wl.LN1.gamma, beta=wl.LN1.beta,
                        dy=wl.LN1.dy, eps=1e-5, seed=N * 11 + k)
        compare_ln_with_oracle(LnRun(w))
