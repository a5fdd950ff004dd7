"""The C ABI from plain C++ (no Python binding, no PyTorch): the program
tests/native/abi_example.cpp, built by ``row_normalization_amd.build``, runs
the worked examples printed on the Triton RMSNorm tutorial (kept with their
citations in tests/golden/worked_examples.json) through rmsnorm_fwd and
rmsnorm_bwd on the GPU; its printed outputs must round to the printed values.
dgamma, which the page does not print for these rows, is compared with the
fp64 oracle."""
import json
import os
import subprocess

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "native", "bin", "abi_example")
GOLDEN = os.path.join(ROOT, "tests", "golden", "worked_examples.json")


def _run(x, gamma, dy, eps, gemma=False):
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: build with `python -m row_normalization_amd.build`")
    args = [EXE, str(len(x)), repr(eps), "1" if gemma else "0", *map(repr, x), *map(repr, gamma), *map(repr, dy)]
    r = subprocess.run(args, capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    out = {}
    for line in r.stdout.splitlines():
        name, *vals = line.split()
        out[name] = vals
    assert out["rejected"][0] == "-1"  # RMSNORM_E_NULL for a null x
    return {k: np.array(v, dtype=np.float64) for k, v in out.items() if k != "rejected"}


def _printed(value, printed, decimals, what):
    err = np.max(np.abs(np.asarray(value) - np.asarray(printed)))
    assert err <= 0.5 * 10.0 ** -decimals + 1e-6, f"{what}: {value} vs printed {printed}"


def test_worked_examples_through_the_c_abi():
    g = json.load(open(GOLDEN))
    f = g["forward_two_values"]
    out = _run(f["x"], f["gamma"], [0.0, 0.0], f["eps"])
    _printed(out["y"], f["y"], f["decimals"], "y")
    _printed(out["r"], [f["r"]], f["decimals"], "r")
    f2 = g["forward_two_values_gamma"]
    out = _run(f2["x"], f2["gamma"], [0.0, 0.0], f2["eps"])
    _printed(out["y"], f2["y"], f2["decimals"], "y (gamma = [2, 0.5])")
    b = g["backward_two_values"]
    out = _run(b["x"], b["gamma"], b["dy"], b["eps"])
    _printed(out["dx"], b["dx"], b["decimals"], "dx")
    _, dg = oracle.backward(np.array([b["x"]]), np.array(b["gamma"]), np.array([b["dy"]]), b["eps"])
    assert np.max(np.abs(out["dgamma"] - dg) / (np.abs(dg) + 1e-30)) < 1e-5


def test_gemma_flag_through_the_c_abi():
    # gamma = [0, 0] under the Gemma weight 1 + gamma is the unit weight of the first example
    f = json.load(open(GOLDEN))["forward_two_values"]
    out = _run(f["x"], [0.0, 0.0], [1.0, 2.0], f["eps"], gemma=True)
    _printed(out["y"], f["y"], f["decimals"], "y (Gemma, gamma = 0)")
