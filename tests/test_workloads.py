"""Seeded synthetic inputs: determinism, shapes, special rows, byte model (CPU)."""
import numpy as np
import torch

import workloads as wl


def test_inputs_are_deterministic_and_quantised():
    w = wl.C2.scaled(M=64, N=256)
    a = wl.make_inputs(w)
    b = wl.make_inputs(w)
    for k in ("x", "gamma", "dy"):
        assert a[k].dtype == torch.bfloat16
        assert torch.equal(a[k].view(torch.int16), b[k].view(torch.int16))
    assert a["x"].shape == (64, 256) and a["gamma"].shape == (256,)


def test_distributions_roughly_as_stated():
    w = wl.C3.scaled(M=512, N=1024)
    t = wl.make_inputs(w)
    x, g, dy = (wl.to_f64(t[k]) for k in ("x", "gamma", "dy"))
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    assert abs(g.mean()) < 0.005 and abs(g.std() - 0.02) < 0.002
    assert abs(dy.std() - 1e-2) < 2e-4
    c1 = wl.make_inputs(wl.C1)
    g1 = wl.to_f64(c1["gamma"])
    assert c1["x"].dtype == torch.float32 and g1.min() >= 0.5 and g1.max() <= 1.5


def test_special_rows_of_c4():
    w = wl.C4
    assert (w.n_scaled, w.n_zero) == (328, 33)
    scaled, zero = wl.special_rows(w)
    assert len(set(scaled) | set(zero)) == 361
    small = w.scaled(M=2000, N=64)  # 20 scaled rows, 2 zero rows
    t = wl.make_inputs(small)
    x = wl.to_f64(t["x"])
    s, z = wl.special_rows(small)
    assert len(s) == 20 and len(z) == 2
    assert np.all(x[z] == 0)
    others = np.setdiff1d(np.arange(2000), np.concatenate([s, z]))
    assert np.sqrt(np.mean(x[s] ** 2)) > 50 * np.sqrt(np.mean(x[others] ** 2))


def test_algorithmic_bytes_table():
    # fwd = 2MNb + Nb + 4M; bwd = 3MNb + Nb + 4M + 4N
    assert wl.algorithmic_bytes(16384, 8192, 2) == {
        "fwd": 536_952_832, "bwd_rows": 805_388_288, "bwd": 805_421_056, "fwd_bwd": 1_342_373_888}
    assert wl.algorithmic_bytes(64, 128, 4)["fwd_bwd"] == 165_888
    assert wl.algorithmic_bytes(32768, 5120, 2)["fwd_bwd"] == 1_678_024_704
