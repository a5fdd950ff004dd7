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


def test_layernorm_inputs():
    w = wl.LN1.scaled(M=256, N=1024)
    t = wl.make_inputs(w)
    assert sorted(t) == ["beta", "dy", "gamma", "x"]
    assert all(v.dtype == torch.float16 for v in t.values())
    x, g, b, dy = (wl.to_f64(t[k]) for k in ("x", "gamma", "beta", "dy"))
    assert abs(x.mean() + 2.3) < 0.01 and abs(x.std() - 0.5) < 0.01
    assert g.min() >= 0 and g.max() <= 1 and b.min() >= 0 and b.max() <= 1
    assert not np.array_equal(g, b)  # weight and bias come from different streams
    assert abs(dy.std() - 0.1) < 0.002
    # the bias stream leaves the other inputs as an RMSNorm workload draws them
    r = wl.make_inputs(wl.Workload("same", "f16", 256, 1024, x=w.x, gamma=w.gamma, dy=w.dy))
    for k in ("x", "gamma", "dy"):
        assert torch.equal(r[k].view(torch.int16), t[k].view(torch.int16))
    assert wl.LN_SWEEP_NS[0] == 1024 and wl.LN_SWEEP_NS[-1] == 15872 and len(wl.LN_SWEEP_NS) == 30
    assert wl.ln_sweep(2048).M == 4096 and wl.ln_sweep(2048).eps == 1e-5


def test_layernorm_algorithmic_bytes():
    # fwd = 2MNb + 2Nb + 8M; bwd = 3MNb + Nb + 8M + 8N
    assert wl.ln_algorithmic_bytes(4096, 8192, 2) == {
        "fwd": 134_283_264, "bwd_rows": 201_375_744, "bwd": 201_441_280, "fwd_bwd": 335_724_544}


def test_rope_inputs():
    w = wl.ROPE1.scaled(tokens=300)
    t = wl.make_rope_inputs(w)
    assert t["q"].shape == (300, 32, 128) and t["q"].dtype == torch.bfloat16
    assert t["cos"].shape == (2048, 64) and t["cos"].dtype == torch.float32
    assert t["positions"].dtype == torch.int32 and t["positions"][257].item() == 257
    c, s = t["cos"].double(), t["sin"].double()
    assert torch.allclose(c * c + s * s, torch.ones_like(c), atol=1e-6)  # unit phasors up to fp32 rounding
    assert torch.all(c[0] == 1) and torch.all(s[0] == 0)
    r = wl.make_rope_inputs(w.scaled(positions="random", tokens=4096))["positions"]
    assert r.min() >= 0 and r.max() < 2048 and len(set(r.tolist())) > 1000
    assert torch.equal(wl.make_rope_inputs(w)["q"].view(torch.int16), t["q"].view(torch.int16))


def test_swiglu_inputs():
    w = wl.SWIGLU1.scaled(M=256, N=1024)
    t = wl.make_swiglu_inputs(w)
    assert all(v.shape == (256, 1024) and v.dtype == torch.bfloat16 for v in t.values())
    e, dh = wl.to_f64(t["e"]), wl.to_f64(t["dh"])
    assert abs(e.std() - 1) < 0.01 and abs(dh.std() - 0.01) < 2e-4
    assert wl.swiglu_algorithmic_bytes(11136, 14336, 2) == {"fwd": 957_874_176, "bwd": 1_915_748_352}
    assert wl.rope_algorithmic_bytes(8192, 32, 128, 2, 2048) == 2 * 8192 * 32 * 128 * 2 + 2 * 2048 * 64 * 4 + 4 * 8192
