"""The parity bounds are frozen: every value the GPU parity tests apply is
pinned here.  A change to one of them has to change this file too, in a
commit that names the passage (or the reading of it, and the fp32 emulation
on the CPU) that justifies it."""
from tests.parity import TOL
from tests.parity_ln import TOL_LN


def test_rmsnorm_bounds_frozen():
    assert TOL == {
        "f32_y": 1e-5, "f32_dx": 1e-5, "f32_dgamma": 1e-4, "16bit_dgamma": 1e-3,
        "bf16_atol": 2e-2, "bf16_rtol": 1.6e-2, "f16_atol": 3e-3, "f16_rtol": 3e-3,
        "16bit_normwise": 4e-3, "dx_invariant": 1e-3, "rstd_rel": 2e-6,
        "f32_direct_units": 2.0**-22, "16bit_direct_units": 2.0**-20, "rms_dx_direct_multiple": 4.0,
        "plain_floor": 0.1,
    }


def test_layernorm_bounds_frozen():
    assert TOL_LN == {"mean_rel": 2e-6, "rstd_rel": 4e-6, "row_sums": 1e-3, "dw_center_factor": 4.0}
