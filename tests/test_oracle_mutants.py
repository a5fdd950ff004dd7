"""Plant plausible mistakes in a copy of the oracle and check the pins catch each.

Each mutant is the oracle's source with one textual change (a dropped term, a
wrong sign, denominator, index or reduction), loaded as a separate module on
the CPU.  The pins in ``oracle_pins`` must reject every one of them; a mutant
no pin rejects would mean a part of the oracle is not really pinned.
"""
import importlib.util
import os
import types

import pytest

from tests import oracle_pins, oracle_pins_ln, oracle_pins_rope, oracle_pins_swiglu

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
SRC = os.path.join(ORACLE_DIR, "rmsnorm_oracle.py")
LN_SRC = os.path.join(ORACLE_DIR, "layernorm_oracle.py")
ROPE_SRC = os.path.join(ORACLE_DIR, "rope_oracle.py")
SWIGLU_SRC = os.path.join(ORACLE_DIR, "swiglu_oracle.py")

MUTANTS = {
    "denominator_n_plus_1": ("mean_sq = np.sum(x * x, axis=1) / n", "mean_sq = np.sum(x * x, axis=1) / (n + 1)"),
    "denominator_padded_pow2": ("mean_sq = np.sum(x * x, axis=1) / n",
                                "mean_sq = np.sum(x * x, axis=1) / (1 << (n - 1).bit_length())"),
    "rows_for_columns": ("    n = x.shape[1]\n    mean_sq", "    n = x.shape[0]\n    mean_sq"),
    "eps_outside_root": ("return 1.0 / np.sqrt(mean_sq + eps)", "return 1.0 / np.sqrt(mean_sq) + eps"),
    "eps_dropped": ("return 1.0 / np.sqrt(mean_sq + eps)", "return 1.0 / np.sqrt(mean_sq)"),
    "sqrt_not_inverse": ("return 1.0 / np.sqrt(mean_sq + eps)", "return np.sqrt(mean_sq + eps)"),
    "gemma_ignored": ("return 1.0 + g", "return g"),
    "gemma_sign": ("return 1.0 + g", "return 1.0 - g"),
    "forward_drops_weight": ("y = x * r[:, None] * w[None, :]", "y = x * r[:, None]"),
    "u_drops_weight": ("u = dy * w[None, :]", "u = dy"),
    "m_wrong_operand": ("m = np.sum(u * x, axis=1) / n", "m = np.sum(u * dy, axis=1) / n"),
    "m_sum_not_mean": ("m = np.sum(u * x, axis=1) / n", "m = np.sum(u * x, axis=1)"),
    "m_padded_denominator": ("m = np.sum(u * x, axis=1) / n", "m = np.sum(u * x, axis=1) / (1 << (n - 1).bit_length())"),
    "bwd_rows_for_columns": ("    n = x.shape[1]\n    r = inverse_rms", "    n = x.shape[0]\n    r = inverse_rms"),
    "dx_projection_dropped": ("dx = r[:, None] * u - x * (r**3 * m)[:, None]", "dx = r[:, None] * u"),
    "dx_projection_sign": ("dx = r[:, None] * u - x * (r**3 * m)[:, None]", "dx = r[:, None] * u + x * (r**3 * m)[:, None]"),
    "dx_r_squared": ("dx = r[:, None] * u - x * (r**3 * m)[:, None]", "dx = r[:, None] * u - x * (r**2 * m)[:, None]"),
    "dx_direct_term_no_r": ("dx = r[:, None] * u - x * (r**3 * m)[:, None]", "dx = u - x * (r**3 * m)[:, None]"),
    "dgamma_drops_r": ("dgamma = dgamma_from_rows(dy * x * r[:, None])", "dgamma = dgamma_from_rows(dy * x)"),
    "dgamma_includes_weight": ("dgamma = dgamma_from_rows(dy * x * r[:, None])",
                               "dgamma = dgamma_from_rows(dy * x * r[:, None] * w[None, :])"),
    "dgamma_uses_u": ("dgamma = dgamma_from_rows(dy * x * r[:, None])", "dgamma = dgamma_from_rows(u * x * r[:, None])"),
    "dgamma_mean_not_sum": ("return np.sum(_f64(contributions), axis=0)", "return np.mean(_f64(contributions), axis=0)"),
    "dgamma_sums_columns": ("return np.sum(_f64(contributions), axis=0)", "return np.sum(_f64(contributions), axis=1)"),
    "quantize_truncates": ("return np.ldexp(np.round(m * 2.0**p), e - p)", "return np.ldexp(np.floor(m * 2.0**p), e - p)"),
    "quantize_bf16_bits": ('_SIGNIFICAND_BITS = {"bf16": 8,', '_SIGNIFICAND_BITS = {"bf16": 7,'),
    "quantize_f16_as_f32": ("return v.astype(np.float16).astype(np.float64)", "return v.astype(np.float32).astype(np.float64)"),
    "normed_not_rounded": ("normed = quantize(x * r[:, None], dtype)", "normed = x * r[:, None]"),
    "product_not_rounded": ("return quantize(normed * w[None, :], dtype), r", "return normed * w[None, :], r"),
    "normed_weight_dropped": ("return quantize(normed * w[None, :], dtype), r", "return quantize(normed, dtype), r"),
}


LN_MUTANTS = {
    "ln_mean_denominator": ("mean = np.sum(x, axis=1) / n", "mean = np.sum(x, axis=1) / (n + 1)"),
    "ln_mean_rows_for_columns": ("    n = x.shape[1]\n    mean = np.sum", "    n = x.shape[0]\n    mean = np.sum"),
    "ln_var_unbiased": ("var = np.sum(diff * diff, axis=1) / n", "var = np.sum(diff * diff, axis=1) / (n - 1)"),
    "ln_var_one_pass": ("var = np.sum(diff * diff, axis=1) / n",
                        "var = np.sum(x * x, axis=1) / n - mean * mean"),
    "ln_var_not_centred": ("diff = x - mean[:, None]", "diff = x"),
    "ln_eps_outside_root": ("rstd = 1.0 / np.sqrt(var + eps)\n    x_hat = (x - mean[:, None]) * rstd[:, None]\n    y",
                            "rstd = 1.0 / np.sqrt(var) + eps\n    x_hat = (x - mean[:, None]) * rstd[:, None]\n    y"),
    "ln_std_not_inverse": ("rstd = 1.0 / np.sqrt(var + eps)\n    x_hat = (x - mean[:, None]) * rstd[:, None]\n    y",
                           "rstd = np.sqrt(var + eps)\n    x_hat = (x - mean[:, None]) * rstd[:, None]\n    y"),
    "ln_fwd_mean_not_subtracted": ("x_hat = (x - mean[:, None]) * rstd[:, None]\n    y",
                                   "x_hat = x * rstd[:, None]\n    y"),
    "ln_fwd_drops_bias": ("y = x_hat * _f64(w)[None, :] + _f64(b)[None, :]", "y = x_hat * _f64(w)[None, :]"),
    "ln_fwd_bias_times_weight": ("y = x_hat * _f64(w)[None, :] + _f64(b)[None, :]",
                                 "y = (x_hat + _f64(b)[None, :]) * _f64(w)[None, :]"),
    "ln_bwd_eps_dropped": ("rstd = 1.0 / np.sqrt(var + eps)\n    x_hat = (x - mean[:, None]) * rstd[:, None]\n    g",
                           "rstd = 1.0 / np.sqrt(var)\n    x_hat = (x - mean[:, None]) * rstd[:, None]\n    g"),
    "ln_bwd_mean_not_subtracted": ("x_hat = (x - mean[:, None]) * rstd[:, None]\n    g",
                                   "x_hat = x * rstd[:, None]\n    g"),
    "ln_g_drops_weight": ("g = _f64(w)[None, :] * dy", "g = dy"),
    "ln_c1_sum_not_mean": ("c1 = np.sum(x_hat * g, axis=1) / n", "c1 = np.sum(x_hat * g, axis=1)"),
    "ln_c1_wrong_operand": ("c1 = np.sum(x_hat * g, axis=1) / n", "c1 = np.sum(x_hat * dy, axis=1) / n"),
    "ln_c2_sum_not_mean": ("c2 = np.sum(g, axis=1) / n", "c2 = np.sum(g, axis=1)"),
    "ln_c2_dropped": ("(x_hat * c1[:, None] + c2[:, None])", "(x_hat * c1[:, None])"),
    "ln_c1_dropped": ("(x_hat * c1[:, None] + c2[:, None])", "(c2[:, None])"),
    "ln_c2_sign": ("(x_hat * c1[:, None] + c2[:, None])", "(x_hat * c1[:, None] - c2[:, None])"),
    "ln_dx_no_rstd": ("dx = (g - (x_hat * c1[:, None] + c2[:, None])) * rstd[:, None]",
                      "dx = (g - (x_hat * c1[:, None] + c2[:, None]))"),
    "ln_dw_not_normalised": ("dw = column_sums(dy * x_hat)", "dw = column_sums(dy * x)"),
    "ln_dw_includes_weight": ("dw = column_sums(dy * x_hat)", "dw = column_sums(g * x_hat)"),
    "ln_db_includes_weight": ("db = column_sums(dy)", "db = column_sums(g)"),
    "ln_sums_are_means": ("return np.sum(_f64(contributions), axis=0)", "return np.mean(_f64(contributions), axis=0)"),
    "ln_sums_over_columns": ("return np.sum(_f64(contributions), axis=0)", "return np.sum(_f64(contributions), axis=1)"),
}


def _load_mutant(name, old, new, src_path=SRC):
    with open(src_path) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation {name!r} does not match the oracle source exactly once"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _load_mutant(name, *MUTANTS[name])
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # an assertion or a shape error both reject the mutant
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin rejects the mutant {name!r}"


@pytest.mark.parametrize("name", sorted(LN_MUTANTS))
def test_layernorm_mutant_is_caught(name):
    mod = _load_mutant(name, *LN_MUTANTS[name], src_path=LN_SRC)
    caught = []
    for pin in oracle_pins_ln.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin rejects the LayerNorm mutant {name!r}"


ROPE_MUTANTS = {
    "rope_first_sign": ("q1 * c - q2 * s", "q1 * c + q2 * s"),
    "rope_second_sign": ("q2 * c + q1 * s", "q2 * c - q1 * s"),
    "rope_interleaved_pairs": ("    q1 = q[..., :half]\n    q2 = q[..., half:]", "    q1 = q[..., ::2]\n    q2 = q[..., 1::2]"),
    "rope_halves_swapped": ("    q1 = q[..., :half]\n    q2 = q[..., half:]", "    q1 = q[..., half:]\n    q2 = q[..., :half]"),
    "rope_cos_sin_swapped": ("c = np.asarray(cos, dtype=np.float64)[pos]", "c = np.asarray(sin, dtype=np.float64)[pos]"),
    "rope_backward_same_sin": ("return rotate(dq, cos, -np.asarray(sin, dtype=np.float64), pos)",
                               "return rotate(dq, cos, np.asarray(sin, dtype=np.float64), pos)"),
    "rope_backward_negates_cos": ("return rotate(dq, cos, -np.asarray(sin, dtype=np.float64), pos)",
                                  "return rotate(dq, -np.asarray(cos, dtype=np.float64), sin, pos)"),
    "rope_positions_offset": ("% seq_len", "% seq_len + 1"),
    "rope_positions_ignored": ("return np.asarray(positions, dtype=np.int64)", "return np.arange(n_tokens) % seq_len"),
    "rope_output_halves_swapped": ("np.concatenate([q1 * c - q2 * s, q2 * c + q1 * s], axis=-1)",
                                   "np.concatenate([q2 * c + q1 * s, q1 * c - q2 * s], axis=-1)"),
}

SWIGLU_MUTANTS = {
    "swiglu_sigmoid_sign": ("return 1.0 / (1.0 + np.exp(-e))", "return 1.0 / (1.0 + np.exp(e))"),
    "swiglu_silu_is_sigmoid": ("return e * sigmoid(e)", "return sigmoid(e)"),
    "swiglu_fwd_f_not_rounded": ("f = _t(silu(e), dtype)", "f = silu(e)"),
    "swiglu_fwd_h_not_rounded": ("return _t(f * np.asarray(g, dtype=np.float64), dtype)",
                                 "return f * np.asarray(g, dtype=np.float64)"),
    "swiglu_bwd_f_not_rounded": ("f = _t(e * s, dtype)", "f = e * s"),
    "swiglu_bwd_h_not_rounded": ("h = _t(f * g, dtype)", "h = f * g"),
    "swiglu_df_uses_g": ("df = _t(dh * f, dtype)", "df = _t(dh * g, dtype)"),
    "swiglu_df_drops_dh": ("df = _t(dh * f, dtype)", "df = _t(f, dtype)"),
    "swiglu_de_drops_chain": ("de = _t(dh * g * s * (1.0 + e * (1.0 - s)), dtype)", "de = _t(dh * g * s, dtype)"),
    "swiglu_de_sign": ("de = _t(dh * g * s * (1.0 + e * (1.0 - s)), dtype)",
                       "de = _t(dh * g * s * (1.0 - e * (1.0 - s)), dtype)"),
    "swiglu_de_drops_g": ("de = _t(dh * g * s * (1.0 + e * (1.0 - s)), dtype)",
                          "de = _t(dh * s * (1.0 + e * (1.0 - s)), dtype)"),
    "swiglu_de_uses_rounded_f": ("de = _t(dh * g * s * (1.0 + e * (1.0 - s)), dtype)",
                                 "de = _t(dh * g * (s + f * (1.0 - s)), dtype)"),
    "swiglu_de_not_rounded": ("de = _t(dh * g * s * (1.0 + e * (1.0 - s)), dtype)",
                              "de = dh * g * s * (1.0 + e * (1.0 - s))"),
}


def _caught(mod, pins):
    caught = []
    for pin in pins:
        try:
            pin(mod)
        except Exception as e:
            caught.append((pin.__name__, type(e).__name__))
    return caught


@pytest.mark.parametrize("name", sorted(ROPE_MUTANTS))
def test_rope_mutant_is_caught(name):
    mod = _load_mutant(name, *ROPE_MUTANTS[name], src_path=ROPE_SRC)
    assert _caught(mod, oracle_pins_rope.ALL_PINS), f"no pin rejects the RoPE mutant {name!r}"


@pytest.mark.parametrize("name", sorted(SWIGLU_MUTANTS))
def test_swiglu_mutant_is_caught(name):
    src = open(SWIGLU_SRC).read()
    old, new = SWIGLU_MUTANTS[name]
    assert src.count(old) == 1, f"mutation {name!r} does not match the oracle source exactly once"
    # the SwiGLU oracle imports its rounding from the package: load the mutant as a package module
    mod = types.ModuleType(f"oracle.swiglu_mutant_{name}")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    assert _caught(mod, oracle_pins_swiglu.ALL_PINS), f"no pin rejects the SwiGLU mutant {name!r}"
