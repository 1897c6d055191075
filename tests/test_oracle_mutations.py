"""Plant plausible mistakes in a scratch copy of the oracle (CPU only) and check
that the pins in test_oracle_pins.py reject every one of them."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fmlp_oracle.cpp")

MUTATIONS = {
    "eps_outside_sqrt": ("std::sqrt(ss / (double)d + eps)", "(std::sqrt(ss / (double)d) + eps)"),
    "sum_not_mean": ("std::sqrt(ss / (double)d + eps)", "std::sqrt(ss + eps)"),
    "gamma_dropped": ("* r * bf16_value(gamma[k])", "* r"),
    "gate_up_rows_swapped": ("gu, 0, 2, gu, 1, 2", "gu, 1, 2, gu, 0, 2"),
    "silu_on_up_branch": ("gate_act(act, g) * u", "gate_act(act, u) * g"),
    "w_down_transposed": ("wd[i] = dv.at(j, i);", "wd[i] = dv.at((i * d + j) / ff, (i * d + j) % ff);"),
    "round_half_away": ("float rq = std::nearbyint(ratio_k);", "float rq = std::round(ratio_k);"),
    "nibble_order_swapped": ("const uint8_t byte = qrow[k / 2];\n  const int nib = (k & 1) ? (byte >> 4) : (byte & 0xF);",
                             "const uint8_t byte = qrow[k / 2];\n  const int nib = (k & 1) ? (byte & 0xF) : (byte >> 4);"),
    "tile_slot_transposed": ("(((k % 32) / 8) * 16 + r % 16) * 8 + k % 8",
                             "((r % 16) * 4 + (k % 32) / 8) * 8 + k % 8"),
    "int4_tile_word_order": ("lane * 4 + g % 4", "(g % 4) * 64 + lane"),
    "sigmoid_not_silu": ("return t / (1.0 + std::exp(-t));", "return 1.0 / (1.0 + std::exp(-t));"),
    "gelu_erf_unscaled": ("std::erf(t / std::sqrt(2.0))", "std::erf(t)"),
    "gelu_tanh_cubic_coefficient": ("0.044715 * t * t * t", "0.0447 * t * t * t"),
    "gelu_forms_swapped": ("if (act == 1) return oracle_gelu_tanh(t);", "if (act == 1) return oracle_gelu_erf(t);"),
    "bf16_round_toward_zero": ("std::nearbyint(std::ldexp(a, 8 - e2))", "std::trunc(std::ldexp(a, 8 - e2))"),
    "residual_not_normalised": ("      xm = h.data();\n", "      (void)xm;\n"),
    "f16_subnormal_rounds_nearest": ("std::floor(std::ldexp(a, 24))", "std::nearbyint(std::ldexp(a, 24))"),
    "f16_sign_dropped": ("out[i] = (uint16_t)((w[i] & 0x8000u) | bits);", "out[i] = bits;"),
    "f16_exponent_bias": ("(((e2 - 1 + 15) << 10)", "(((e2 - 1 + 16) << 10)"),
    "f16_range_one_binade_high": ("a > 65504.0", "a > 65536.0"),
    "f16_weights_read_as_bf16": ("if (kind == 2) return f16[bf[row * K + k]];",
                                 "if (kind == 2) return bf16_value(bf[row * K + k]);"),
    "int4_scale_of_next_group": ("f16[s[row * (K / 32) + k / 32]]", "f16[s[row * (K / 32) + (k + 1) / 32]]"),
    "rms_mean_over_d_minus_1": ("std::sqrt(ss / (double)d + eps)", "std::sqrt(ss / (double)(d - 1) + eps)"),
    "token_chunk_offset_dropped": ("y[(m0 + m) * d + j] = acc;", "y[m * d + j] = acc;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_reject_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    text = open(SRC).read()
    assert old in text, f"mutation anchor for {name} no longer in the oracle"
    src = tmp_path / "mutant.cpp"
    src.write_text(text.replace(old, new, 1))
    env = dict(os.environ, FMLP_ORACLE_SRC=str(src), FMLP_ORACLE_LIB=str(tmp_path / "libmutant.so"),
               OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins accepted mutant {name}:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout
