"""Plant plausible mistakes in copies of the oracle's C source (on the CPU)
and show that every one of them fails at least one pin of
test_oracle_pins.py.  The shipped oracle is never modified."""
import os
import tempfile

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kvq_oracle.c")

# (name, text to find, replacement, occurrence index of the match to change)
MUTANTS = [
    ("butterfly_sign", "x[j + h] = a - b;", "x[j + h] = b - a;", 0),
    ("butterfly_order", "for (int h = 1; h < d; h *= 2) {", "for (int h = d / 2; h >= 1; h /= 2) {", 0),
    ("no_normalisation", "for (int k = 0; k < d; ++k) x[k] = x[k] * c;", "(void)c;", 0),
    ("f64_no_normalisation", "for (int k = 0; k < d; ++k) x[k] = x[k] * c;", "(void)c;", 1),
    ("scale_off_by_one", "int e = (E - 1) - emax_elem;", "int e = E - emax_elem;", 0),
    ("scale_clamp", "if (e < -127) e = -127;", "if (e < -126) e = -126;", 0),
    ("ties_to_odd", "(dk == best_d && (k % 2) == 0)", "(dk == best_d && (k % 2) == 1)", 0),
    ("ties_away", "(dk == best_d && (k % 2) == 0)", "(dk == best_d)", 0),
    ("sign_of_zero", "return best | (signbit(y) ? 8 : 0);", "return best | ((y < 0) ? 8 : 0);", 0),
    ("grid_typo", "3.0, 4.0, 6.0}", "3.0, 4.0, 5.0}", 0),
    ("nibble_order", "(uint8_t)(lo | (hi << 4));", "(uint8_t)(hi | (lo << 4));", 0),
    ("amax_no_abs", "if (fabsf(y[c]) > amax) amax = fabsf(y[c]);", "if (y[c] > amax) amax = y[c];", 0),
    ("dequant_scale_bias", "scales[c / 32] - 127);\n  }", "scales[c / 32] - 126);\n  }", 0),
    ("e4m3_bias", "v = ldexp(1.0 + m / 8.0, e - 7);", "v = ldexp(1.0 + m / 8.0, e - 8);", 0),
    ("e4m3_subnormal", "v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);", 0),
    ("e4m3_ties_to_odd", "(dk == best_d && (k % 2) == 0)", "(dk == best_d && (k % 2) == 1)", 1),
    ("no_causal_mask", "const int last = L - n_q + j; /* inclusive */", "const int last = L - 1;", 0),
    ("gqa_modulo", "const int kv = h / g;", "const int kv = h % hkv;", 0),
    ("no_softmax_scale", "s[t] = sm_scale * acc;", "s[t] = acc;", 0),
    ("unnormalised_weights", "const double p = s[t] / Z;", "const double p = s[t];", 0),
    ("q_not_rotated", "if (rotate) orc_fwht_f32(tmp, d);", "(void)0;", 0),
    ("out_not_rotated_back", "for (size_t r = 0; r < (size_t)n_q * hq; ++r) orc_fwht_f64(out + r * d, d);", "(void)0;", 0),
]


def _mutate(text, find, repl, occ):
    idx = -1
    for _ in range(occ + 1):
        idx = text.find(find, idx + 1)
        assert idx >= 0, "mutation anchor not found: %r (occurrence %d)" % (find, occ)
    return text[:idx] + repl + text[idx + len(find):]


PIN_CALLS = [
    lambda: [pins.test_fwht_unit_vectors_exact_sylvester_signs(d) for d in (32, 128)],
    lambda: [pins.test_fwht_f64_equals_sylvester_product(d) for d in (32, 128)],
    lambda: [pins.test_fwht_f32_close_to_exact_and_involution(d) for d in (32, 128)],
    pins.test_fwht_f32_butterfly_order,
    lambda: pins.test_scale_byte_closed_form(2, 125),
    lambda: pins.test_scale_byte_closed_form(8, 119),
    pins.test_e2m1_decode_table,
    pins.test_e2m1_rounding_table,
    pins.test_e2m1_grid_round_trips_at_every_scale,
    pins.test_e2m1_sign_of_zero_and_saturation,
    pins.test_e4m3_decode_matches_torch,
    pins.test_e4m3_encode_matches_torch_cast,
    pins.test_byte_budget_matches_page,
    pins.test_nibble_order_and_scale_of_a_known_vector,
    lambda: pins.test_quantize_error_bound_and_scale_rule(128),
    pins.test_fp8_vector_error_bound,
    lambda: pins.test_attend_matches_numpy_scipy(33, 3, 8, 2, 32),
    pins.test_attend_special_cases,
    pins.test_gqa_head_mapping,
    pins.test_rotation_invariance_without_quantisation,
    pins.test_decode_rotated_cache_matches_plain_attention,
]


def _failing_pins(L):
    failed = []
    with oracle.use_library(L):
        for i, call in enumerate(PIN_CALLS):
            try:
                call()
            except AssertionError:
                failed.append(i)
    return failed


def test_unmutated_source_passes_all_pins(tmp_path):
    out = str(tmp_path / "orc_clean.so")
    oracle.compile_source(SRC, out)
    assert _failing_pins(oracle.load(out)) == []


@pytest.mark.parametrize("name,find,repl,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, find, repl, occ):
    text = open(SRC).read()
    src = tmp_path / ("orc_%s.c" % name)
    src.write_text(_mutate(text, find, repl, occ))
    out = str(tmp_path / ("orc_%s.so" % name))
    oracle.compile_source(str(src), out)
    assert _failing_pins(oracle.load(out)), "planted mistake %s passed every pin" % name
