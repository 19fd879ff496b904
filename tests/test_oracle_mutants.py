"""Planted mistakes: each test compiles a copy of the C oracle with one plausible slip and
checks that the pin suite rejects it. This shows the pins constrain every part of the
definition (selection, sinks, bias sign, rotation, frequency, weights, scale, head map,
ring slot, chunk offsets, gradients), not only the parts a random-input comparison would notice. CPU only."""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "swa_oracle.c")

# (name, text in swa_oracle.c, replacement)
MUTANTS = [
    ("window_off_by_one", "int64_t lo = i - dil * (w - 1) > 0 ? i - dil * (w - 1) : 0;",
     "int64_t lo = i - dil * w > 0 ? i - dil * w : 0;"),
    ("chunk_window_off_by_one", "int64_t lo = i - w + 1 > 0 ? i - w + 1 : 0;",
     "int64_t lo = i - w > 0 ? i - w : 0;"),
    ("bias_sign", "slopes[h] * (double)(i - j)", "slopes[h] * (double)(j - i)"),
    ("rotation_sign", "y[2 * t] = a * c[t] - b * s[t];", "y[2 * t] = a * c[t] + b * s[t];"),
    ("rotation_pairing", "double a = x[2 * t], b = x[2 * t + 1];\n        y[2 * t] = a * c[t]",
     "double a = x[t], b = x[t + d / 2];\n        y[2 * t] = a * c[t]"),
    ("frequency", "double freq = pow(theta, -2.0 * (double)t / (double)d);\n            double phi",
     "double freq = pow(theta, -1.0 * (double)t / (double)d);\n            double phi"),
    ("sigmoid_sign", "x[e] = 1.0 / (1.0 + exp(-x[e]));", "x[e] = 1.0 / (1.0 + exp(x[e]));"),
    ("softmax_unnormalised", "x[e] /= z;", "x[e] /= 1.0;"),
    ("sinks_counted_twice", "for (int64_t j = 0; j < s && j < lo; ++j) key[n++] = j;",
     "for (int64_t j = 0; j < s && j <= i; ++j) key[n++] = j;"),
    ("gqa_head_map", "int64_t hk = h / group;\n                const double *qi",
     "int64_t hk = h % Hkv;\n                const double *qi"),
    ("ring_slot", "int64_t slot = p % w;", "int64_t slot = (p + 1) % w;"),
    ("scale", "if (scale <= 0.0) scale = 1.0 / sqrt((double)d);\n    int64_t nr",
     "if (scale <= 0.0) scale = 1.0 / (double)d;\n    int64_t nr"),
    ("chunk_query_position", "int64_t i = p0 + (row - cu[sq]);", "int64_t i = row - cu[sq];"),
    ("chunk_key_row", "int64_t src = cu[sq] + (j - p0);", "int64_t src = j - p0;"),
    ("chunk_key_rotation", "rotate_direct(kn, kt, d, j, theta);",
     "rotate_direct(kn, kt, d, p0, theta);"),
    ("chunk_boundary", "if (j >= p0) {", "if (j > p0) {"),
    ("bwd_sigmoid_derivative", "dp[e] * p * (1.0 - p)", "dp[e] * p"),
    ("bwd_softmax_row_term", "p * (dp[e] - rowsum)", "p * (dp[e] + rowsum)"),
    ("bwd_inverse_rotation", "dqi[2 * t] = a * c + bb * sv;", "dqi[2 * t] = a * c - bb * sv;"),
    ("bwd_scale", "dqr[c] += scale * dx * kr[j * d + c];", "dqr[c] += dx * kr[j * d + c];"),
    ("bwd_value_gradient", "dvj[c] += p * gi[c];", "dvj[c] += dx * gi[c];"),
    ("dilated_stride", "if ((i - j) % dil == 0 || j < s) key[n++] = j;",
     "if ((i - j) % (dil + 1) == 0 || j < s) key[n++] = j;"),
    ("dilated_sink_rule", "if ((i - j) % dil == 0 || j < s) key[n++] = j;",
     "if ((i - j) % dil == 0) key[n++] = j;"),
    ("dilated_bwd_key_set", "int64_t n = key_set(i, w, s, dil, key);\n                        for",
     "int64_t n = key_set(i, w, s, 1, key);\n                        for"),
]

PIN_TESTS = [
    (pins.test_band_mask_counts_match_page, {}),
    (pins.test_reach_by_mask_composition_matches_page, {}),
    (pins.test_selection_bit_readout, dict(N=33, w=7, s=9)),
    (pins.test_softmax_worked_example, {}),
    (pins.test_sigmoid_values, {}),
    (pins.test_alibi_closed_form_and_direction, dict(mode=oracle.SIGMOID)),
    (pins.test_rope_closed_form, dict(pair=3, theta=1e4)),
    (pins.test_softmax_equals_torch_sdpa_with_float_mask,
     dict(w=7, s=3, theta=1e4, alibi=True)),
    (pins.test_window_of_one, {}),
    (pins.test_windowed_loop_equals_dense_masked,
     dict(mode=oracle.SOFTMAX, w=13, s=5, Hq=4, Hkv=1, theta=1e6, alibi=True)),
    (pins.test_ring_slot_closed_form, dict(w=7)),
    (pins.test_append_writes_position_mod_w, dict(w=3)),
    (pins.test_decode_equals_prefill_row_by_row, dict(mode=oracle.SIGMOID, w=5, s=2)),
    (pins.test_chunked_prefill_equals_whole_prefill, dict(mode=oracle.SOFTMAX, w=6, s=2)),
    (pins.test_backward_matches_finite_differences,
     dict(mode=oracle.SOFTMAX, w=4, s=2, theta=1e4, alibi=True)),
    (pins.test_backward_window_of_one_closed_form, {}),
    (pins.test_dilated_selection_readout, dict(N=33, w=7, s=9, r=4)),
    (pins.test_dilated_selection_readout, dict(N=40, w=5, s=0, r=2)),
    (pins.test_dilated_backward_is_plain_backward_per_residue_class, dict(mode=oracle.SOFTMAX)),
]


def test_unmutated_oracle_passes_the_mutant_harness():
    for fn, kw in PIN_TESTS:
        fn(**kw)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_planted_mistake(name, old, new, tmp_path, monkeypatch):
    src = open(SRC).read()
    # an anchor shared by several functions is mutated in all of them
    assert src.count(old) >= 1, "mutation anchor not found: " + name
    mutant_c = tmp_path / ("oracle_%s.c" % name)
    mutant_c.write_text(src.replace(old, new))
    so = tmp_path / ("liboracle_%s.so" % name)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-o", str(so),
                    str(mutant_c), "-lm"], check=True)
    monkeypatch.setattr(oracle, "_lib", oracle.bind(str(so)))
    caught = []
    for fn, kw in PIN_TESTS:
        try:
            fn(**kw)
        except (AssertionError, ValueError):
            caught.append(fn.__name__)
    assert caught, "no pin caught the planted mistake " + name
