"""Planted mistakes: each mutant copy of the oracle must fail at least one pin.

The mutants are textual edits of oracle.c compiled into a temporary library on
the CPU; the real oracle is untouched.  This shows that the pins in
test_oracle_pins.py are strong enough to catch a dropped term, a wrong sign, a
wrong index or a transposed operand.
"""
import ctypes
import os
import subprocess

import pytest

from oracle import replay_oracle as ro
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "oracle.c")

MUTANTS = {
    "mamba2_no_decay": ("a * s[(size_t)p * N + n] + d * xv[p] * bv[n]", "s[(size_t)p * N + n] + d * xv[p] * bv[n]"),
    "mamba2_update_sign": ("a * s[(size_t)p * N + n] + d * xv[p] * bv[n]", "a * s[(size_t)p * N + n] - d * xv[p] * bv[n]"),
    "mamba2_no_dt": ("a * s[(size_t)p * N + n] + d * xv[p] * bv[n]", "a * s[(size_t)p * N + n] + xv[p] * bv[n]"),
    "mamba2_B_for_C": ("acc += s[(size_t)p * N + n] * cv[n];", "acc += s[(size_t)p * N + n] * bv[n];"),
    "mamba2_drop_D": ("acc + D[h] * xv[p]", "acc"),
    "mamba2_group_index": ("const int g = h / heads_per_group;\n            double *s = S + ((size_t)b * H + h) * (size_t)P * N;",
                           "const int g = h % G;\n            double *s = S + ((size_t)b * H + h) * (size_t)P * N;"),
    "gdn_alpha_on_state_only": ("al * (s[(size_t)i * DK + j] - be * u * kv[j])", "al * s[(size_t)i * DK + j] - be * u * kv[j]"),
    "gdn_beta_sign": ("+ be * vv[i] * kv[j]", "- be * vv[i] * kv[j]"),
    "gdn_transposed_Sk": ("u += s[(size_t)i * DK + j] * kv[j];", "u += s[(size_t)(j % DV) * DK + (i % DK)] * kv[j];"),
    "gdn_readout_k": ("acc += nv * qv[j];", "acc += nv * kv[j];"),
    "gdn_no_scale": ("= scale * acc;", "= acc;"),
    "e4m3_ties_odd": ("(err == best_err && (c & 1) == 0)) {\n            best = c;\n            best_err = err;\n        }\n    }\n    return sign | best;\n}\n\n/* FP4",
                      "(err == best_err && (c & 1) == 1)) {\n            best = c;\n            best_err = err;\n        }\n    }\n    return sign | best;\n}\n\n/* FP4"),
    "e4m3_bias8": ("ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)"),
    "e2m1_ties_odd": ("(err == best_err && (c & 1) == 0)) {\n            best = c;\n            best_err = err;\n        }\n    }\n    return sign | best;        /*",
                      "(err == best_err && (c & 1) == 1)) {\n            best = c;\n            best_err = err;\n        }\n    }\n    return sign | best;        /*"),
    "mx_scale_off_by_one": ("X = (e2 - 1) - 2;          /*", "X = (e2 - 1) - 1;          /*"),
    "mx_no_saturation_floor": ("X = (e2 - 1) - 2;          /*", "X = e2 - 2;          /*"),
    "mx_ceil_strict": ("!(amax <= ldexp(6.0, X))", "!(amax < ldexp(6.0, X))"),
    "mx_ceil_is_floor_plus_one": ("!(amax <= ldexp(6.0, X))", "!(amax < ldexp(4.0, X))"),
}

PIN_TESTS = [
    lambda: pins.test_mamba2_matches_unrolled_sum(1),
    lambda: pins.test_mamba2_matches_unrolled_sum(2),
    pins.test_mamba2_single_step_from_zero,
    pins.test_mamba2_zero_decay_is_running_sum,
    pins.test_mamba2_zero_dt_keeps_state,
    pins.test_mamba2_group_mapping,
    lambda: pins.test_gdn_matches_transition_products(1),
    pins.test_gdn_rectangular_state_orientation,
    pins.test_gdn_zero_beta_is_pure_decay,
    pins.test_gdn_unit_beta_overwrites_key_direction,
    pins.test_gdn_single_step_from_zero,
    pins.test_gdn_orthonormal_keys_projection,
    pins.test_e4m3_table_landmarks,
    pins.test_e4m3_encode_matches_torch_cast_in_range,
    pins.test_e2m1_table_and_ties,
    pins.test_mxfp4_block_scale_rule,
    pins.test_mxfp4_ceil_scale_rule,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} must match exactly once"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", str(src), "-o", str(so), "-lm"],
                   check=True)
    prev = ro.use_library(ro.configure(ctypes.CDLL(str(so))))
    failures = 0
    try:
        for pin in PIN_TESTS:
            try:
                pin()
            except AssertionError:
                failures += 1
    finally:
        ro.use_library(prev)
    assert failures > 0, f"mutant {name} passed every pin"
