"""Each plausible mistake planted in a copy of the oracle fails at least one pin.

The copy is compiled with gcc into a temporary directory on the CPU; the
real oracle source is never modified.
"""
import os
import re
import subprocess

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "dsc_oracle.c")

# (name, exact source fragment, replacement, expected occurrences)
MUTANTS = [
    ("drop_residual_fwd", "double acc = residual ? x[n * D + d] : 0.0;", "double acc = 0.0;", 3),
    ("drop_residual_dx", "double acc = residual ? g[m * D + d] : 0.0;", "double acc = 0.0;", 3),
    ("unshifted_tap", "w[(n * G + d / H) * W + k] * x[(n - k) * D + d]",
     "w[(n * G + d / H) * W + k] * x[n * D + d]", 1),
    ("strict_segment_test", "if (n - k >= seg[n]) acc += w", "if (n - k > seg[n]) acc += w", 1),
    ("group_modulo", "w[(n * G + d / H) * W + k] * x", "w[(n * G + d % G) * W + k] * x", 1),
    ("reversed_taps", "w[(n * G + d / H) * W + k] * x", "w[(n * G + d / H) * W + (W - 1 - k)] * x", 1),
    ("dx_wrong_segment", "if (n < N && m >= seg[n]) acc += w", "if (n < N) acc += w", 1),
    ("dx_tap_of_m", "acc += w[(n * G + d / H) * W + k] * g[n * D + d];",
     "acc += w[(m * G + d / H) * W + k] * g[n * D + d];", 1),
    ("dw_unshifted", "acc += g[m * D + d] * x[(m - k) * D + d];", "acc += g[m * D + d] * x[m * D + d];", 1),
    ("U_transposed", "U[(int64_t)r * D * W + d * W + k];", "U[(int64_t)r * D * W + k * D + d];", 2),
    ("lowrank_fwd_no_shift", "lowrank_filter(D, W, R, z, U, n, d, k) * x[(n - k) * D + d]",
     "lowrank_filter(D, W, R, z, U, n, d, k) * x[n * D + d]", 1),
    ("lowrank_dx_filter_at_m", "lowrank_filter(D, W, R, z, U, n, d, k) * g[n * D + d]",
     "lowrank_filter(D, W, R, z, U, m, d, k) * g[n * D + d]", 1),
    ("dz_transposed_U", "acc += U[(int64_t)r * D * W + d * W + k] * (g[m * D + d]",
     "acc += U[(int64_t)r * D * W + k * D + d] * (g[m * D + d]", 1),
    ("dz_missing_mask", "if (m - k >= seg[m])\n                        acc += U", "if (1)\n                        acc += U", 1),
    ("dU_wrong_z", "acc += z[n * R + r] * (g[n * D + d]", "acc += z[n * R + (R - 1 - r)] * (g[n * D + d]", 1),
    ("dU_unshifted", "(g[n * D + d] * x[(n - k) * D + d]);", "(g[n * D + d] * x[n * D + d]);", 1),
    ("segment_from_row", "seg[n] = cu_seqlens[i];", "seg[n] = (n / T) * T;", 1),
    ("static_unshifted", "acc += c[d * W + k] * x[(n - k) * D + d];", "acc += c[d * W + k] * x[n * D + d];", 1),
    ("static_reversed_taps", "acc += c[d * W + k] * x[", "acc += c[d * W + (W - 1 - k)] * x[", 1),
    ("static_no_mask", "if (n - k >= seg[n]) acc += c[", "if (n - k >= 0) acc += c[", 1),
    ("static_dx_filter_lag", "acc += c[d * W + k] * g[n * D + d];", "acc += c[d * W + k] * g[m * D + d];", 1),
    ("static_dx_no_mask", "if (n < N && m >= seg[n]) acc += c[", "if (n < N) acc += c[", 1),
    ("static_dc_unshifted", "acc += g[n * D + d] * x[(n - k) * D + d];", "acc += g[n * D + d] * x[n * D + d];", 1),
    ("static_dc_no_mask", "if (n - k >= seg[n]) acc += g[", "if (n - k >= 0) acc += g[", 1),
    ("decode_state_slot", "state[(b * (W - 1) + (k - 1)) * D + d];", "state[(b * (W - 1) + (W - 1 - k)) * D + d];", 2),
    ("decode_no_shift", "state[(b * (W - 1) + i) * D + d] = state[(b * (W - 1) + i - 1) * D + d];",
     "state[(b * (W - 1) + i) * D + d] = state[(b * (W - 1) + i) * D + d];", 2),
    ("decode_lowrank_U_transposed", "wk += z[b * R + r] * U[(int64_t)r * D * W + d * W + k];",
     "wk += z[b * R + r] * U[(int64_t)r * D * W + k * D + d];", 1),
    ("prefill_off_by_one", "const int64_t t = hi - 1 - i;", "const int64_t t = hi - i;", 1),
    ("prefill_pads_with_first_token", "= t >= lo ? x[t * D + d] : 0.0;", "= t >= lo ? x[t * D + d] : x[lo * D + d];", 1),
    ("rope_sin_sign", "b[h + 2 * i + 1] = q * c + p * s;", "b[h + 2 * i + 1] = q * c - p * s;", 1),
    ("rope_theta_exponent", "pow(base, -2.0 * i / hd)", "pow(base, -1.0 * i / hd)", 2),
    ("rope_position_global", "const double m = (double)(n - seg[n]);", "const double m = (double)n;", 1),
    ("rope_rotates_values", "for (int64_t h = 0; h < rot; h += hd)", "for (int64_t h = 0; h + hd <= D; h += hd)", 1),
    ("rope_backward_not_inverted", "const double sign = inverse ? -1.0 : 1.0;", "const double sign = 1.0;", 1),
    ("rope_half_split_pairs", "const double p = a[h + 2 * i], q = a[h + 2 * i + 1];",
     "const double p = a[h + i], q = a[h + i + hd / 2];", 1),
    ("rope_table_cos_sin_swapped", "table[(m * (hd / 2) + i) * 2 + 0] = cos(ang);",
     "table[(m * (hd / 2) + i) * 2 + 0] = sin(ang);", 1),
    ("generate_V_transposed", "acc += h[n * K + j] * V[c * K + j];", "acc += h[n * K + j] * V[j * C + c];", 1),
    ("generate_dh_reversed", "acc += dw[n * C + c] * V[c * K + j];", "acc += dw[n * C + c] * V[c * K + (K - 1 - j)];",
     1),
    ("generate_dV_wrong_row", "acc += dw[n * C + c] * h[n * K + j];",
     "acc += dw[n * C + c] * h[(N - 1 - n) * K + j];", 1),
    ("rope_decode_position_off_by_one", "rotate_row(D, rot, hd, base, (double)pos[b], 1.0,",
     "rotate_row(D, rot, hd, base, (double)(pos[b] + 1), 1.0,", 1),
]


@pytest.mark.parametrize("name,old,new,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, count):
    src = open(SRC).read()
    assert src.count(old) == count, f"fragment for {name} found {src.count(old)} times"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    so = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(mutant), "-o", so, "-lm"],
                   check=True)
    orc = oracle.Oracle(oracle.load(so))
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
