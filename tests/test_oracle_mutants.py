"""The pins are strong enough: each plausible mistake planted in a copy of the
oracle's C source fails at least one of them (CPU only).

A mutant is a textual edit of oracle.c (a dropped term, a flipped sign, a
wrong index, a skipped offset); it is compiled into a temporary library and
the pin tests are run against it.  The unmutated copy must pass them all.
"""
import os
import shutil
import subprocess

import pytest

import oracle
import test_oracle_attn as A
import test_oracle_rope as R

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

PINS = [
    R.test_split_matches_workload_statement,
    lambda: R.test_positions_match_raster_enumeration(18, 2925, 585, 30, 52),
    lambda: R.test_positions_match_raster_enumeration(5, 7, 200, 3, 5),
    R.test_positions_sp_slice_closed_form,
    R.test_identity_at_origin,
    lambda: R.test_table_closed_forms(64),
    lambda: R.test_table_closed_forms(128),
    R.test_table_matches_rotation_matrix_entries,
    lambda: R.test_norm_preserved_per_pair(64, 3),
    R.test_group_structure,
    R.test_relative_position_property,
    R.test_matches_brute_force_matrices_tiny,
    R.test_matches_brute_force_matrices_d128,
    R.test_append_is_a_transposed_copy,
    lambda: A.test_matches_brute_force_full_sequence_tiny(1),
    A.test_lse_is_natural_logsumexp,
    A.test_constant_values_give_that_constant,
    A.test_identical_keys_give_mean_of_visible_values,
    A.test_single_chunk_matches_torch_sdpa_fp64,
    lambda: A.test_future_chunks_and_capacity_do_not_leak(float("nan")),
    A.test_cache_form_equals_full_sequence_form,
    A.test_lse_merge_of_disjoint_key_sets,
]

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("rotation_by_minus_phi", "y[d0] = u * c - v * s;\n                        y[d0 + 1] = u * s + v * c;",
     "y[d0] = u * c + v * s;\n                        y[d0 + 1] = -u * s + v * c;"),
    ("dropped_term", "y[d0 + 1] = u * s + v * c;", "y[d0 + 1] = v * c;"),
    ("not_a_rotation", "y[d0] = u * c - v * s;", "y[d0] = u * c + v * s;"),
    ("freq_over_full_head_dim", "pow(theta, -2.0 * (double)j / (double)Da)",
     "pow(theta, -2.0 * (double)j / (double)(3 * Da))"),
    ("freq_missing_factor_two", "pow(theta, -2.0 * (double)j / (double)Da)",
     "pow(theta, -1.0 * (double)j / (double)Da)"),
    ("no_global_time_offset", "pos[3 * i + 0] = t0 + f;", "pos[3 * i + 0] = f;"),
    ("row_col_swapped", "pos[3 * i + 1] = in_frame / gw;\n        pos[3 * i + 2] = in_frame % gw;",
     "pos[3 * i + 1] = in_frame % gw;\n        pos[3 * i + 2] = in_frame / gw;"),
    ("axes_h_w_swapped", "double p = (double)pos[3 * i + a];",
     "double p = (double)pos[3 * i + (a == 0 ? 0 : 3 - a)];"),
    ("split_swapped", "*Dh = dhw;\n    *Dw = dhw;\n    *Dt = D - 2 * dhw;",
     "*Dt = dhw;\n    *Dw = dhw;\n    *Dh = D - 2 * dhw;"),
    ("table_sin_cos_swapped", "cos_out[e] = cos(phi);\n                sin_out[e] = sin(phi);",
     "cos_out[e] = sin(phi);\n                sin_out[e] = cos(phi);"),
    ("mask_hides_own_chunk", "if (j / J->chunk_tokens > q_chunk)\n            continue;\n        double acc",
     "if (j / J->chunk_tokens >= q_chunk && q_chunk > 0)\n            continue;\n        double acc"),
    ("mask_sees_next_chunk", "if (j / J->chunk_tokens > q_chunk)\n            continue;\n        double acc",
     "if (j / J->chunk_tokens > q_chunk + 1)\n            continue;\n        double acc"),
    ("mask_ignores_query_offset", "int64_t q_chunk = (J->q_pos0 + i) / J->chunk_tokens;",
     "int64_t q_chunk = i / J->chunk_tokens;"),
    ("scale_dropped", "s[j] = J->scale * acc;", "s[j] = acc;"),
    ("lse_log2", "m + log(l)", "m + log2(l)"),
    ("no_normalisation", "orow[d] /= l;", "orow[d] /= 1.0;"),
    ("values_from_keys", "orow[d] += p * vh[j * D + d];", "orow[d] += p * kh[j * D + d];"),
    ("max_not_subtracted_in_lse", "J->lse[((int64_t)b * J->H + h) * nr + r] = m + log(l);",
     "J->lse[((int64_t)b * J->H + h) * nr + r] = log(l);"),
    ("append_ignores_cache_pos", "cache[(((int64_t)b * H + h) * cap + cache_pos + i) * D + d]",
     "cache[(((int64_t)b * H + h) * cap + i) * D + d]"),
    ("append_head_token_transposed", "x[(((int64_t)b * n + i) * H + h) * D + d];",
     "x[(((int64_t)b * n + (i % n)) * H + (h % H)) * D + ((d + 1) % D)];"),
]


def _build(tmp_path, name, text):
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    out = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-o", str(out), str(src),
                    "-lm", "-lpthread"], check=True)
    return oracle.Oracle(str(out))


def _run_pins(variant):
    saved = oracle._default
    oracle._get()
    oracle._default = variant
    failed = []
    try:
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError) as e:  # noqa: PERF203
                failed.append((getattr(pin, "__name__", "pin"), type(e).__name__))
    finally:
        oracle._default = saved
    return failed


@pytest.fixture(scope="module")
def source():
    if shutil.which("gcc") is None:
        pytest.skip("no host C compiler")
    return open(SRC).read()


def test_unmutated_copy_passes_every_pin(tmp_path, source):
    assert _run_pins(_build(tmp_path, "clean", source)) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_a_pin(tmp_path, source, name, old, new):
    assert source.count(old) == 1, f"mutation site for {name} not unique/found"
    failed = _run_pins(_build(tmp_path, name, source.replace(old, new)))
    assert failed, f"mutant {name} passed every pin"
