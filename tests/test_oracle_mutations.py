"""Planted mistakes in the oracle must be caught by its pins.

Each case copies the oracle's C source, plants one plausible mistake (a
dropped term, a wrong comparison, a swapped index, a wrong constant), builds
it with the same flags on the CPU, swaps it in for the real oracle, and runs
the deterministic pin battery below: at least one check must fail.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import build as obuild
from oracle import oracle as omod
import test_oracle_pins as pins

MUTATIONS = {
    "tie_to_largest_index": ("better = key < best_key[q];", "better = key <= best_key[q];"),
    "absmin_keeps_max": ("better = key < best_key[q];", "better = key > best_key[q];"),
    "row_col_swapped": ("int64_t r = l / N, j = l % N;", "int64_t r = l % R, j = l / R;"),
    "importance_dropped": ("fabsf(w) * (imp ? imp[j] : 1.0f)", "fabsf(w) * 1.0f"),
    "key_without_abs": ("float key = fabsf(w) *", "float key = (w) *"),
    "golden_ratio_constant": ("(uint32_t)(l * 0x9E3779B1u) ^ seed", "(uint32_t)(l * 0x9E3779B9u) ^ seed"),
    "fmix_shift": ("h ^= h >> 13;", "h ^= h >> 15;"),
    "seed_ignored": ("(uint32_t)(l * 0x9E3779B1u) ^ seed", "(uint32_t)(l * 0x9E3779B1u)"),
    "decode_block_index": ("What[i * N + j] = oracle_f16_to_f64(S[(i / R) * Bg + q]);",
                           "What[i * N + j] = oracle_f16_to_f64(S[(i % R) * Bg + q]);"),
    "decode_position": ("oracle_bucket((uint32_t)((i % R) * N + j), seed, (uint32_t)Bg);\n            What",
                        "oracle_bucket((uint32_t)(j * R + (i % R)), seed, (uint32_t)Bg);\n            What"),
    "product_abs_weight": ("acc += x * w;", "acc += x * fabs(w);"),
    "product_transposed_x": ("(double)load_as_f32(X, x_dtype, t * N + j);",
                             "(double)load_as_f32(X, x_dtype, j * 1 + t);"),
    "f16_truncates": ("double n = nearbyint(a / q);", "double n = floor(a / q);"),
    "f16_no_subnormals": ("if (E < -14)\n        E = -14;", "if (E < -14)\n        return sign;"),
    "empty_bucket_negzero": ("uint16_t v = 0;", "uint16_t v = 0x8000;"),
    "range_check_loose": ("fabsf(w) >= 65520.0f", "fabsf(w) > 65520.0f"),
    "importance_negative_allowed": ("imp[j] < 0.0f", "imp[j] < -1.0f"),
}


# planted mistakes in the multi-row sketch, caught by its own pins
ROWS_MUTATIONS = {
    "rows_share_one_seed": ("oracle_bucket(l, seed + (uint32_t)rho, Bgr)", "oracle_bucket(l, seed, Bgr)"),
    "rows_share_one_segment": ("return (uint32_t)rho * Bgr + oracle_bucket", "return 0u * Bgr + oracle_bucket"),
    "rows_decode_takes_min": ("int better = rule == OR_ABSMIN ? fabs(v) > fabs(best) : fabs(v) < fabs(best);",
                              "int better = rule == OR_ABSMIN ? fabs(v) < fabs(best) : fabs(v) > fabs(best);"),
    "rows_decode_ties_to_last": ("int better = rule == OR_ABSMIN ? fabs(v) > fabs(best)",
                                 "int better = rule == OR_ABSMIN ? fabs(v) >= fabs(best)"),
    "rows_encode_row0_only": ("uint32_t q = row_bucket((uint32_t)l, seed, rho, Bgr);",
                              "uint32_t q = row_bucket((uint32_t)l, seed, 0, Bgr);"),
    "rows_product_skips_row": ("acc += (double)load_as_f32(X, x_dtype, t * N + j) * decode_rows_one(N, R, Bg, seed, rule, rows,",
                               "acc += (double)load_as_f32(X, x_dtype, t * N + j) * decode_rows_one(N, R, Bg, seed, rule, rows - (rows > 2),"),
}

# planted mistakes in the importance-aware allocation, caught by its own pins
ALLOC_MUTATIONS = {
    "plan_ties_to_higher_block": ("if (!used[b] && (pick < 0 || rem[b] > rem[pick]))",
                                  "if (!used[b] && (pick < 0 || rem[b] >= rem[pick]))"),
    "plan_smallest_remainder_first": ("if (!used[b] && (pick < 0 || rem[b] > rem[pick]))",
                                      "if (!used[b] && (pick < 0 || rem[b] < rem[pick]))"),
    "plan_floor_not_reserved": ("const int64_t E = total - nb * lo;", "const int64_t E = total - nb;"),
    "importance_abs_not_square": ("acc += w * w * (double)a2[j];", "acc += fabs(w) * (double)a2[j];"),
    "alloc_encode_rotated_slot": ("S[off[b] + q] = v;", "S[off[b] + (q + 1) % Bg] = v;"),
    "alloc_decode_wrong_count": ("oracle_bucket((uint32_t)((i % R) * N + j), seed, (uint32_t)bg[b]);",
                                 "oracle_bucket((uint32_t)((i % R) * N + j), seed, (uint32_t)(bg[b] > 1 ? bg[b] - 1 : 1));"),
    "alloc_product_drops_last_column": ("for (int64_t j = 0; j < N; ++j)\n        acc += (double)load_as_f32(X, x_dtype, t * N + j) * decode_alloc_one",
                                        "for (int64_t j = 0; j < N - 1; ++j)\n        acc += (double)load_as_f32(X, x_dtype, t * N + j) * decode_alloc_one"),
}

# planted mistakes in the 4-bit buckets, caught by their own pins
Q4_MUTATIONS = {
    "q4_scale_over_8": ("uint16_t s16 = oracle_f32_to_f16(amax / 7.0f);", "uint16_t s16 = oracle_f32_to_f16(amax / 8.0f);"),
    "q4_truncates": ("float v = rintf(w / s);", "float v = truncf(w / s);"),
    "q4_nibbles_swapped": ("Tb[q / 2] |= (q % 2 == 0) ? nib : (uint8_t)(nib << 4);",
                           "Tb[q / 2] |= (q % 2 == 1) ? nib : (uint8_t)(nib << 4);"),
    "q4_unsigned_codes": ("return v >= 8 ? v - 16 : v;", "return v;"),
    "q4_scale_from_keys": ("float w = fabsf(load_as_f32(W, w_dtype, (b * R + l / N) * N + l % N));\n                    if (w > amax)",
                           "float w = best_key[q];\n                    if (w > amax)"),
    "q4_bucket_count_of_binary16": ("uint32_t q = oracle_bucket((uint32_t)l, seed, (uint32_t)Bg4);",
                                    "uint32_t q = oracle_bucket((uint32_t)l, seed, (uint32_t)(Bg4 / 4));"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(obuild.SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found: " + name
    mut = src.replace(old, new, 1)
    c = tmp_path / (name + ".c")
    c.write_text(mut)
    so = tmp_path / ("lib" + name + ".so")
    subprocess.run(["gcc", *obuild.CFLAGS, str(c), "-o", str(so), "-lm"], check=True)
    return omod.bind(ctypes.CDLL(str(so)))


BATTERY = [
    pins.test_bpw_accounting_golden,
    pins.test_hash32_published_murmur3_vectors,
    pins.test_bucket_map_matches_independent_hash,
    pins.test_f32_to_f16_all_bf16_patterns,
    pins.test_single_bucket_collapses_to_block_extreme,
    pins.test_constant_magnitude_keeps_sign_of_smallest_index,
    pins.test_single_collider_buckets_are_exact,
    pins.test_importance_changes_the_winner,
    pins.test_decode_is_S_times_P_transpose,
    pins.test_product_dense_identity_and_factorized_form,
    pins.test_product_constant_weight_closed_form,
    pins.test_encode_accepts_largest_finite_rounding,
    lambda: pins.test_encode_rejects_out_of_range_weights(65520.0, -2),
    lambda: pins.test_encode_rejects_bad_importance(-1.0),
    lambda: pins.test_membership_and_bound_on_outlier_linear(oracle.ABSMIN),
    lambda: pins.test_membership_and_bound_on_outlier_linear(oracle.ABSMAX),
    pins.test_outlier_linear_argmin_argmax_at_full_size,
]


def _brute_cases():
    g = np.random.default_rng(2024)
    for _ in range(12):
        R = int(g.integers(1, 5))
        N = int(g.integers(3, 20))
        Bg = int(g.choice([1, 2, 3, 5, 8]))
        M = R * int(g.integers(1, 4))
        W = (g.standard_normal((M, N))).astype(np.float32)
        if g.random() < 0.5:
            W = np.round(W * 2) / 2
        imp = g.choice(np.array([0.0, 0.5, 1.0, 2.0], dtype=np.float32), size=N)
        seed = int(g.integers(0, 2**32))
        for rule in (oracle.ABSMIN, oracle.ABSMAX):
            yield W, imp, R, Bg, seed, rule


def _brute_force_check():
    for W, imp, R, Bg, seed, rule in _brute_cases():
        M, N = W.shape
        S = oracle.encode(W, imp, R, 16.0 * Bg / (R * N), seed, rule)
        np.testing.assert_array_equal(S, pins.brute_encode(W, imp, R, Bg, seed, rule))


def test_battery_passes_on_real_oracle():
    for check in BATTERY + [_brute_force_check]:
        check()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(tmp_path, monkeypatch, name):
    old, new = MUTATIONS[name]
    lib = _build_mutant(tmp_path, name, old, new)
    monkeypatch.setattr(omod, "_lib", lib)
    failures = 0
    for check in BATTERY + [_brute_force_check]:
        try:
            check()
        except (AssertionError, oracle.OracleError, pytest.fail.Exception):
            failures += 1
    assert failures > 0, "planted mistake '%s' went unnoticed by every pin" % name


def _rows_battery():
    import test_oracle_rows as rp
    return [rp.test_rows_one_is_the_single_row_sketch,
            lambda: rp.test_each_row_is_an_independent_single_row_sketch(2, oracle.ABSMIN),
            lambda: rp.test_each_row_is_an_independent_single_row_sketch(4, oracle.ABSMAX),
            rp.test_multi_row_decode_brute_force,
            rp.test_multi_row_bound_and_max_over_rows,
            rp.test_multi_row_absmax_picks_the_smallest_magnitude,
            rp.test_multi_row_product_is_the_dense_product,
            rp.test_multi_row_ties_go_to_the_first_row]


@pytest.mark.parametrize("name", sorted(ROWS_MUTATIONS))
def test_planted_multi_row_mistake_is_caught(tmp_path, monkeypatch, name):
    old, new = ROWS_MUTATIONS[name]
    lib = _build_mutant(tmp_path, name, old, new)
    monkeypatch.setattr(omod, "_lib", lib)
    failures = 0
    for check in _rows_battery():
        try:
            check()
        except (AssertionError, oracle.OracleError, pytest.fail.Exception):
            failures += 1
    assert failures > 0, "planted mistake '%s' went unnoticed by every multi-row pin" % name


def _alloc_battery():
    import test_oracle_alloc as ap
    return [ap.test_plan_worked_example,
            ap.test_plan_ties_go_to_the_lower_block,
            lambda: ap.test_plan_properties(0),
            lambda: ap.test_plan_properties(3),
            ap.test_plan_largest_remainder_brute_force,
            ap.test_block_importance_is_expected_squared_output,
            ap.test_uniform_allocation_is_the_uniform_sketch,
            lambda: ap.test_each_block_is_a_brute_force_sketch_of_its_own_size(oracle.ABSMIN),
            ap.test_decode_and_product_of_an_allocated_sketch,
            ap.test_more_buckets_reconstruct_more_weights_exactly]


@pytest.mark.parametrize("name", sorted(ALLOC_MUTATIONS))
def test_planted_allocation_mistake_is_caught(tmp_path, monkeypatch, name):
    old, new = ALLOC_MUTATIONS[name]
    lib = _build_mutant(tmp_path, name, old, new)
    monkeypatch.setattr(omod, "_lib", lib)
    failures = 0
    for check in _alloc_battery():
        try:
            check()
        except (AssertionError, oracle.OracleError, pytest.fail.Exception):
            failures += 1
    assert failures > 0, "planted mistake '%s' went unnoticed by every allocation pin" % name


def _q4_battery():
    import test_oracle_q4 as qp
    return [qp.test_layout_same_bytes_as_binary16_buckets,
            lambda: qp.test_brute_force(oracle.ABSMIN),
            qp.test_codes_follow_the_binary16_sketch,
            qp.test_decode_and_product,
            qp.test_quantization_error_bound,
            qp.test_zero_and_underflowing_blocks_give_zero_codes]


@pytest.mark.parametrize("name", sorted(Q4_MUTATIONS))
def test_planted_q4_mistake_is_caught(tmp_path, monkeypatch, name):
    old, new = Q4_MUTATIONS[name]
    lib = _build_mutant(tmp_path, name, old, new)
    monkeypatch.setattr(omod, "_lib", lib)
    failures = 0
    for check in _q4_battery():
        try:
            check()
        except (AssertionError, oracle.OracleError, pytest.fail.Exception):
            failures += 1
    assert failures > 0, "planted mistake '%s' went unnoticed by every 4-bit pin" % name
