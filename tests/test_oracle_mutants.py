"""The oracle's pins catch plausible mistakes.

Each case plants one mistake (a dropped term, a wrong sign, index or operand,
a wrong rounding) in a copy of the oracle's C source, builds it on the CPU,
and runs the pins of ``test_oracle.py`` against the mutant: at least one
must fail.
"""
import functools
import os
import subprocess
import tempfile

import pytest

import oracle
import test_oracle as T

MUTANTS = {
    "embbag_drops_last_index": ("p < off[kb + 1]; ++p", "p + 1 < off[kb + 1]; ++p",
                                ["test_embbag_dyadic_exact_and_linear", "test_embbag_brute_force_tiny"]),
    "embbag_wrong_table": ("tables[k] + idx[p]", "tables[0] + idx[p]",
                           ["test_embbag_one_index_bag_is_row_lookup", "test_embbag_dyadic_exact_and_linear"]),
    "embbag_negative_zero_init": ("o[c] = 0.0f;", "o[c] = -0.0f;", ["test_embbag_empty_bag_is_positive_zero"]),
    "interact_reversed_column_index": ("o[d + (int64_t)i * (i - 1) / 2 + j]", "o[d + (int64_t)i * (i - 1) / 2 + (i - 1 - j)]",
                                       ["test_interact_integer_X_exact_against_integer_gram"]),
    "interact_transposed_operand": ("(double)x[(int64_t)j * d + c]", "(double)x[(int64_t)c * d + j]",
                                    ["test_interact_integer_X_exact_against_integer_gram", "test_interact_against_torch_bmm_fp64"]),
    "interact_drops_last_pair": ("for (int32_t j = 0; j < i; ++j)", "for (int32_t j = 0; j + 1 < i; ++j)",
                                 ["test_interact_integer_X_exact_against_integer_gram"]),
    "interact_dense_row_missing": ("for (int32_t c = 0; c < d; ++c) o[c] = x[c];", "",
                                   ["test_interact_integer_X_exact_against_integer_gram", "test_hand_example_forward_and_sgd"]),
    "interact_bwd_lower_half_only": ("if (j == i) continue;", "if (j >= i) continue;",
                                     ["test_interact_bwd_structure", "test_interact_bwd_against_autograd"]),
    "interact_bwd_no_dense_part": ("double s = (i == 0) ? (double)gb[c] : 0.0;", "double s = 0.0;",
                                   ["test_interact_bwd_structure", "test_interact_bwd_finite_differences"]),
    "interact_bwd_reversed_pair_index": ("gb[d + (int64_t)a * (a - 1) / 2 + e]", "gb[d + (int64_t)a * (a - 1) / 2 + (a - 1 - e)]",
                                         ["test_interact_bwd_structure", "test_interact_bwd_against_autograd"]),
    "interact_bwd_own_row": ("(double)xr[(int64_t)j * d + c]", "(double)xr[(int64_t)i * d + c]",
                             ["test_interact_bwd_structure", "test_interact_bwd_finite_differences"]),
    "mlp_drops_bias": ("float y = (float)(s + (double)bias[l][o]);", "float y = (float)s;",
                       ["test_mlp_against_torch_linear", "test_hand_example_forward_and_sgd"]),
    "mlp_relu_on_logit": ("const int relu = (l < L - 1) || last_relu;\n        for (int32_t o = 0; o < fo; ++o) {\n          const float* w",
                          "const int relu = 1;\n        for (int32_t o = 0; o < fo; ++o) {\n          const float* w",
                          ["test_mlp_against_torch_linear", "test_mlp_identity_weights_give_relu"]),
    "bf16_round_half_up": ("u += 0x7fffu + ((u >> 16) & 1u);", "u += 0x8000u;", ["test_bf16_round_against_torch"]),
    "bf16_truncates": ("u += 0x7fffu + ((u >> 16) & 1u);", "", ["test_bf16_round_against_torch"]),
    "mlp_bwd_no_relu_mask": ("delta[b * fo + o] = (relu && !(y[b * fo + o] > 0.0f)) ? 0.0 : gv;", "delta[b * fo + o] = gv;",
                             ["test_mlp_bwd_against_autograd", "test_mlp_bwd_finite_differences"]),
    "mlp_bwd_transposed_weight": ("(double)W[l][(int64_t)o * fi + i]", "(double)W[l][(int64_t)(i % fo) * fi + (o % fi)]",
                                  ["test_mlp_bwd_against_autograd"]),
    "lp_int8_fused_multiply_add": ("const float prod = sb[2 * r] * (float)q;\n  return prod + sb[2 * r + 1];",
                                   "return fmaf(sb[2 * r], (float)q, sb[2 * r + 1]);",
                                   ["test_embbag_lp_int8_two_roundings"]),
    "lp_int8_drops_bias": ("return prod + sb[2 * r + 1];", "return prod;", ["test_embbag_lp_int8_affine_dyadic"]),
    "lp_int8_unsigned_bytes": ("const int8_t q = ((const int8_t*)table)", "const uint8_t q = ((const uint8_t*)table)",
                               ["test_embbag_lp_int8_unit_scale_is_integer_sum"]),
    "lp_bf16_low_half": ("const uint32_t u = (uint32_t)h << 16;", "const uint32_t u = (uint32_t)h;",
                         ["test_embbag_lp_bf16_is_exact_widening"]),
    "sgd_wrong_sign": ("T[r * (int64_t)d + c] - step", "T[r * (int64_t)d + c] + step",
                       ["test_sparse_sgd_single_occurrence_and_untouched", "test_sparse_sgd_dyadic_exact"]),
    "sgd_ignores_table_slot": ("G + b * g_ld + g_col0 + (int64_t)k * d", "G + b * g_ld + g_col0",
                               ["test_sparse_sgd_matches_sort_based_formulation", "test_sparse_sgd_dyadic_exact"]),
    "sgd_plain_order": ("count[r] > 0 && count[r] % SGD_BLOCK == 0", "0",
                        ["test_sparse_sgd_long_rows_sum_in_blocks_of_128"]),
    "sgd_block_of_64": ("count[r] % SGD_BLOCK == 0", "count[r] % 64 == 0",
                        ["test_sparse_sgd_long_rows_sum_in_blocks_of_128"]),
    "sgd_drops_last_block": ("acc[r * (int64_t)d + c] + blk[r * (int64_t)d + c]", "acc[r * (int64_t)d + c]",
                             ["test_sparse_sgd_single_occurrence_and_untouched", "test_sparse_sgd_dyadic_exact"]),
    "sgd_never_marks_touched": ("touched[r] = 1;", "",
                                   ["test_sparse_sgd_single_occurrence_and_untouched", "test_sparse_sgd_matches_sort_based_formulation"]),
}

PARAMS = {
    "test_interact_integer_X_exact_against_integer_gram": [dict(n=9, d=16), dict(n=27, d=128)],
    "test_mlp_against_torch_linear": [dict(name="tiny", which="top"), dict(name="forward", which="top"),
                                      dict(name="forward", which="bottom")],
}


class _Bound:
    def __init__(self, L):
        self.L = L

    def __getattr__(self, name):
        return functools.partial(getattr(oracle, name), L=self.L)


@pytest.fixture(scope="module")
def tmpdir_mod():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmpdir_mod):
    old, new, pins = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path_c = os.path.join(tmpdir_mod, f"{name}.c")
    path_so = os.path.join(tmpdir_mod, f"{name}.so")
    open(path_c, "w").write(src.replace(old, new))
    subprocess.run(["gcc", *oracle.CFLAGS, path_c, "-o", path_so, "-lm"], check=True)
    mut = _Bound(oracle.lib(path_so))
    caught = []
    for pin in pins:
        for kw in PARAMS.get(pin, [{}]):
            try:
                getattr(T, pin)(mut, **kw)
            except (AssertionError, ValueError, IndexError):
                caught.append((pin, kw))
    assert caught, f"no pin caught mutant {name}"
