"""The oracle's pins must catch plausible mistakes: each case below plants one
mistake in a copy of lid_oracle.c (on the CPU), builds it, and requires that
at least one pin of tests/test_oracle.py fails against the broken copy."""
import os

import numpy as np
import pytest

import oracle
import test_oracle as T  # noqa: E402

SRC = os.path.join(os.path.dirname(oracle.__file__), "lid_oracle.c")

MUTATIONS = {
    "no_relu": ("if (dot > 0.0)              /*", "if (1)              /*"),
    "abs_for_relu": ("if (dot > 0.0)              /* ReLU: a non-positive dot contributes nothing */\n            I += wd[h] * dot;",
                     "I += wd[h] * fabs(dot);"),
    "w_inside_relu": ("if (dot > 0.0)              /* ReLU: a non-positive dot contributes nothing */\n            I += wd[h] * dot;",
                      "if (wd[h] * dot > 0.0)\n            I += wd[h] * dot;"),
    "transposed_q": ("qd[(int64_t)h * D + d] * kd[d]", "qd[(int64_t)d * H + h] * kd[d]"),
    "dropped_last_head": ("for (int h = 0; h < H; ++h) {\n        double dot", "for (int h = 0; h < H - 1; ++h) {\n        double dot"),
    "dropped_last_dim": ("for (int d = 0; d < D; ++d)\n            dot +=", "for (int d = 1; d < D; ++d)\n            dot +="),
    "tie_by_larger_index": ("return (x->s < y->s) ? -1 : (x->s > y->s);", "return (x->s > y->s) ? -1 : (x->s < y->s);"),
    "ascending_scores": ("if (x->v > y->v) return -1;\n    if (x->v < y->v) return 1;",
                         "if (x->v < y->v) return -1;\n    if (x->v > y->v) return 1;"),
    "mask_ignored": ("v = v + (float)lid_oracle_f16_to_f64(mask[t * mask_ld + s]);", "(void)0;"),
    "mask_subtracted": ("v = v + (float)lid_oracle_f16_to_f64(mask[t * mask_ld + s]);",
                        "v = v - (float)lid_oracle_f16_to_f64(mask[t * mask_ld + s]);"),
    "range_lo_off_by_one": ("for (int64_t s = lo; s < hi; ++s) {\n            double I", "for (int64_t s = lo + 1; s < hi; ++s) {\n            double I"),
    "range_ignored": ("    if (kv_range) {\n        a = kv_range[2 * t];", "    if (0) {\n        a = kv_range[2 * t];"),
    "f16_exponent_bias": ("v = ldexp((double)(1024 + m), e - 25);", "v = ldexp((double)(1024 + m), e - 24);"),
    "f16_subnormal": ("v = ldexp((double)m, -24);", "v = ldexp((double)m, -23);"),
    "no_padding": ("idx_out[t * k_top + j] = valid ? (int32_t)c[j].s : -1;", "idx_out[t * k_top + j] = valid ? (int32_t)c[j].s : 0;"),
    "neg_zero_kept": ("*out = v + 0.0f;", "*out = v;"),
    "f8_exponent_bias": ("v = ldexp((double)(8 + m), e - 10);", "v = ldexp((double)(8 + m), e - 11);"),
    "f8_subnormal": ("v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    "k_scale_wrong_row": ("kd[i] *= (double)k_scale[i / D];", "kd[i] *= (double)k_scale[i % D];"),
    "q_scale_wrong_head": ("qd[i] *= (double)q_scale[t * H + i / D];\n        }\n        for (int h = 0; h < H; ++h)\n            wd[h] = (double)w[t * H + h];\n\n        int64_t n = 0;",
                           "qd[i] *= (double)q_scale[t * H];\n        }\n        for (int h = 0; h < H; ++h)\n            wd[h] = (double)w[t * H + h];\n\n        int64_t n = 0;"),
    "shared_skips_minus_inf": ("if (isinf(v)) { selectable = 0; break; }                 /* -inf term */",
                               "if (isinf(v)) { continue; }                 /* -inf term */"),
    "shared_range_ignored": ("if (s < lo[t] || s >= hi[t]) { selectable = 0; break; }   /* v = -inf */",
                             "if (0) { selectable = 0; break; }   /* v = -inf */"),
    "shared_first_query_only": ("for (int64_t t = 0; t < n_tok && selectable; ++t) {",
                                "for (int64_t t = 0; t < 1 && selectable; ++t) {"),
    "shared_w_of_first_query": ("double I = head_reduced_score(qd + t * H * D, wd + t * H, kd + s * D, H, D);",
                                "double I = head_reduced_score(qd + t * H * D, wd, kd + s * D, H, D);"),
    "shared_max_not_sum": ("U += (double)v;", "U = U > (double)v ? U : (double)v;"),
    "attn_no_scale": ("s[j] = scale * dot;", "s[j] = dot;"),
    "attn_not_normalised": ("for (int32_t d = 0; d < L; ++d) o[d] /= den;", "(void)den;"),
    "attn_first_row_only": ("for (int32_t j = 0; j < k_sel; ++j) {\n                if (s[j] == -INFINITY) continue;",
                            "for (int32_t j = 0; j < 1; ++j) {\n                if (s[j] == -INFINITY) continue;"),
    "attn_no_max_shift": ("const double p = exp(s[j] - mx);", "const double p = exp(s[j] - 0.5 * mx);"),
}

PINS = [
    T.test_golden_hand_example,
    lambda o: T.test_closed_form_single_head_single_dim(o, 0),
    T.test_zero_query_ties_resolve_by_index,
    T.test_underflowing_negative_score_is_positive_zero,
    *[(lambda s: (lambda o: T.test_bruteforce_exact_small_integers(o, s)))(s) for s in range(6)],
    lambda o: T.test_bruteforce_random(o, "f16"),
    T.test_f16_decode_exhaustive,
    T.test_invariants_random,
    T.test_f8e4m3_decode_exhaustive,
    lambda o: T.test_f8_scaled_equals_dequantised(o, 0),
    T.test_f8_closed_form_single_head_single_dim,
    *[(lambda s: (lambda o: T.test_shared_bruteforce_exact(o, s)))(s) for s in range(4)],
    T.test_shared_bruteforce_random,
    T.test_shared_one_query_is_per_query_topk,
    T.test_shared_identical_queries_scale,
    T.test_shared_minus_inf_term_excludes_key,
    T.test_attn_bruteforce,
    T.test_attn_closed_forms,
    T.test_attn_permutation_and_scale,
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {name}"
    bad_src = tmp_path / f"bad_{name}.c"
    bad_src.write_text(src.replace(old, new, 1))
    lib = oracle.load_library(oracle.compile_source(str(bad_src), str(tmp_path / f"bad_{name}.so")))
    bad = oracle.Oracle(lib)
    caught = []
    for pin in PINS:
        try:
            pin(bad)
        except (AssertionError, RuntimeError, ValueError) as e:  # a pin failed: mistake caught
            caught.append(type(e).__name__)
            break
    assert caught, f"no pin catches the planted mistake {name!r}"


def test_unmutated_copy_passes_all_pins(tmp_path):
    lib = oracle.load_library(oracle.compile_source(SRC, str(tmp_path / "good.so")))
    good = oracle.Oracle(lib)
    for pin in PINS:
        pin(good)
