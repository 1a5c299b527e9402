"""Planted-mistake checks for the oracle's pins (CPU only).

Each case copies the oracle source, plants one plausible mistake (a dropped
term, a wrong sign or index, a swapped operand or table), compiles the copy
into a temporary library and runs the pins against it: at least one pin must
fail.  The product oracle is never modified.
"""
import os
import shutil
import tempfile

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "sdpa_oracle.c")

# (name, original text, planted text)
MUTATIONS = [
    ("gqa_head_mapping_mod", "int32_t kvh = h / (c->hq / c->hkv);\n    /* visible",
     "int32_t kvh = h % c->hkv;\n    /* visible"),
    ("causal_top_left", "const int64_t diag = i + lk - lq;", "const int64_t diag = i;"),
    ("causal_off_by_one", "if (c->causal && diag + 1 < j1) j1 = diag + 1;",
     "if (c->causal && diag < j1) j1 = diag;"),
    ("lse_base_two", "*lse = m + log(l);", "*lse = m + log2(l);"),
    ("scale_dropped", "s[j] = scale * dot;", "s[j] = dot;"),
    ("exp_sign", "s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    ("normalizer_dropped", "for (int d = 0; d < dv; ++d) o[d] /= l;", ""),
    ("k_strides_swapped", "koff[j] = (c->cu_kv[b] + j0 + j) * c->k_st + (int64_t)kvh * c->k_sh;",
     "koff[j] = (c->cu_kv[b] + j0 + j) * c->k_sh + (int64_t)kvh * c->k_st;"),
    ("window_one_too_wide", "if (c->window > 0 && diag - c->window + 1 > j0) j0 = diag - c->window + 1;",
     "if (c->window > 0 && diag - c->window > j0) j0 = diag - c->window;"),
    ("window_ignored", "if (c->window > 0 && diag - c->window + 1 > j0) j0 = diag - c->window + 1;",
     ""),
    ("window_keys_not_shifted", "koff[j] = (c->cu_kv[b] + j0 + j) * c->k_st",
     "koff[j] = (c->cu_kv[b] + j) * c->k_st"),
    ("sink_dropped_from_denominator", "double l = sink == -INFINITY ? 0.0 : exp(sink - m);",
     "double l = 0.0;"),
    ("sink_row_without_keys_empty", "if (n == 0 && sink == -INFINITY) {", "if (n == 0) {"),
    ("v_uses_k_table", "int64_t vpage = c->pt_v[", "int64_t vpage = c->pt_k["),
    ("merge_weight_uses_max", "double w = exp(ll[sp] - L_all);",
     "double w = exp(ll[sp] - m_all);"),
    ("decode_causal_position", "const int64_t pos = L - c->sq + tq;",
     "const int64_t pos = L - 1 - tq;"),
    ("decode_window_off_by_one", "if (c->window > 0 && pos - c->window + 1 > first) first = pos - c->window + 1;",
     "if (c->window > 0 && pos - c->window > first) first = pos - c->window;"),
    ("decode_window_ignored", "if (c->window > 0 && pos - c->window + 1 > first)",
     "if (0 && pos - c->window + 1 > first)"),
    ("decode_sink_in_every_split", "c->scale, S == 1 ? sink : -INFINITY, s,", "c->scale, sink, s,"),
    ("decode_sink_dropped_from_merge", "if (sink != -INFINITY) w_sum += exp(sink - m_all);",
     "if (0) w_sum += exp(sink - m_all);"),
    ("combine_lse_dropped_log", "double L = m + log(w_sum);", "double L = m + w_sum;"),
    ("e4m3_bias_off_by_one", "ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)"),
    ("e4m3_subnormal_as_normal", "e == 0 ? ldexp((double)m / 8.0, -6)",
     "e == 0 ? ldexp(1.0 + (double)m / 8.0, -7)"),
    ("e4m3_nan_code_wrong", "if (e == 15 && m == 7) return NAN;", "if (e == 15) return NAN;"),
    ("descale_v_dropped", "o[d] += s[j] * (vscale * load_elem", "o[d] += s[j] * (1.0 * load_elem"),
    ("descales_k_v_swapped", "c->dk, c->dv_scale,", "c->dv_scale, c->dk,"),
    ("descale_q_dropped", "qrow[d] = c->dq * load_elem", "qrow[d] = load_elem"),
    ("prefill_descale_q_dropped", "qrow[d] = c->q_descale * load_elem", "qrow[d] = load_elem"),
    ("prefill_descales_k_v_swapped", "c->k_descale,\n               c->v_descale,",
     "c->v_descale,\n               c->k_descale,"),
]


def _pin_suite():
    """Pins run against a variant; returns the names of the pins that failed."""
    checks = [
        ("brute_gqa", lambda: pins.test_brute_force_vs_torch(8, 2, 128, 128, True,
                                                             pins.torch.bfloat16)),
        ("brute_mla", lambda: pins.test_brute_force_vs_torch(16, 1, 576, 512, True,
                                                             pins.torch.float32)),
        ("natural_log", pins.test_lse_is_natural_log),
        ("rows_sum_to_one", pins.test_softmax_rows_sum_to_one),
        ("causal_bitwise", pins.test_causal_rows_ignore_future_keys_bitwise),
        ("scale_zero", pins.test_closed_form_scale_zero),
        ("first_row", pins.test_closed_form_first_causal_row),
        ("golden", pins.test_golden_hand_examples),
        ("empty_rows", pins.test_empty_and_degenerate_rows),
        ("paged_dense", lambda: pins.test_paged_equals_gathered_dense_bitwise(
            (4, 2, 8, 2, 64, 64, 16))),
        ("split_merge", lambda: pins.test_split_merge_equals_unsplit(3)),
        ("combine_closed", pins.test_combine_closed_forms),
        ("decode_causal", pins.test_decode_causal_two_tokens),
        ("window_brute", lambda: pins.test_window_and_sinks_brute_force_vs_torch(3, True, False)),
        ("window_one", pins.test_window_one_sees_only_the_diagonal_key),
        ("sink_brute", lambda: pins.test_window_and_sinks_brute_force_vs_torch(40, False, True)),
        ("sink_closed", pins.test_sink_closed_form_single_key),
        ("sink_empty_rows", pins.test_rows_without_keys_take_the_sink_as_lse),
        ("decode_window_brute", lambda: pins.test_decode_window_and_sinks_brute_force_vs_torch(
            5, 3, False, True)),
        ("decode_sink_brute", lambda: pins.test_decode_window_and_sinks_brute_force_vs_torch(
            0, 3, True, False)),
        ("decode_window_one", pins.test_decode_window_one_sees_only_its_own_key),
        ("decode_sink_empty", pins.test_decode_rows_without_keys_take_the_sink),
        ("e4m3_codes", pins.test_e4m3_values_match_torch_float8_e4m3fn),
        ("fp8_brute", lambda: pins.test_fp8_decode_brute_force_vs_torch(3, 2)),
        ("fp8_single_key", pins.test_fp8_single_key_closed_form),
        ("fp8_prefill_brute", lambda: pins.test_fp8_prefill_brute_force_vs_torch(5, True, True)),
    ]
    failed = []
    for name, fn in checks:
        try:
            fn()
        except Exception:  # an assertion, or the oracle rejecting / crashing
            failed.append(name)
    return failed


def test_unmutated_oracle_passes_every_pin():
    assert _pin_suite() == []


@pytest.mark.parametrize("name,orig,planted", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, orig, planted):
    text = open(SRC).read()
    assert text.count(orig) == 1, "mutation anchor for %s not unique in the oracle" % name
    tmp = tempfile.mkdtemp(prefix="oracle_mut_")
    try:
        src = os.path.join(tmp, "mut.c")
        with open(src, "w") as f:
            f.write(text.replace(orig, planted))
        lib = oracle.compile_source(src, os.path.join(tmp, "libmut.so"))
        with oracle.variant(lib):
            failed = _pin_suite()
        assert failed, "planted mistake %s passed every pin" % name
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
