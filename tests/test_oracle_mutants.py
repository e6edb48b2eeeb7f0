"""Planted mistakes in a private copy of the oracle must each fail at least one pin.

Each mutant is the oracle's C source with one plausible slip (a dropped term, a wrong
sign, an off-by-one index, a swapped operand), compiled with gcc into a temporary
library and swapped in for the real one while the pins in test_oracle_pins run against
it.  CPU only; the real oracle library is restored afterwards.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

MUTANTS = {
    "own_block_excludes_self": ("for (int64_t j = start; j <= p; ++j)", "for (int64_t j = start; j < p; ++j)"),
    "anchor_one_too_long": ("for (int64_t j = 0; j < anchor; ++j)", "for (int64_t j = 0; j <= anchor; ++j)"),
    "anchor_skips_block2": ("if (i >= 1)\n        for", "if (i >= 2)\n        for"),
    "missing_scale": ("xbuf[t] = c->scale * dot;", "xbuf[t] = dot;"),
    "no_max_subtraction": ("double w = exp(xbuf[t] - M);", "double w = exp(xbuf[t]);"),
    "gqa_interleaved": ("c.kv_off = (int64_t)(h / G) * J->L * J->d;", "c.kv_off = (int64_t)(h % J->hkv) * J->L * J->d;"),
    "merge_weight_sign": ("double w = l[idx] * exp(m[idx] - M);", "double w = l[idx] * exp(M - m[idx]);"),
    "causal_strict": ("(j - J->lo) <= J->causal_offset + i", "(j - J->lo) < J->causal_offset + i"),
    "lse_sign": ("J->lse[(int64_t)h * J->n_rows + r] = M + log(l);", "J->lse[(int64_t)h * J->n_rows + r] = M - log(l);"),
    "values_from_keys": ("out[e] += w * load_elem(c->v, c->dtype, c->kv_off + j * d + e);",
                         "out[e] += w * load_elem(c->k, c->dtype, c->kv_off + j * d + e);"),
    "merge_drops_l": ("double w = l[idx] * exp(m[idx] - M);", "double w = exp(m[idx] - M);"),
}

PIN_CALLS = [
    lambda o: pins.test_single_block_is_global_causal(o, "f32", 37),
    lambda o: pins.test_anchor_equal_block_first_two_blocks_global(o),
    lambda o: pins.test_no_anchor_is_block_diagonal(o),
    lambda o: [pins.test_zero_keys_closed_form(o, *c) for c in [(50, 16, 16), (50, 16, 5), (64, 16, 0)]],
    lambda o: pins.test_literal_augmentation_bruteforce(o, 14, 4, 2),
    lambda o: pins.test_merge_equals_dense_softmax(o, [0, 7, 19, 33, 34, 50, 61]),
    lambda o: pins.test_partial_is_local_softmax_and_sum(o),
    lambda o: pins.test_merge_no_overflow_at_large_scores(o),
    lambda o: pins.test_partial_causal_offset(o),
    lambda o: pins.test_phase2_equals_global_causal_rows(o, [0, 10, 20, 30, 40]),
    lambda o: pins.test_needle_peaked_softmax(o),
    lambda o: pins.test_gqa_contiguous_groups(o),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, "mutation site for %s not unique" % name
    path = tmp_path / ("mut_%s.c" % name)
    path.write_text(src.replace(old, new))
    so = tmp_path / ("mut_%s.so" % name)
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-std=c99", "-pthread", str(path),
                           "-o", str(so), "-lm"])
    return str(so)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, oracle_lib, name):
    old, new = MUTANTS[name]
    so = _build_mutant(tmp_path, name, old, new)
    real = oracle._load()
    mut = ctypes.CDLL(so)
    for fn in ("star_oracle_phase1", "star_oracle_partial", "star_oracle_merge"):
        getattr(mut, fn).argtypes = getattr(real, fn).argtypes
        getattr(mut, fn).restype = getattr(real, fn).restype
    caught = []
    oracle._lib = mut
    try:
        for i, call in enumerate(PIN_CALLS):
            try:
                call(oracle)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(i)
    finally:
        oracle._lib = real
    assert caught, "mutant %s passed every pin" % name
    os.remove(so)


# ---- the E4M3 context cache (oracle/kv_fp8.py): one slip each, in a private copy of the
# module, must fail at least one of the pins in test_oracle_fp8.
FP8_MUTANTS = {
    "ties_to_odd": ("np.where(lo % 2 == 0, lo, hi)", "np.where(lo % 2 == 1, lo, hi)"),
    "ties_up": ("np.where(lo % 2 == 0, lo, hi)", "hi"),
    "overflow_to_nan": ("pick = np.where(a >= E4M3_MAX, 0x7E, pick)", "pick = np.where(a > E4M3_MAX, 0x7F, pick)"),
    "bias_8": ("np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    "subnormal_exponent": ("(m / 8.0) * 2.0 ** -6", "(m / 8.0) * 2.0 ** -7"),
    "sign_dropped": ("code = np.where(np.isnan(x), 0x7F, pick) | sign", "code = np.where(np.isnan(x), 0x7F, pick)"),
    "v_takes_k_scale": ("vd = np.ascontiguousarray(kv_dequantize(v8, v_scale))",
                        "vd = np.ascontiguousarray(kv_dequantize(v8, k_scale))"),
    "query_tail_not_causal": ("parts.append(partial(q3, kt, vt, 0, int(tail_len), int(tail_len) - rows, scale, threads))",
                              "parts.append(partial(q3, kt, vt, 0, int(tail_len), -1, scale, threads))"),
    "query_tail_offset_off_by_one": ("int(tail_len) - rows, scale, threads))",
                                     "int(tail_len) - rows - 1, scale, threads))"),
    "partial_ignores_causal_offset": ("int(lo), int(hi), int(causal_offset), scale, threads)",
                                      "int(lo), int(hi), -1, scale, threads)"),
    "quantize_multiplies": ("qv = (v / s).astype(np.float32)", "qv = (v * s).astype(np.float32)"),
    "absmax_over_256": ("s = (amax.astype(np.float32) / np.float32(E4M3_MAX))",
                        "s = (amax.astype(np.float32) / np.float32(256.0))"),
}


def _fp8_pin_calls():
    from tests import test_oracle_fp8 as p8
    return p8, [p8.test_decode_matches_torch_float8_e4m3fn, p8.test_decode_format_values,
                p8.test_encode_matches_torch_inside_the_finite_range, p8.test_encode_ties_saturation_and_specials,
                p8.test_encode_round_trips_every_finite_code, p8.test_rounding_error_within_half_a_step,
                p8.test_absmax_scales_map_each_heads_largest_element_to_448,
                p8.test_kv8_decode_equals_plain_oracle_on_fp32_exact_values,
                lambda: p8.test_kv8_decode_against_dense_softmax(None),
                p8.test_kv8_query_equals_plain_oracle_on_fp32_exact_values,
                p8.test_kv8_query_rows_after_cached_tokens_against_dense_softmax,
                lambda: p8.test_kv8_partial_equals_plain_oracle_on_fp32_exact_values(3),
                p8.test_kv8_partial_against_brute_force]


def test_fp8_pins_pass_on_the_real_module():
    _, calls = _fp8_pin_calls()
    for c in calls:
        c()


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_mutant_is_caught(monkeypatch, name):
    import types
    from oracle import kv_fp8
    old, new = FP8_MUTANTS[name]
    src = open(kv_fp8.__file__).read()
    assert src.count(old) == 1, "mutation site for %s not unique" % name
    mod = types.ModuleType("oracle.kv_fp8_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "kv_fp8_mutant.py", "exec"), mod.__dict__)
    p8, calls = _fp8_pin_calls()
    monkeypatch.setattr(p8, "f8", mod)
    failed = 0
    for c in calls:
        try:
            c()
        except Exception:
            failed += 1
    assert failed > 0, "mutant %s passed every fp8 pin" % name
