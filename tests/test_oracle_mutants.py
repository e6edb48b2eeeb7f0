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
