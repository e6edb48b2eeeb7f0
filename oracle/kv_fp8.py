"""fp8 (E4M3) context KV cache for the oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the GPU product path never does.

What the pages fix.  "Star Attention: Efficient LLM Inference over Long
Sequences" (paper-graph-ui summary), section "Related Work", part "Memory
Optimization and KV Cache Compression": KV-cache quantisation is orthogonal to
the method and can be combined with it.  No format, granularity or placement is
given there, so the following reading is taken:

* the context hosts hold their cached K and V as E4M3 codes, with one fp32
  scale per kv head for K and one for V; the query host's own (small, growing)
  cache stays in the compute dtype;
* quantisation: code = E4M3 rounding (nearest, ties to even, saturating at
  +-448) of the fp32 quotient x / scale, with x widened exactly to fp32 and the
  quotient correctly rounded;
* dequantisation: value = scale * decode(code), exact in float64;
* default scale of a kv head: its largest |x| divided by 448 in fp32 (1 when
  the head is all zeros), so the largest element maps to +-448;
* the query phase and a decode step over a quantised context are the plain
  Phase-2 query phase (section 3.4, Phase 2 Steps 1-5) and decode step (Steps
  3-5 and 7) over the dequantised values.

The E4M3 format itself is the OCP 8-bit floating point specification's: one
sign bit, four exponent bits with bias 7, three mantissa bits; exponent field 0
holds subnormals m/8 * 2^-6; S.1111.111 is NaN; there are no infinities and the
largest finite magnitude is 448.
"""
from __future__ import annotations

import numpy as np

from . import _as_input, merge, partial, widen

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8) as float64; NaN for the two NaN codes."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where(sign == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


# Non-negative finite magnitudes in code order: code c in [0, 0x7E] has value _MAGS[c],
# strictly increasing, so a code's neighbours in value are its neighbours in number.
_MAGS = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(x) -> np.ndarray:
    """Round fp32 values to E4M3 codes: nearest representable value, a tie going to the
    even code (mantissa bit 0), magnitudes at or beyond 448 (infinities included) to
    +-448, NaN to the NaN code of its sign.  The sign bit is kept, so -0.0 and negative
    values that round to zero give the code 0x80."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    sign = np.signbit(x).astype(np.int64) << 7
    hi = np.clip(np.searchsorted(_MAGS, np.where(np.isnan(a), 0.0, a), side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - _MAGS[lo]
    d_hi = _MAGS[hi] - a
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a >= E4M3_MAX, 0x7E, pick)
    code = np.where(np.isnan(x), 0x7F, pick) | sign
    return code.astype(np.uint8)


def kv_absmax_scales(x) -> np.ndarray:
    """Per-kv-head scale of x [Hkv, n, d] (bf16 bits, fp32 or a torch tensor): max |x| / 448
    in fp32, or 1 for a head whose elements are all zero."""
    v = widen(x).astype(np.float32)   # exact: every input value is an fp32 number
    hkv = v.shape[0]
    amax = np.abs(v.reshape(hkv, -1)).max(axis=1) if v.size else np.zeros(hkv, np.float32)
    s = (amax.astype(np.float32) / np.float32(E4M3_MAX)).astype(np.float32)
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def kv_quantize(x, scale) -> np.ndarray:
    """E4M3 codes [Hkv, n, d] of x [Hkv, n, d] with per-head fp32 scales [Hkv]."""
    v = widen(x).astype(np.float32)
    s = np.asarray(scale, dtype=np.float32).reshape(-1, *([1] * (v.ndim - 1)))
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        qv = (v / s).astype(np.float32)   # one correctly rounded fp32 division per element
    return e4m3_encode(qv)


def kv_dequantize(codes, scale) -> np.ndarray:
    """scale[g] * decode(codes[g]) in float64 (exact: a 4-bit significand times an fp32)."""
    c = np.asarray(codes, dtype=np.uint8)
    s = np.asarray(scale, dtype=np.float32).astype(np.float64).reshape(-1, *([1] * (c.ndim - 1)))
    return s * e4m3_decode(c)


def _dequantized_cache(k8, v8, k_scale, v_scale):
    """The context cache's values: K with the K scales, V with the V scales (float64)."""
    kd = np.ascontiguousarray(kv_dequantize(k8, k_scale))
    vd = np.ascontiguousarray(kv_dequantize(v8, v_scale))
    return kd, vd


def partial_kv8(q, k8, v8, k_scale, v_scale, lo, hi, causal_offset=-1, scale=None, threads=None):
    """The local (A, m, l) of q [Hq, rows, d] over tokens [lo, hi) of an E4M3 cache k8/v8
    [Hkv, T, d] with per-kv-head scales: the plain partial (section 3.4, Phase 2 Step 3) over
    the dequantised values, with the same optional causal offset."""
    kd, vd = _dequantized_cache(k8, v8, k_scale, v_scale)
    return partial(np.ascontiguousarray(widen(q)), kd, vd, int(lo), int(hi), int(causal_offset), scale, threads)


def phase2_decode_kv8(q_t, k8, v8, k_scale, v_scale, shard_bounds, k_tail, v_tail, tail_len,
                      scale=None, threads=None):
    """One generated token over an E4M3 context cache: q_t [Hq, d] attends to every context
    shard of the dequantised k8/v8 [Hkv, L, d] and to the query host's cache
    k_tail/v_tail [Hkv, >=tail_len, d] (compute dtype), which already holds the new
    token's own k/v at index tail_len - 1.  Returns (O [Hq, d], LSE [Hq]) in float64."""
    kd, vd = _dequantized_cache(k8, v8, k_scale, v_scale)
    q3 = np.ascontiguousarray(widen(q_t)[:, None, :])
    kt = np.ascontiguousarray(widen(k_tail))
    vt = np.ascontiguousarray(widen(v_tail))
    assert _as_input(kd)[1] == _as_input(q3)[1] == _as_input(kt)[1]
    parts = [partial(q3, kd, vd, int(lo), int(hi), -1, scale, threads)
             for lo, hi in zip(shard_bounds[:-1], shard_bounds[1:])]
    parts.append(partial(q3, kt, vt, 0, int(tail_len), -1, scale, threads))
    o, lse = merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]),
                   np.stack([p[2] for p in parts]))
    return o[:, 0, :], lse[:, 0]


def phase2_query_kv8(q_qry, k8, v8, k_scale, v_scale, shard_bounds, k_tail, v_tail, tail_len,
                     scale=None, threads=None):
    """Query encoding over an E4M3 context cache: the rows of q_qry [Hq, rows, d] are the last
    rows of the query host's cache k_tail/v_tail [Hkv, >=tail_len, d] (compute dtype), so
    row i sees cache positions [0, tail_len - rows + i] causally, and every token of every
    context shard of the dequantised k8/v8 [Hkv, L, d].  One partial per context shard plus
    the query host's own partial, merged.  Returns (O [Hq, rows, d], LSE [Hq, rows])."""
    kd, vd = _dequantized_cache(k8, v8, k_scale, v_scale)
    q3 = np.ascontiguousarray(widen(q_qry))
    kt = np.ascontiguousarray(widen(k_tail))
    vt = np.ascontiguousarray(widen(v_tail))
    rows = q3.shape[1]
    assert _as_input(kd)[1] == _as_input(q3)[1] == _as_input(kt)[1]
    assert rows <= int(tail_len) <= kt.shape[1]
    parts = [partial(q3, kd, vd, int(lo), int(hi), -1, scale, threads)
             for lo, hi in zip(shard_bounds[:-1], shard_bounds[1:])]
    parts.append(partial(q3, kt, vt, 0, int(tail_len), int(tail_len) - rows, scale, threads))
    return merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]),
                 np.stack([p[2] for p in parts]))
