"""Comparison helpers for GPU-vs-oracle parity (test helpers only).

Tolerances for bf16 inputs with fp32 accumulation: max-abs <= 2e-2 and mean-abs <= 2e-3 on
outputs, and relative error <= 1e-5 on log-sum-exps with denominator max(|LSE|, 1).
"""
import numpy as np
import torch

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
LSE_REL = 1e-5


def to_np(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_out(got, ref, what, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    g = to_np(got)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), "%s: non-finite output" % what
    err = np.abs(g - ref)
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= max_abs and mean <= mean_abs, "%s: max-abs %.3g mean-abs %.3g" % (what, mx, mean)
    return mx, mean


def assert_lse(got, ref, what, rel=LSE_REL):
    g = to_np(got)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    neg = np.isneginf(ref)
    assert np.array_equal(np.isneginf(g), neg), "%s: -inf pattern differs" % what
    r = np.abs(g[~neg] - ref[~neg]) / np.maximum(np.abs(ref[~neg]), 1.0)
    worst = float(r.max()) if r.size else 0.0
    assert worst <= rel, "%s: LSE relative error %.3g" % (what, worst)
    return worst


def flush_print(*args):
    print(*args, flush=True)
