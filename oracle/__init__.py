"""fp64 CPU oracle for Star Attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU product path never does, and
this package imports nothing from it.

The arithmetic lives in ``star_oracle.c`` (plain C, double precision); this
module only builds it, marshals numpy arrays into it and composes its three
primitives (phase-1 rows, one partition's local attention, the global
aggregation) into the two-phase procedure, in the order the pages give:

* "Star Attention: Efficient LLM Inference over Long Sequences"
  (paper-graph-ui summary of arXiv 2411.17116), section 3.4, Phase 1 Steps
  1-5 and Phase 2 Steps 1-7;
* "NVIDIA/Star-Attention" README (shadowgraph.io mirror), section
  "Two Phases of Star Attention".

bf16 tensors are passed as their uint16 bit patterns; fp32 as float32; float64
arrays (a dequantised fp8 cache, see ``kv_fp8``) as float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "star_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libstar_oracle.so")
_lib = None
_lock = threading.Lock()

F32, BF16, F64 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile star_oracle.c with gcc into oracle/libstar_oracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fPIC", "-shared", "-std=c99", "-pthread", "-fno-fast-math",
             "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
            p, i64, i32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
            lib.star_oracle_phase1.argtypes = [p, p, p, i32, i64, i64, i64, i32, i32, i32, f64,
                                               p, i64, i32, p, p, i32]
            lib.star_oracle_phase1.restype = i32
            lib.star_oracle_partial.argtypes = [p, i64, p, p, i32, i64, i64, i64, i64,
                                                i32, i32, i32, f64, p, p, p, i32]
            lib.star_oracle_partial.restype = i32
            lib.star_oracle_merge.argtypes = [p, p, p, i32, i64, i32, p, p]
            lib.star_oracle_merge.restype = None
            _lib = lib
    return _lib


def default_threads() -> int:
    """Host threads for the oracle: the cores present, at most 16 (one GPU's share of a host)."""
    return max(1, min(os.cpu_count() or 1, 16))


def _as_input(x):
    """numpy (float32 / uint16 bf16 bits) or torch CPU tensor -> (contiguous array, dtype code)."""
    if hasattr(x, "detach"):  # torch tensor; no torch import needed here
        name = str(x.dtype)
        x = x.detach().cpu().contiguous()
        if name == "torch.bfloat16":
            import torch  # only reached when the caller already holds a torch tensor
            return np.ascontiguousarray(x.view(torch.int16).numpy().view(np.uint16)), BF16
        if name == "torch.float32":
            return np.ascontiguousarray(x.numpy()), F32
        raise TypeError("oracle inputs must be bf16 or fp32, got %s" % name)
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, BF16
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.float64:
        return x, F64
    raise TypeError("oracle inputs must be float32, float64 or uint16 (bf16 bits), got %s" % x.dtype)


def widen(x) -> np.ndarray:
    """The exact values of an oracle input (bf16 bits, fp32 or fp64) as float64."""
    a, dt = _as_input(x)
    if dt == BF16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def phase1(q, k, v, block: int, anchor: int, rows=None, q_sampled: bool = False,
           scale: float | None = None, threads: int | None = None):
    """Phase-1 outputs (O, LSE) in fp64.

    q: [Hq, L, d] (or [Hq, len(rows), d] with q_sampled=True); k, v: [Hkv, L, d].
    rows: context positions to evaluate (default: all).  Returns
    o [Hq, n_rows, d] float64 and lse [Hq, n_rows] float64 (natural log).
    """
    q, dq = _as_input(q)
    k, dk = _as_input(k)
    v, dv = _as_input(v)
    assert dq == dk == dv, "q, k, v must share a dtype"
    hkv, L, d = k.shape
    hq = q.shape[0]
    if rows is None:
        rows = np.arange(L, dtype=np.int64)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if q_sampled:
        assert q.shape[1] == rows.size
    else:
        assert q.shape[1] == L
    scale = float(1.0 / np.sqrt(d)) if scale is None else float(scale)
    o = np.zeros((hq, rows.size, d), dtype=np.float64)
    lse = np.zeros((hq, rows.size), dtype=np.float64)
    rc = _load().star_oracle_phase1(_ptr(q), _ptr(k), _ptr(v), dq, L, block, anchor, hq, hkv, d,
                                    scale, _ptr(rows), rows.size, int(q_sampled), _ptr(o), _ptr(lse),
                                    threads or default_threads())
    if rc != 0:
        raise ValueError("star_oracle_phase1: invalid arguments")
    return o, lse


def partial(q, k, v, lo: int, hi: int, causal_offset: int = -1, scale: float | None = None,
            threads: int | None = None):
    """Local attention of q [Hq, rows, d] over tokens [lo, hi) of k/v [Hkv, T, d].

    Returns (A [Hq, rows, d], m [Hq, rows], l [Hq, rows]) in fp64, A normalised over the
    partition, s = e^m * l.  causal_offset >= 0 lets row i see partition token t only if
    t <= causal_offset + i.
    """
    q, dq = _as_input(q)
    k, dk = _as_input(k)
    v, dv = _as_input(v)
    assert dq == dk == dv
    hkv, T, d = k.shape
    hq, rows, _ = q.shape
    scale = float(1.0 / np.sqrt(d)) if scale is None else float(scale)
    a = np.zeros((hq, rows, d), dtype=np.float64)
    m = np.zeros((hq, rows), dtype=np.float64)
    l = np.zeros((hq, rows), dtype=np.float64)
    rc = _load().star_oracle_partial(_ptr(q), rows, _ptr(k), _ptr(v), dq, T, lo, hi, causal_offset,
                                     hq, hkv, d, scale, _ptr(a), _ptr(m), _ptr(l),
                                     threads or default_threads())
    if rc != 0:
        raise ValueError("star_oracle_partial: invalid arguments")
    return a, m, l


def merge(a, m, l):
    """Aggregate partitions: a [P, ..., d], m and l [P, ...] -> (O [..., d], LSE [...])."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    P = a.shape[0]
    lead = a.shape[1:-1]
    d = a.shape[-1]
    n = int(np.prod(lead)) if lead else 1
    o = np.zeros(lead + (d,), dtype=np.float64)
    lse = np.zeros(lead, dtype=np.float64)
    _load().star_oracle_merge(_ptr(a), _ptr(m), _ptr(l), P, n, d, _ptr(o), _ptr(lse))
    return o, lse


def phase2_query(q_qry, k_ctx, v_ctx, shard_bounds, k_tail, v_tail, scale=None, threads=None):
    """Query encoding (Phase 2, Steps 2-5): one partial per context shard plus the
    query host's own partial over its cache (causal among the query tokens), merged.

    q_qry [Hq, lq, d]; k_ctx/v_ctx [Hkv, L, d]; shard_bounds: S+1 increasing token
    offsets covering [0, L); k_tail/v_tail [Hkv, >=lq, d] hold the query tokens' K/V.
    Returns (O [Hq, lq, d], LSE [Hq, lq]).
    """
    parts = [partial(q_qry, k_ctx, v_ctx, int(lo), int(hi), -1, scale, threads)
             for lo, hi in zip(shard_bounds[:-1], shard_bounds[1:])]
    lq = _as_input(q_qry)[0].shape[1]
    parts.append(partial(q_qry, k_tail, v_tail, 0, lq, 0, scale, threads))
    return merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]),
                 np.stack([p[2] for p in parts]))


def phase2_decode(q_t, k_ctx, v_ctx, shard_bounds, k_tail, v_tail, tail_len, scale=None,
                  threads=None):
    """One generated token (Phase 2, Steps 3-5 and 7): q_t [Hq, d] attends to every context
    shard and to the query host's cache k_tail/v_tail [Hkv, >=tail_len, d], which already
    holds the new token's own k/v at index tail_len - 1.  Returns (O [Hq, d], LSE [Hq])."""
    q3, _ = _as_input(q_t)
    q3 = q3.reshape(q3.shape[0], 1, q3.shape[1])
    parts = [partial(q3, k_ctx, v_ctx, int(lo), int(hi), -1, scale, threads)
             for lo, hi in zip(shard_bounds[:-1], shard_bounds[1:])]
    parts.append(partial(q3, k_tail, v_tail, 0, int(tail_len), -1, scale, threads))
    o, lse = merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]),
                   np.stack([p[2] for p in parts]))
    return o[:, 0, :], lse[:, 0]
