"""Seeded random sweep of shapes for every entry point, each case against the oracle.

The cases are drawn once from a fixed seed (so a failure names a reproducible case): random
GQA group sizes, head dims (the MFMA path at 64 and 128, the vector path at 96), context
lengths, block and anchor sizes (anchor from 0 to block, blocks longer than the context),
shard splits with empty shards, numbers of cached query tokens and decode steps, and bf16 or
E4M3 context caches.  Sizes stay small enough for the fp64 oracle to finish in seconds.  A
second draw from another seed repeats the mix with contexts three to four times longer.
"""
import random

import numpy as np
import pytest
import torch

import block_sparse_long_phase1_amd as sa
import oracle
from oracle import kv_fp8 as of8
from block_sparse_long_phase1_amd import inputs as sin
from block_sparse_long_phase1_amd.configs import StarConfig
from tests._parity import assert_lse, assert_out, flush_print

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
_RNG = random.Random(20241203)


def _bounds(rng, L, S):
    cuts = sorted(rng.randint(0, L) for _ in range(S - 1))
    return [0] + cuts + [L]


def _phase1_cases(n, rng=_RNG, max_len=2000):
    out = []
    for _ in range(n):
        hkv = rng.choice([1, 2, 4])
        G = rng.choice([1, 2, 4, 8, 16])
        d = rng.choice([64, 128, 128, 96])
        L = rng.randint(1, max_len if hkv * G <= 8 else max_len * 9 // 20)
        block = rng.randint(1, L + 100)
        anchor = rng.randint(0, block)
        out.append((hkv * G, hkv, L, block, anchor, d))
    return out


def _decode_cases(n, rng=_RNG, max_len=5000):
    out = []
    for _ in range(n):
        hkv = rng.choice([1, 2, 4])
        G = rng.choice([1, 2, 4, 8, 16])
        kv8 = rng.random() < 0.5
        d = rng.choice([64, 128] if kv8 else [64, 128, 96])
        L = rng.randint(1, max_len)
        S = rng.randint(1, 6)
        lq = rng.randint(0, 60)
        T = rng.randint(1, 3)
        out.append((hkv * G, hkv, L, _bounds(rng, L, S), lq, T, d, kv8))
    return out


def _query_cases(n, rng=_RNG, max_len=4000):
    out = []
    for _ in range(n):
        hkv = rng.choice([1, 2, 4])
        G = rng.choice([1, 2, 4, 8])
        d = rng.choice([64, 128])
        L = rng.randint(1, max_len)
        S = rng.randint(1, 5)
        tail_len = rng.randint(1, 300)
        rows = rng.randint(1, tail_len)
        out.append((hkv * G, hkv, L, _bounds(rng, L, S), rows, tail_len, d))
    return out


PHASE1 = _phase1_cases(14)
DECODE = _decode_cases(12)
QUERY = _query_cases(8)
# A second draw from a generator of its own, with contexts up to three or four times longer
# (more tiles and key splits per case); the lists above stay as drawn.
_RNG_MORE = random.Random(20261204)
PHASE1 += _phase1_cases(14, _RNG_MORE, max_len=6000)
DECODE += _decode_cases(12, _RNG_MORE, max_len=20000)
QUERY += _query_cases(8, _RNG_MORE, max_len=12000)


def _query_kv8_cases(n):
    """E4M3 context query cases from a generator of their own (the lists above stay as drawn)."""
    rng = random.Random(20241204)
    out = []
    for _ in range(n):
        hkv = rng.choice([1, 2, 4])
        G = rng.choice([1, 2, 4, 8, 16])
        d = rng.choice([64, 128])
        L = rng.randint(1, 4000)
        S = rng.randint(1, 5)
        tail_len = rng.randint(1, 300)
        rows = rng.randint(1, tail_len)
        out.append((hkv * G, hkv, L, _bounds(rng, L, S), rows, tail_len, d))
    return out


QUERY8 = _query_kv8_cases(8)


def _cfg(hq, hkv, L, d, lq=4, T=1, seed=1):
    return StarConfig("sweep", hq=hq, hkv=hkv, d=d, L=L, block=L, anchor=L, lq=max(lq, 1), decode_steps=T,
                      shards=1, dtype="bf16", needle=False, seed=seed)


@pytest.mark.parametrize("i", range(len(PHASE1)), ids=[str(c) for c in PHASE1])
def test_sweep_phase1(i):
    case = PHASE1[i]
    hq, hkv, L, block, anchor, d = case
    flush_print("sweep phase1", case)
    cfg = _cfg(hq, hkv, L, d, seed=300 + i)
    q, k, v = sin.phase1_inputs(cfg, DEV)
    o, lse = sa.star_phase1_encode(q, k, v, block, anchor)
    torch.cuda.synchronize()
    ro, rl = oracle.phase1(q.cpu(), k.cpu(), v.cpu(), block, anchor)
    assert_out(o, ro, "O %s" % (case,))
    assert_lse(lse, rl, "LSE %s" % (case,))


@pytest.mark.parametrize("i", range(len(QUERY)), ids=[str(c) for c in QUERY])
def test_sweep_query(i):
    case = QUERY[i]
    hq, hkv, L, bounds, rows, tail_len, d = case
    flush_print("sweep query", case)
    cfg = _cfg(hq, hkv, L, d, lq=tail_len, seed=400 + i)
    _, k, v = sin.phase1_inputs(cfg, DEV)
    p2 = sin.phase2_inputs(cfg, DEV)
    qr = p2["q_qry"][:, tail_len - rows:].contiguous()
    kt = torch.zeros((hkv, tail_len + 3, d), dtype=torch.bfloat16, device=DEV)
    vt = torch.zeros_like(kt)
    kt[:, :tail_len] = p2["k_qry"]
    vt[:, :tail_len] = p2["v_qry"]
    o, lse = sa.star_phase2_query(qr, k, v, bounds, kt, vt, tail_len)
    torch.cuda.synchronize()
    qc, kc, vc = qr.cpu(), k.cpu(), v.cpu()
    parts = [oracle.partial(qc, kc, vc, lo, hi) for lo, hi in zip(bounds[:-1], bounds[1:])]
    parts.append(oracle.partial(qc, kt.cpu(), vt.cpu(), 0, tail_len, tail_len - rows))
    ro, rl = oracle.merge(np.stack([x[0] for x in parts]), np.stack([x[1] for x in parts]),
                          np.stack([x[2] for x in parts]))
    assert_out(o, ro, "O %s" % (case,))
    assert_lse(lse, rl, "LSE %s" % (case,))


@pytest.mark.parametrize("i", range(len(QUERY8)), ids=[str(c) for c in QUERY8])
def test_sweep_query_kv8(i):
    case = QUERY8[i]
    hq, hkv, L, bounds, rows, tail_len, d = case
    flush_print("sweep query kv8", case)
    cfg = _cfg(hq, hkv, L, d, lq=tail_len, seed=600 + i)
    _, k, v = sin.phase1_inputs(cfg, DEV)
    p2 = sin.phase2_inputs(cfg, DEV)
    qr = p2["q_qry"][:, tail_len - rows:].contiguous()
    kt = torch.zeros((hkv, tail_len + 3, d), dtype=torch.bfloat16, device=DEV)
    vt = torch.zeros_like(kt)
    kt[:, :tail_len] = p2["k_qry"]
    vt[:, :tail_len] = p2["v_qry"]
    ks, vs = of8.kv_absmax_scales(k.cpu()), of8.kv_absmax_scales(v.cpu())
    hk8, hv8 = of8.kv_quantize(k.cpu(), ks), of8.kv_quantize(v.cpu(), vs)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    o, lse = sa.star_phase2_query_kv8(qr, to(hk8), to(hv8), to(ks), to(vs), bounds, kt, vt, tail_len)
    torch.cuda.synchronize()
    ro, rl = of8.phase2_query_kv8(qr.cpu(), hk8, hv8, ks, vs, bounds, kt.cpu(), vt.cpu(), tail_len)
    assert_out(o, ro, "O %s" % (case,))
    assert_lse(lse, rl, "LSE %s" % (case,))


@pytest.mark.parametrize("i", range(len(DECODE)), ids=[str(c) for c in DECODE])
def test_sweep_decode(i):
    case = DECODE[i]
    hq, hkv, L, bounds, lq, T, d, kv8 = case
    flush_print("sweep decode", case)
    cfg = _cfg(hq, hkv, L, d, lq=lq, T=T, seed=500 + i)
    _, k, v = sin.phase1_inputs(cfg, DEV)
    p2 = sin.phase2_inputs(cfg, DEV)
    kt = torch.zeros((hkv, lq + T, d), dtype=torch.bfloat16, device=DEV)
    vt = torch.zeros_like(kt)
    kt[:, :lq] = p2["k_qry"][:, :lq]
    vt[:, :lq] = p2["v_qry"][:, :lq]
    ws = sa.decode_workspace(L, lq + T, len(bounds) - 1, hq, hkv, d, DEV)
    if kv8:
        ks, vs = of8.kv_absmax_scales(k.cpu()), of8.kv_absmax_scales(v.cpu())
        hk8, hv8 = of8.kv_quantize(k.cpu(), ks), of8.kv_quantize(v.cpu(), vs)
        k8, v8 = torch.from_numpy(hk8).to(DEV), torch.from_numpy(hv8).to(DEV)
        dks, dvs = torch.from_numpy(ks).to(DEV), torch.from_numpy(vs).to(DEV)
    for t in range(T):
        if kv8:
            o, lse = sa.star_decode_step_kv8(p2["q_dec"][t], p2["k_dec"][t], p2["v_dec"][t], k8, v8, dks, dvs, bounds,
                                             kt, vt, lq + t, workspace=ws)
        else:
            o, lse = sa.star_decode_step(p2["q_dec"][t], p2["k_dec"][t], p2["v_dec"][t], k, v, bounds, kt, vt, lq + t,
                                         workspace=ws)
        torch.cuda.synchronize()
        if kv8:
            ro, rl = of8.phase2_decode_kv8(p2["q_dec"][t].cpu(), hk8, hv8, ks, vs, bounds, kt.cpu(), vt.cpu(), lq + t + 1)
        else:
            ro, rl = oracle.phase2_decode(p2["q_dec"][t].cpu(), k.cpu(), v.cpu(), bounds, kt.cpu(), vt.cpu(), lq + t + 1)
        assert_out(o, ro, "O %s step %d" % (case, t))
        assert_lse(lse, rl, "LSE %s step %d" % (case, t))
