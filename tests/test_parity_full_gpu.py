"""Full-size parity at every workload, in the launch configuration bench.py times.

Phase 1 runs over the whole context; the oracle recomputes a seeded sample of rows (block
edges, key-tile edges, the middle and random rows, all q heads each).  The query phase runs
as the benchmark runs it (star_phase2_query, every partition in one call) and also as S+1
separate partial calls plus a merge; the oracle recomputes sampled query rows of both.  Every
decode step runs; the oracle recomputes every step at 8b_32k and, at the larger workloads,
every eighth step plus the middle and the last one.  Outputs must also be finite everywhere.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_phase1_amd as sa
import oracle
from block_sparse_long_phase1_amd import inputs as sin
from block_sparse_long_phase1_amd.configs import CONFIGS, StarConfig
from tests._parity import assert_lse, assert_out, flush_print

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def sample_rows(cfg, per_block_random=3):
    rng = np.random.default_rng(cfg.seed)
    rows = set()
    for i in range(cfg.n_blocks):
        lo, hi = i * cfg.block, min(cfg.L, (i + 1) * cfg.block)
        for off in (0, 1, 31, 32, 63, 64, 255, 256):
            if lo + off < hi:
                rows.add(lo + off)
        rows.update({(lo + hi) // 2, hi - 2, hi - 1})
        rows.update(int(r) for r in rng.integers(lo, hi, per_block_random))
    return np.array(sorted(r for r in rows if 0 <= r < cfg.L), dtype=np.int64)


def _query_phase(cfg, x, bounds, k_tail, v_tail):
    S = len(bounds) - 1
    q = x["q_qry"]
    pa = torch.empty((S + 1, cfg.hq, cfg.lq, cfg.d), dtype=torch.float32, device=DEV)
    pm = torch.empty((S + 1, cfg.hq, cfg.lq), dtype=torch.float32, device=DEV)
    pl = torch.empty_like(pm)
    for r, (lo, hi) in enumerate(zip(bounds[:-1], bounds[1:])):
        sa.star_phase2_partial(q, x["k_ctx"][:, lo:], x["v_ctx"][:, lo:], cfg.L * cfg.d, hi - lo, -1,
                               a_out=pa[r], m_out=pm[r], l_out=pl[r])
    sa.star_phase2_partial(q, k_tail, v_tail, cfg.tail_cap * cfg.d, cfg.lq, 0, a_out=pa[S], m_out=pm[S], l_out=pl[S])
    return sa.star_softmax_merge(pa, pm, pl, out_dtype=q.dtype)


@pytest.mark.timeout(400)
@pytest.mark.parametrize("name", ["8b_32k", "8b_128k_needle", "70b_128k", "8b_1m"])
def test_full_workload(name):
    cfg = CONFIGS[name]
    flush_print("full workload", name)
    x = sin.all_inputs(cfg, DEV)
    q, k, v = x["q_ctx"], x["k_ctx"], x["v_ctx"]
    bounds = cfg.bounds()

    # ---- Phase 1
    o, lse = sa.star_phase1_encode(q, k, v, cfg.block, cfg.anchor)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(lse).all()) and bool(torch.isfinite(o.float()).all())
    rows = sample_rows(cfg)
    kh, vh = k.cpu(), v.cpu()
    ridx = torch.from_numpy(rows).to(DEV)
    ro, rl = oracle.phase1(q[:, ridx].cpu(), kh, vh, cfg.block, cfg.anchor, rows=rows, q_sampled=True)
    flush_print("  phase1 rows", rows.size)
    assert_out(o[:, ridx], ro, "%s phase-1 O" % name)
    assert_lse(lse[:, ridx], rl, "%s phase-1 LSE" % name)
    del o, lse

    # ---- Phase 2 query encoding
    k_tail = torch.zeros((cfg.hkv, cfg.tail_cap, cfg.d), dtype=q.dtype, device=DEV)
    v_tail = torch.zeros_like(k_tail)
    k_tail[:, :cfg.lq] = x["k_qry"]
    v_tail[:, :cfg.lq] = x["v_qry"]
    oq, lq_lse = sa.star_phase2_query(x["q_qry"], k, v, bounds, k_tail, v_tail, cfg.lq)
    op, lp_lse = _query_phase(cfg, x, bounds, k_tail, v_tail)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(lq_lse).all()) and bool(torch.isfinite(lp_lse).all())
    kq, vq = x["k_qry"].cpu(), x["v_qry"].cpu()
    for i in sorted({0, 1, cfg.lq // 2, cfg.lq - 1}):
        qi = x["q_qry"][:, i:i + 1].cpu()
        parts = [oracle.partial(qi, kh, vh, lo, hi) for lo, hi in zip(bounds[:-1], bounds[1:])]
        parts.append(oracle.partial(qi, kq, vq, 0, cfg.lq, i))
        ro_q, rl_q = oracle.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]),
                                  np.stack([p[2] for p in parts]))
        assert_out(oq[:, i:i + 1], ro_q, "%s query row %d O" % (name, i))
        assert_lse(lq_lse[:, i:i + 1], rl_q, "%s query row %d LSE" % (name, i))
        assert_out(op[:, i:i + 1], ro_q, "%s query row %d O (per partition)" % (name, i))
        assert_lse(lp_lse[:, i:i + 1], rl_q, "%s query row %d LSE (per partition)" % (name, i))
        if cfg.needle and i == 0:
            for g in range(cfg.hkv):
                h = g * cfg.G
                assert float(lq_lse[h, 0]) > 60.0, "needle should dominate row 0 of q head %d" % h
    flush_print("  query rows ok")

    # ---- Phase 2 decode, every step; the oracle on every step at 8b_32k, else on a spread
    T = cfg.decode_steps
    ws = sa.decode_workspace(cfg.L, cfg.tail_cap, cfg.shards, cfg.hq, cfg.hkv, cfg.d, DEV)
    od = torch.empty((T, cfg.hq, cfg.d), dtype=q.dtype, device=DEV)
    ld = torch.empty((T, cfg.hq), dtype=torch.float32, device=DEV)
    for t in range(T):
        sa.star_decode_step(x["q_dec"][t], x["k_dec"][t], x["v_dec"][t], k, v, bounds, k_tail, v_tail,
                            cfg.lq + t, o=od[t], lse=ld[t], workspace=ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(ld).all())
    assert torch.equal(k_tail[:, cfg.lq:], x["k_dec"].transpose(0, 1))
    assert torch.equal(v_tail[:, cfg.lq:], x["v_dec"].transpose(0, 1))
    kt, vt = k_tail.cpu(), v_tail.cpu()
    checked = range(T) if cfg.L <= 32768 else sorted(set(range(0, T, 8)) | {T // 2, T - 1})
    for t in checked:
        rod, rld = oracle.phase2_decode(x["q_dec"][t].cpu(), kh, vh, bounds, kt, vt, cfg.lq + t + 1)
        assert_out(od[t], rod, "%s decode step %d O" % (name, t))
        assert_lse(ld[t], rld, "%s decode step %d LSE" % (name, t))
    flush_print("  decode ok (%d steps checked)" % len(checked))


@pytest.mark.timeout(600)
def test_phase1_and_query_at_the_token_limit():
    """The longest context the MFMA kernels take: 2^31 / d tokens per kv head (L = 2^24 at
    d = 128), where a key's byte offset inside its head reaches 2^32 - 256.  Phase 1 (blocks of
    4096) and the query phase over four shards, checked on rows at the start and at the very
    end of the context, where the offsets are largest; then one decode step over it all."""
    L = 1 << 24
    cfg = StarConfig("limit", hq=2, hkv=1, d=128, L=L, block=4096, anchor=4096, lq=8, decode_steps=1,
                     shards=4, dtype="bf16", needle=False, seed=131)
    flush_print("token limit", L)
    q, k, v = sin.phase1_inputs(cfg, DEV)
    o, lse = sa.star_phase1_encode(q, k, v, cfg.block, cfg.anchor)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(lse).all())
    rows = np.array([0, 1, 4095, 4096, 4097, L // 2 + 77, L - 4096, L - 4095, L - 65, L - 64, L - 2, L - 1],
                    dtype=np.int64)
    kh, vh = k.cpu(), v.cpu()
    ridx = torch.from_numpy(rows).to(DEV)
    ro, rl = oracle.phase1(q[:, ridx].cpu(), kh, vh, cfg.block, cfg.anchor, rows=rows, q_sampled=True)
    assert_out(o[:, ridx], ro, "limit phase-1 O")
    assert_lse(lse[:, ridx], rl, "limit phase-1 LSE")
    flush_print("  phase1 ok")
    del o, lse, q
    p2 = sin.phase2_inputs(cfg, DEV)
    bounds = cfg.bounds()
    k_tail = torch.zeros((1, cfg.tail_cap, 128), dtype=torch.bfloat16, device=DEV)
    v_tail = torch.zeros_like(k_tail)
    k_tail[:, :cfg.lq] = p2["k_qry"]
    v_tail[:, :cfg.lq] = p2["v_qry"]
    oq, lq_lse = sa.star_phase2_query(p2["q_qry"], k, v, bounds, k_tail, v_tail, cfg.lq)
    torch.cuda.synchronize()
    ro, rl = oracle.phase2_query(p2["q_qry"].cpu(), kh, vh, bounds, p2["k_qry"].cpu(), p2["v_qry"].cpu())
    assert_out(oq, ro, "limit query O")
    assert_lse(lq_lse, rl, "limit query LSE")
    flush_print("  query ok")
    # one decode step over the whole context (chunks of about 62K tokens)
    ws = sa.decode_workspace(L, cfg.tail_cap, len(bounds) - 1, 2, 1, 128, DEV)
    od, ld = sa.star_decode_step(p2["q_dec"][0], p2["k_dec"][0], p2["v_dec"][0], k, v, bounds, k_tail, v_tail,
                                 cfg.lq, workspace=ws)
    torch.cuda.synchronize()
    ro, rl = oracle.phase2_decode(p2["q_dec"][0].cpu(), kh, vh, bounds, k_tail.cpu(), v_tail.cpu(), cfg.lq + 1)
    assert_out(od, ro, "limit decode O")
    assert_lse(ld, rl, "limit decode LSE")
    flush_print("  decode ok")
