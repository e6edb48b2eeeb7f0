"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle on the same
seeded inputs.  Sizes span several tiles and ragged tails so the oracle finishes in seconds.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_phase1_amd as sa
import oracle
from block_sparse_long_phase1_amd.configs import CONFIGS, StarConfig, shard_bounds
from block_sparse_long_phase1_amd import inputs as sin
from tests._parity import assert_lse, assert_out, flush_print, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _cfg(hq, hkv, L, b, a, d=128, dtype="bf16", lq=16, T=3, S=2, seed=7, needle=False):
    return StarConfig("test", hq=hq, hkv=hkv, d=d, L=L, block=b, anchor=a, lq=lq, decode_steps=T,
                      shards=S, dtype=dtype, needle=needle, seed=seed)


def test_native_library_is_the_in_tree_build():
    lib = sa.load_library()
    assert lib._name == sa.LIB_PATH
    assert torch.cuda.is_available()


# ----------------------------------------------------------------------------- Phase 1
PHASE1_CASES = [
    # hq, hkv, L, block, anchor
    (8, 2, 1000, 320, 320),    # G=4, ragged last block (40 rows), anchor = block
    (8, 2, 1000, 320, 200),    # anchor < block, not a multiple of the key tile
    (8, 2, 1000, 320, 0),      # no anchor: block-diagonal causal
    (8, 2, 700, 1024, 1024),   # one block covers the context: global causal
    (16, 2, 600, 256, 256),    # G=8
    (2, 2, 500, 200, 200),     # G=1
    (4, 2, 513, 128, 77),      # G=2, ragged everything
    (4, 1, 1, 1, 1),           # a single token
    (4, 2, 97, 1, 1),          # every token its own block
]


@pytest.mark.parametrize("hq,hkv,L,b,a", PHASE1_CASES)
def test_phase1_bf16(hq, hkv, L, b, a):
    flush_print("phase1 bf16", hq, hkv, L, b, a)
    cfg = _cfg(hq, hkv, L, b, a)
    q, k, v = sin.phase1_inputs(cfg, DEV)
    o, lse = sa.star_phase1_encode(q, k, v, b, a)
    torch.cuda.synchronize()
    ro, rl = oracle.phase1(q.cpu(), k.cpu(), v.cpu(), b, a)
    assert_out(o, ro, "O")
    assert_lse(lse, rl, "LSE")


@pytest.mark.parametrize("b", [512, 2048])
def test_phase1_f32_tiny(b):
    cfg = CONFIGS["tiny_f32"]
    flush_print("phase1 f32", cfg.name, b)
    q, k, v = sin.phase1_inputs(cfg, DEV)
    o, lse = sa.star_phase1_encode(q, k, v, b, min(b, cfg.anchor))
    torch.cuda.synchronize()
    ro, rl = oracle.phase1(q.cpu(), k.cpu(), v.cpu(), b, min(b, cfg.anchor))
    assert_out(o, ro, "O", max_abs=1e-5, mean_abs=1e-6)
    assert_lse(lse, rl, "LSE", rel=1e-6)


def test_phase1_bf16_vector_path_d96():
    """bf16 with a head dim the MFMA kernels do not take (96) uses the vector path; same
    reading, same bar."""
    cfg = _cfg(4, 2, 300, 128, 128, d=96)
    q, k, v = sin.phase1_inputs(cfg, DEV)
    o, lse = sa.star_phase1_encode(q, k, v, 128, 128)
    torch.cuda.synchronize()
    ro, rl = oracle.phase1(q.cpu(), k.cpu(), v.cpu(), 128, 128)
    assert_out(o, ro, "O")
    assert_lse(lse, rl, "LSE")


@pytest.mark.parametrize("hq,hkv,L,b,a", [
    (4, 2, 300, 128, 128),      # G=2
    (8, 2, 1000, 320, 200),     # G=4, ragged last block, anchor < block and not tile-aligned
    (16, 2, 600, 256, 256),     # G=8
    (2, 2, 500, 200, 200),      # G=1
    (8, 2, 700, 1024, 1024),    # one block: global causal
])
def test_phase1_bf16_d64(hq, hkv, L, b, a):
    """Head dim 64 on the MFMA kernel (8-row LDS blocks)."""
    flush_print("phase1 bf16 d64", hq, hkv, L, b, a)
    cfg = _cfg(hq, hkv, L, b, a, d=64, seed=53)
    q, k, v = sin.phase1_inputs(cfg, DEV)
    o, lse = sa.star_phase1_encode(q, k, v, b, a)
    torch.cuda.synchronize()
    ro, rl = oracle.phase1(q.cpu(), k.cpu(), v.cpu(), b, a)
    assert_out(o, ro, "O")
    assert_lse(lse, rl, "LSE")


def test_phase1_head_by_head_order_ragged():
    """A K/V cache above 256 MB takes the head-by-head work order; ragged last block, anchor
    not a multiple of the key tile, sampled rows against the oracle."""
    hq, hkv, L, b, a = 16, 8, 70000, 20000, 19999
    flush_print("phase1 head-by-head", hq, hkv, L, b, a)
    assert 2 * hkv * L * 128 * 2 > 256 << 20
    cfg = _cfg(hq, hkv, L, b, a, seed=41)
    q, k, v = sin.phase1_inputs(cfg, DEV)
    o, lse = sa.star_phase1_encode(q, k, v, b, a)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 1, 63, 64, a - 1, a, b - 1, b, b + 1, 2 * b - 1, 2 * b, 3 * b, 3 * b + 1,
                            L - 2, L - 1} | set(int(x) for x in np.random.default_rng(41).integers(0, L, 24))),
                    dtype=np.int64)
    ridx = torch.from_numpy(rows).to(DEV)
    ro, rl = oracle.phase1(q[:, ridx].cpu(), k.cpu(), v.cpu(), b, a, rows=rows, q_sampled=True)
    assert_out(o[:, ridx], ro, "O")
    assert_lse(lse[:, ridx], rl, "LSE")


def test_phase1_scores_jumping_past_the_reference():
    """A key scaled 30x in the middle of blocks makes scores jump far above the running
    reference, so Phase 1 must move its reference mid-row (the recompute path)."""
    hq, hkv, L, b, a = 8, 2, 2000, 640, 640
    cfg = _cfg(hq, hkv, L, b, a, seed=47)
    q, k, v = sin.phase1_inputs(cfg, DEV)
    k = k.clone()
    for p in (300, 900, 1500, 1900):
        k[:, p] = (k[:, p].float() * 30).to(k.dtype)
    o, lse = sa.star_phase1_encode(q, k, v, b, a)
    torch.cuda.synchronize()
    ro, rl = oracle.phase1(q.cpu(), k.cpu(), v.cpu(), b, a)
    assert float(np.max(rl)) > 60.0
    assert_out(o, ro, "O")
    assert_lse(lse, rl, "LSE")


def test_score_jump_in_the_second_half_of_a_tile():
    """A score far above every earlier one among keys 32..63 of a 64-key tile: the kernels
    take a tile's first half of probabilities before its second half's max, so when that max
    moves the reference the pending probabilities must move with it.  Phase 1 meets this on a
    work item's first tile (the anchor tile), Phase-2 partials on any tile."""
    hq, hkv, L, b, a = 8, 2, 1000, 320, 320
    G = hq // hkv
    cfg = _cfg(hq, hkv, L, b, a, seed=53)
    q, k, v = sin.phase1_inputs(cfg, DEV)
    k = k.clone()
    for g in range(hkv):                       # row 400 (block 1) meets anchor key 40
        k[g, 40] = (8 * q[g * G, 400].float()).to(k.dtype)
    o, lse = sa.star_phase1_encode(q, k, v, b, a)
    torch.cuda.synchronize()
    ro, rl = oracle.phase1(q.cpu(), k.cpu(), v.cpu(), b, a)
    assert rl[0, 400] > 40.0
    assert_out(o, ro, "phase-1 O")
    assert_lse(lse, rl, "phase-1 LSE")

    rows, n = 20, 1000
    qq = sin.randn(cfg, "q_qry", (hq, rows, 128), DEV)
    kk = sin.randn(cfg, "k_ctx", (hkv, n, 128), DEV).clone()
    vv = sin.randn(cfg, "v_ctx", (hkv, n, 128), DEV)
    for g in range(hkv):                       # tile 0 and tile 5, both in the second half
        kk[g, 40] = (8 * qq[g * G, 3].float()).to(kk.dtype)
        kk[g, 5 * 64 + 50] = (10 * qq[g * G + 1, 7].float()).to(kk.dtype)
    am, mm, lm = sa.star_phase2_partial(qq, kk, vv, n * 128, n, -1)
    torch.cuda.synchronize()
    ra, rm, rl2 = oracle.partial(qq.cpu(), kk.cpu(), vv.cpu(), 0, n, -1)
    assert float(np.max(rm)) > 40.0
    assert_out(am, ra, "partial A")
    assert_lse(mm + torch.log(lm), rm + np.log(rl2), "partial LSE")
    assert_lse(mm, rm, "m (largest scaled score)")


def test_phase1_locality_bitwise():
    """Keys outside a row's visible set cannot change its output, bit for bit."""
    cfg = _cfg(8, 2, 768, 256, 256)
    q, k, v = sin.phase1_inputs(cfg, DEV)
    o1, l1 = sa.star_phase1_encode(q, k, v, 256, 256)
    k2, v2 = k.clone(), v.clone()
    k2[:, 256:512] = -k2[:, 256:512]          # block 1 is invisible to block 2
    v2[:, 256:512] = 3.0
    o2, l2 = sa.star_phase1_encode(q, k2, v2, 256, 256)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, 512:], o2[:, 512:]) and torch.equal(l1[:, 512:], l2[:, 512:])
    assert torch.equal(o1[:, :256], o2[:, :256])
    assert not torch.equal(l1[:, 256:512], l2[:, 256:512])


# ----------------------------------------------------------------------------- Phase 2 partial
PARTIAL_CASES = [
    # hq, hkv, rows, T_total, lo, hi, causal_offset
    (8, 2, 128, 1200, 100, 1100, -1),   # shard view inside a longer cache, several splits
    (8, 2, 100, 3000, 0, 3000, -1),     # ragged rows, many splits
    (8, 2, 70, 80, 0, 70, 0),           # query host's own cache: causal among the rows
    (8, 2, 40, 200, 0, 120, 5),         # causal with an offset
    (16, 2, 33, 500, 17, 417, -1),      # G=8
    (8, 2, 16, 64, 10, 10, -1),         # empty partition
]


@pytest.mark.parametrize("hq,hkv,rows,T,lo,hi,off,d", [c + (128,) for c in PARTIAL_CASES] + [
    (8, 2, 100, 3000, 0, 3000, -1, 64),   # head dim 64, several splits
    (8, 2, 70, 80, 0, 70, 0, 64),         # head dim 64, causal
])
def test_phase2_partial_bf16(hq, hkv, rows, T, lo, hi, off, d):
    flush_print("partial", hq, hkv, rows, T, lo, hi, off, d)
    cfg = _cfg(hq, hkv, T, T, T, seed=11)
    q = sin.randn(cfg, "q_qry", (hq, rows, d), DEV)
    k = sin.randn(cfg, "k_ctx", (hkv, T, d), DEV)
    v = sin.randn(cfg, "v_ctx", (hkv, T, d), DEV)
    a, m, l = sa.star_phase2_partial(q, k[:, lo:], v[:, lo:], T * d, hi - lo, off)
    torch.cuda.synchronize()
    ra, rm, rl = oracle.partial(q.cpu(), k.cpu(), v.cpu(), lo, hi, off)
    if hi == lo:
        assert torch.all(a == 0) and torch.all(torch.isneginf(m)) and torch.all(l == 0)
        return
    assert_out(a, ra, "A")
    assert_lse(m + torch.log(l), rm + np.log(rl), "partial LSE")
    assert_lse(m, rm, "m (largest scaled score)")


def test_phase2_partial_f32():
    cfg = CONFIGS["tiny_f32"]
    q = sin.randn(cfg, "q_qry", (1, 16, 64), DEV)
    k = sin.randn(cfg, "k_ctx", (1, 2048, 64), DEV)
    v = sin.randn(cfg, "v_ctx", (1, 2048, 64), DEV)
    for lo, hi, off in [(0, 1024, -1), (1024, 2048, -1), (0, 16, 0)]:
        a, m, l = sa.star_phase2_partial(q, k[:, lo:], v[:, lo:], 2048 * 64, hi - lo, off)
        torch.cuda.synchronize()
        ra, rm, rl = oracle.partial(q.cpu(), k.cpu(), v.cpu(), lo, hi, off)
        assert_out(a, ra, "A", max_abs=1e-5, mean_abs=1e-6)
        assert_lse(m + torch.log(l), rm + np.log(rl), "partial LSE", rel=1e-6)


# ----------------------------------------------------------------------------- merge
@pytest.mark.parametrize("P,hq,rows,d", [(1, 4, 3, 128), (5, 8, 17, 128), (300, 32, 1, 128), (7, 2, 5, 64)])
def test_softmax_merge(P, hq, rows, d):
    rng = np.random.default_rng(P * 131 + rows)
    a = rng.standard_normal((P, hq, rows, d)).astype(np.float32)
    m = (rng.standard_normal((P, hq, rows)) * 20).astype(np.float32)
    l = rng.uniform(0.5, 100.0, (P, hq, rows)).astype(np.float32)
    if P > 1:   # some empty partitions and one row with every partition empty
        m[0, 0, 0] = -np.inf
        l[0, 0, 0] = 0.0
        m[:, -1, -1] = -np.inf
        l[:, -1, -1] = 0.0
    ta, tm, tl = (torch.from_numpy(x).to(DEV) for x in (a, m, l))
    o, lse = sa.star_softmax_merge(ta, tm, tl)
    ob, _ = sa.star_softmax_merge(ta, tm, tl, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ro, rl = oracle.merge(a.astype(np.float64), m.astype(np.float64), l.astype(np.float64))
    assert_out(o, ro, "O", max_abs=2e-5, mean_abs=2e-6)
    assert_lse(lse, rl, "LSE", rel=1e-6)
    assert_out(ob, ro, "O bf16", max_abs=2e-2, mean_abs=2e-3)


def test_merge_needle_scale():
    """Partials whose sums would overflow fp32 (scores near 90) merge exactly in log space."""
    a = torch.tensor([[[[1.0] * 128]], [[[3.0] * 128]]], dtype=torch.float32, device=DEV)
    m = torch.tensor([[[90.0]], [[90.0 + float(np.log(3.0))]]], dtype=torch.float32, device=DEV)
    l = torch.ones((2, 1, 1), dtype=torch.float32, device=DEV)
    o, lse = sa.star_softmax_merge(a, m, l)
    torch.cuda.synchronize()
    assert torch.allclose(o, torch.full_like(o, 2.5), atol=1e-5)
    assert abs(float(lse) - (90.0 + np.log(4.0))) < 1e-4


# ----------------------------------------------------------------------------- full Phase 2
def _run_query_phase(cfg, x, bounds, k_tail, v_tail):
    """S context partials + the query host's causal partial, merged (all through the C ABI)."""
    q = x["q_qry"]
    lq, L = cfg.lq, cfg.L
    parts_a, parts_m, parts_l = [], [], []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        a, m, l = sa.star_phase2_partial(q, x["k_ctx"][:, lo:], x["v_ctx"][:, lo:], L * cfg.d, hi - lo, -1)
        parts_a.append(a); parts_m.append(m); parts_l.append(l)
    a, m, l = sa.star_phase2_partial(q, k_tail, v_tail, cfg.tail_cap * cfg.d, lq, 0)
    parts_a.append(a); parts_m.append(m); parts_l.append(l)
    return sa.star_softmax_merge(torch.stack(parts_a), torch.stack(parts_m), torch.stack(parts_l),
                                 out_dtype=q.dtype)


@pytest.mark.parametrize("hq,hkv,L,b,S,lq,T,dtype,d", [
    (8, 2, 3000, 800, 3, 40, 3, "bf16", 128),
    (16, 2, 1500, 512, 2, 20, 2, "bf16", 128),
    (8, 2, 1500, 512, 3, 20, 2, "bf16", 64),   # head dim 64: MFMA query and decode
    (16, 1, 2333, 700, 4, 5, 3, "bf16", 64),   # d = 64, G = 16, ragged last shard
    (4, 4, 777, 256, 3, 1, 2, "bf16", 64),     # d = 64, G = 1, one cached query token
    (1, 1, 2048, 512, 2, 16, 4, "f32", 64),
])
def test_phase2_query_and_decode(hq, hkv, L, b, S, lq, T, dtype, d):
    flush_print("phase2", hq, hkv, L, b, S, lq, T, dtype)
    cfg = _cfg(hq, hkv, L, b, b, d=d, dtype=dtype, lq=lq, T=T, S=S, seed=23)
    q, k, v = sin.phase1_inputs(cfg, DEV)
    x = {"k_ctx": k, "v_ctx": v}
    x.update(sin.phase2_inputs(cfg, DEV))
    bounds = shard_bounds(L, b, S)
    tdt = x["k_qry"].dtype
    k_tail = torch.zeros((hkv, cfg.tail_cap, d), dtype=tdt, device=DEV)
    v_tail = torch.zeros_like(k_tail)
    k_tail[:, :lq] = x["k_qry"]
    v_tail[:, :lq] = x["v_qry"]
    o, lse = _run_query_phase(cfg, x, bounds, k_tail, v_tail)
    of, lf = sa.star_phase2_query(x["q_qry"], k, v, bounds, k_tail, v_tail, lq)
    torch.cuda.synchronize()
    ro, rl = oracle.phase2_query(x["q_qry"].cpu(), k.cpu(), v.cpu(), bounds, x["k_qry"].cpu(), x["v_qry"].cpu())
    tol = dict(max_abs=2e-2, mean_abs=2e-3) if dtype == "bf16" else dict(max_abs=1e-5, mean_abs=1e-6)
    assert_out(o, ro, "query O", **tol)
    assert_lse(lse, rl, "query LSE", rel=1e-5 if dtype == "bf16" else 1e-6)
    assert_out(of, ro, "fused query O", **tol)
    assert_lse(lf, rl, "fused query LSE", rel=1e-5 if dtype == "bf16" else 1e-6)
    ws = sa.decode_workspace(L, cfg.tail_cap, S, hq, hkv, d, DEV)
    for t in range(T):
        od, ld = sa.star_decode_step(x["q_dec"][t], x["k_dec"][t], x["v_dec"][t], k, v, bounds,
                                     k_tail, v_tail, lq + t, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(k_tail[:, lq + t], x["k_dec"][t]) and torch.equal(v_tail[:, lq + t], x["v_dec"][t])
        rod, rld = oracle.phase2_decode(x["q_dec"][t].cpu(), k.cpu(), v.cpu(), bounds, k_tail.cpu(),
                                        v_tail.cpu(), lq + t + 1)
        assert_out(od, rod, "decode O step %d" % t, **tol)
        assert_lse(ld, rld, "decode LSE step %d" % t, rel=1e-5 if dtype == "bf16" else 1e-6)


@pytest.mark.parametrize("hq,hkv,L,bounds,rows,tail_len,tail_cap", [
    (8, 2, 1000, [0, 250, 250, 900, 1000], 40, 40, 48),        # an empty shard, ragged shards
    (16, 2, 2500, [0, 1300, 2500], 9, 30, 33),                 # G=8; query rows after 21 cached tokens
    (4, 4, 700, [0, 700], 1, 1, 1),                            # G=1, one row, one cached token
    (8, 1, 6000, [0, 1500, 3000, 4500, 6000], 300, 300, 310),  # several row tiles and key splits
])
def test_phase2_query_fused(hq, hkv, L, bounds, rows, tail_len, tail_cap):
    """star_phase2_query (every partition in one call) against the oracle's partials + merge."""
    flush_print("phase2 query", hq, hkv, L, bounds, rows, tail_len)
    cfg = _cfg(hq, hkv, L, L, L, lq=tail_len, T=1, S=len(bounds) - 1, seed=37)
    q, k, v = sin.phase1_inputs(cfg, DEV)
    p2 = sin.phase2_inputs(cfg, DEV)
    qr = p2["q_qry"][:, tail_len - rows:].contiguous()
    k_tail = torch.zeros((hkv, tail_cap, 128), dtype=torch.bfloat16, device=DEV)
    v_tail = torch.zeros_like(k_tail)
    k_tail[:, :tail_len] = p2["k_qry"]
    v_tail[:, :tail_len] = p2["v_qry"]
    o, lse = sa.star_phase2_query(qr, k, v, bounds, k_tail, v_tail, tail_len)
    torch.cuda.synchronize()
    qc, kc, vc = qr.cpu(), k.cpu(), v.cpu()
    parts = [oracle.partial(qc, kc, vc, lo, hi) for lo, hi in zip(bounds[:-1], bounds[1:])]
    parts.append(oracle.partial(qc, k_tail.cpu(), v_tail.cpu(), 0, tail_len, tail_len - rows))
    ro, rl = oracle.merge(np.stack([x[0] for x in parts]), np.stack([x[1] for x in parts]),
                          np.stack([x[2] for x in parts]))
    assert_out(o, ro, "O")
    assert_lse(lse, rl, "LSE")


@pytest.mark.parametrize("d", [128, 64])
def test_decode_empty_shard_and_first_token(d):
    """A shard with no tokens weighs nothing; tail_len = 0 is the first cached token."""
    cfg = _cfg(8, 2, 1000, 250, 250, d=d, lq=1, T=1, S=4, seed=29)
    q, k, v = sin.phase1_inputs(cfg, DEV)
    p2 = sin.phase2_inputs(cfg, DEV)
    bounds = [0, 250, 250, 900, 1000]
    k_tail = torch.zeros((2, 4, d), dtype=torch.bfloat16, device=DEV)
    v_tail = torch.zeros_like(k_tail)
    o, lse = sa.star_decode_step(p2["q_dec"][0], p2["k_dec"][0], p2["v_dec"][0], k, v, bounds, k_tail, v_tail, 0)
    torch.cuda.synchronize()
    ro, rl = oracle.phase2_decode(p2["q_dec"][0].cpu(), k.cpu(), v.cpu(), bounds, k_tail.cpu(), v_tail.cpu(), 1)
    assert_out(o, ro, "O")
    assert_lse(lse, rl, "LSE")


@pytest.mark.parametrize("G,d", [(1, 128), (4, 128), (2, 64), (4, 64)])
def test_decode_merge_over_many_chunks(G, d):
    """One kv head: the chunk plan gives it 271 context chunks' worth of budget, here 158 chunks
    of 128 keys over shards of 7000, 1 and 12999 tokens, plus the query host's chunk (159 in
    all).  The last workgroup of the head then merges three batches of chunk partials (64, 64,
    31), the last one ragged against the 2 (d = 128) or 4 (d = 64) chunk rows each of its
    16-byte loads covers.  Two consecutive steps, both checked against the oracle."""
    hq, hkv, L, lq, T = G, 1, 20000, 5, 2
    flush_print("decode many chunks", G, d)
    cfg = _cfg(hq, hkv, L, L, L, d=d, lq=lq, T=T, S=3, seed=83)
    q, k, v = sin.phase1_inputs(cfg, DEV)
    p2 = sin.phase2_inputs(cfg, DEV)
    bounds = [0, 7000, 7001, 20000]
    k_tail = torch.zeros((hkv, lq + T, d), dtype=torch.bfloat16, device=DEV)
    v_tail = torch.zeros_like(k_tail)
    k_tail[:, :lq] = p2["k_qry"]
    v_tail[:, :lq] = p2["v_qry"]
    ws = sa.decode_workspace(L, lq + T, len(bounds) - 1, hq, hkv, d, DEV)
    for t in range(T):
        o, lse = sa.star_decode_step(p2["q_dec"][t], p2["k_dec"][t], p2["v_dec"][t], k, v, bounds, k_tail, v_tail,
                                     lq + t, workspace=ws)
        torch.cuda.synchronize()
        ro, rl = oracle.phase2_decode(p2["q_dec"][t].cpu(), k.cpu(), v.cpu(), bounds, k_tail.cpu(), v_tail.cpu(),
                                      lq + t + 1)
        assert_out(o, ro, "O step %d" % t)
        assert_lse(lse, rl, "LSE step %d" % t)


def test_decode_shard_split_invariance():
    """Any host split gives the same decode output (partition identity), to fp32 rounding."""
    cfg = _cfg(8, 2, 4096, 1024, 1024, lq=8, T=1, S=4, seed=31)
    q, k, v = sin.phase1_inputs(cfg, DEV)
    p2 = sin.phase2_inputs(cfg, DEV)
    outs = []
    for bounds in ([0, 4096], [0, 1024, 2048, 3072, 4096], [0, 1, 2, 4000, 4096], [0, 17, 1717, 4096]):
        k_tail = torch.zeros((2, 9, 128), dtype=torch.bfloat16, device=DEV)
        v_tail = torch.zeros_like(k_tail)
        k_tail[:, :8] = p2["k_qry"]
        v_tail[:, :8] = p2["v_qry"]
        o, lse = sa.star_decode_step(p2["q_dec"][0], p2["k_dec"][0], p2["v_dec"][0], k, v, bounds,
                                     k_tail, v_tail, 8)
        outs.append((o.float(), lse))
    torch.cuda.synchronize()
    for o, lse in outs[1:]:
        assert (o - outs[0][0]).abs().max().item() <= 1e-2
        assert (lse - outs[0][1]).abs().max().item() <= 1e-5 * max(1.0, outs[0][1].abs().max().item())


@pytest.mark.parametrize("d", [128, 64])
def test_batch_as_folded_heads(d):
    """B equal-length sequences laid out [B, H, tokens, d] are one call with B*Hq q heads and
    B*Hkv kv heads (q head b*Hq + h maps to kv head b*Hkv + h/G): each sequence's slice of
    every output matches the oracle run on that sequence alone."""
    B, hq, hkv, L, b, a, lq, S = 3, 8, 2, 1100, 512, 256, 5, 2
    flush_print("batch", B, hq, hkv, L, b, a, d)
    cfgs = [_cfg(hq, hkv, L, b, a, d=d, lq=lq, T=1, S=S, seed=61 + i) for i in range(B)]
    ins = [sin.phase1_inputs(c, DEV) for c in cfgs]
    p2s = [sin.phase2_inputs(c, DEV) for c in cfgs]
    q, k, v = (torch.cat([x[i] for x in ins]) for i in range(3))
    o, lse = sa.star_phase1_encode(q, k, v, b, a)
    bounds = shard_bounds(L, b, S)
    cap = cfgs[0].tail_cap
    k_tail = torch.zeros((B * hkv, cap, d), dtype=torch.bfloat16, device=DEV)
    v_tail = torch.zeros_like(k_tail)
    k_tail[:, :lq] = torch.cat([p["k_qry"] for p in p2s])
    v_tail[:, :lq] = torch.cat([p["v_qry"] for p in p2s])
    qq = torch.cat([p["q_qry"] for p in p2s])
    oq, lq_lse = sa.star_phase2_query(qq, k, v, bounds, k_tail, v_tail, lq)
    ws = sa.decode_workspace(L, cap, S, B * hq, B * hkv, d, DEV)
    od, ld = sa.star_decode_step(torch.cat([p["q_dec"][0] for p in p2s]), torch.cat([p["k_dec"][0] for p in p2s]),
                                 torch.cat([p["v_dec"][0] for p in p2s]), k, v, bounds, k_tail, v_tail, lq,
                                 workspace=ws)
    torch.cuda.synchronize()
    for i in range(B):
        qs, ks = slice(i * hq, (i + 1) * hq), slice(i * hkv, (i + 1) * hkv)
        kc, vc = k[ks].cpu(), v[ks].cpu()
        ro, rl = oracle.phase1(q[qs].cpu(), kc, vc, b, a)
        assert_out(o[qs], ro, "phase 1 O, sequence %d" % i)
        assert_lse(lse[qs], rl, "phase 1 LSE, sequence %d" % i)
        ro, rl = oracle.phase2_query(qq[qs].cpu(), kc, vc, bounds, p2s[i]["k_qry"].cpu(), p2s[i]["v_qry"].cpu())
        assert_out(oq[qs], ro, "query O, sequence %d" % i)
        assert_lse(lq_lse[qs], rl, "query LSE, sequence %d" % i)
        ro, rl = oracle.phase2_decode(p2s[i]["q_dec"][0].cpu(), kc, vc, bounds, k_tail[ks].cpu(), v_tail[ks].cpu(),
                                      lq + 1)
        assert_out(od[qs], ro, "decode O, sequence %d" % i)
        assert_lse(ld[qs], rl, "decode LSE, sequence %d" % i)


def test_phase1_and_query_replayed_from_a_hip_graph():
    """Phase 1 and the query phase captured in one HIP graph replay bit-identically to the eager
    calls (several replays, eager work and synchronisation between them)."""
    cfg = _cfg(8, 2, 2600, 1000, 1000, lq=40, T=1, S=3, seed=59)
    q, k, v = sin.phase1_inputs(cfg, DEV)
    p2 = sin.phase2_inputs(cfg, DEV)
    bounds = shard_bounds(cfg.L, cfg.block, cfg.shards)
    kt = torch.zeros((cfg.hkv, cfg.tail_cap, cfg.d), dtype=torch.bfloat16, device=DEV)
    vt = torch.zeros_like(kt)
    kt[:, :cfg.lq] = p2["k_qry"]
    vt[:, :cfg.lq] = p2["v_qry"]
    o_e, l_e = sa.star_phase1_encode(q, k, v, cfg.block, cfg.anchor)
    oq_e, lq_e = sa.star_phase2_query(p2["q_qry"], k, v, bounds, kt, vt, cfg.lq)
    torch.cuda.synchronize()
    o = torch.empty_like(o_e)
    lse = torch.empty_like(l_e)
    oq = torch.empty_like(oq_e)
    lq = torch.empty_like(lq_e)
    ws = torch.empty(max(16, sa.star_phase2_query_workspace_bytes(cfg.lq, len(bounds) - 1, cfg.hq, cfg.hkv, cfg.d)),
                     dtype=torch.uint8, device=DEV)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sa.star_phase1_encode(q, k, v, cfg.block, cfg.anchor, o=o, lse=lse)
        sa.star_phase2_query(p2["q_qry"], k, v, bounds, kt, vt, cfg.lq, o=oq, lse=lq, workspace=ws)
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_e) and torch.equal(lse, l_e), "replay %d: Phase 1 differs" % rep
        assert torch.equal(oq, oq_e) and torch.equal(lq, lq_e), "replay %d: query phase differs" % rep
        for t in (o, lse, oq, lq):
            t.zero_()
        sa.star_decode_step(p2["q_dec"][0], p2["k_dec"][0], p2["v_dec"][0], k, v, bounds, kt.clone(), vt.clone(),
                            cfg.lq)
        torch.cuda.synchronize()


@pytest.mark.parametrize("hq", [8, 16])   # G = 4: merge in the decode launch; G = 8: merge_kernel after it
def test_decode_steps_replayed_from_a_hip_graph(hq):
    """T decode steps captured in one HIP graph (the library allocates nothing and records no
    memsets) replay bit-identically to the eager calls, with eager work between replays."""
    cfg = _cfg(hq, 2, 3000, 1000, 1000, lq=16, T=4, S=3, seed=43)
    q, k, v = sin.phase1_inputs(cfg, DEV)
    p2 = sin.phase2_inputs(cfg, DEV)
    bounds = shard_bounds(cfg.L, cfg.block, cfg.shards)
    T, lq = cfg.decode_steps, cfg.lq

    def fresh_tail():
        kt = torch.zeros((cfg.hkv, cfg.tail_cap, cfg.d), dtype=torch.bfloat16, device=DEV)
        vt = torch.zeros_like(kt)
        kt[:, :lq] = p2["k_qry"]
        vt[:, :lq] = p2["v_qry"]
        return kt, vt

    kt, vt = fresh_tail()
    ws = sa.decode_workspace(cfg.L, cfg.tail_cap, cfg.shards, cfg.hq, cfg.hkv, cfg.d, DEV)
    eager = []
    for t in range(T):
        o, l = sa.star_decode_step(p2["q_dec"][t], p2["k_dec"][t], p2["v_dec"][t], k, v, bounds, kt, vt, lq + t,
                                   workspace=ws)
        eager.append((o.clone(), l.clone()))
    kt2, vt2 = fresh_tail()
    ws2 = sa.decode_workspace(cfg.L, cfg.tail_cap, cfg.shards, cfg.hq, cfg.hkv, cfg.d, DEV)
    outs = [(torch.empty((cfg.hq, cfg.d), dtype=torch.bfloat16, device=DEV),
             torch.empty((cfg.hq,), dtype=torch.float32, device=DEV)) for _ in range(T)]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(T):
            sa.star_decode_step(p2["q_dec"][t], p2["k_dec"][t], p2["v_dec"][t], k, v, bounds, kt2, vt2, lq + t,
                                o=outs[t][0], lse=outs[t][1], workspace=ws2)
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for t in range(T):
            assert torch.equal(outs[t][0], eager[t][0]), "replay %d step %d: O differs" % (rep, t)
            assert torch.equal(outs[t][1], eager[t][1]), "replay %d step %d: LSE differs" % (rep, t)
        assert torch.equal(kt2, kt) and torch.equal(vt2, vt)
        # unrelated eager work between replays
        sa.star_phase1_encode(q, k, v, cfg.block, cfg.anchor)
        for t in range(T):
            outs[t][0].zero_()
            outs[t][1].zero_()
        torch.cuda.synchronize()
