"""Pins for the fp64 oracle: checks against what the pages and the mathematics fix.

Each test names the passage it rests on.  Pages:
  [SUM]    "Star Attention: Efficient LLM Inference over Long Sequences"
           (paper-graph-ui summary of arXiv 2411.17116), section 3.4;
  [README] "NVIDIA/Star-Attention" (shadowgraph.io mirror), "Two Phases of Star Attention".
None of these tests needs a GPU.
"""
import math

import numpy as np
import pytest

from tests._dense import bf16_bits, bf16_to_f64, causal_mask, dense


def _rand(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


def _anchored_mask(L, block, anchor):
    """Visibility of context row p over key j, written from the augmented-block picture:
    block i >= 1 is the sequence [anchor tokens ; block i tokens] attended causally."""
    m = np.zeros((L, L), dtype=bool)
    for p in range(L):
        i = p // block
        start = i * block
        if i >= 1:
            m[p, :anchor] = True
        m[p, start:p + 1] = True
    return m


# --------------------------------------------------------------------------------------
# Pin 1: one block covering the whole context is plain global causal attention.
# [SUM] 3.4 Phase 1 Steps 1 and 4 (n = ceil(L/b) = 1: the only block is attended causally
# as a standalone sequence) and "The Attention Decomposition" (the causal formula).
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("block", [37, 64])
def test_single_block_is_global_causal(oracle_lib, dtype, block):
    rng = np.random.default_rng(1)
    hq, hkv, L, d = 4, 2, 37, 16
    q, k, v = _rand(rng, hq, L, d), _rand(rng, hkv, L, d), _rand(rng, hkv, L, d)
    if dtype == "bf16":
        qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
        o, lse = oracle_lib.phase1(qb, kb, vb, block, min(block, 16))
        q, k, v = bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb)
    else:
        o, lse = oracle_lib.phase1(q, k, v, block, min(block, 16))
        q, k, v = q.astype(np.float64), k.astype(np.float64), v.astype(np.float64)
    od, lsed = dense(q, k, v, causal_mask(L, L))
    np.testing.assert_allclose(o, od, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lsed, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------------------
# Pin 2: with anchor = block, rows of the first two blocks equal global causal rows
# (block 2's augmented sequence [c1 ; c2] is exactly the causal prefix).  Later blocks
# must differ from global attention.  [SUM] 3.4 Phase 1 Step 2.
# --------------------------------------------------------------------------------------
def test_anchor_equal_block_first_two_blocks_global(oracle_lib):
    rng = np.random.default_rng(2)
    hq, hkv, L, d, b = 2, 1, 48, 8, 12
    q, k, v = _rand(rng, hq, L, d), _rand(rng, hkv, L, d), _rand(rng, hkv, L, d)
    o, lse = oracle_lib.phase1(q, k, v, b, b)
    od, lsed = dense(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), causal_mask(L, L))
    np.testing.assert_allclose(o[:, :2 * b], od[:, :2 * b], atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse[:, :2 * b], lsed[:, :2 * b], atol=1e-12, rtol=0)
    assert np.abs(lse[:, 2 * b + 1:] - lsed[:, 2 * b + 1:]).min() > 1e-6


# --------------------------------------------------------------------------------------
# Pin 3: anchor = 0 is block-diagonal causal attention ("no anchor block" ablation,
# [SUM] 3.4 "Why Anchor Blocks Are Necessary").
# --------------------------------------------------------------------------------------
def test_no_anchor_is_block_diagonal(oracle_lib):
    rng = np.random.default_rng(3)
    hq, hkv, L, d, b = 3, 1, 30, 8, 8  # ragged last block (30 = 3*8 + 6)
    q, k, v = _rand(rng, hq, L, d), _rand(rng, hkv, L, d), _rand(rng, hkv, L, d)
    o, lse = oracle_lib.phase1(q, k, v, b, 0)
    blk = np.arange(L) // b
    mask = causal_mask(L, L) & (blk[:, None] == blk[None, :])
    od, lsed = dense(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), mask)
    np.testing.assert_allclose(o, od, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lsed, atol=1e-12, rtol=0)


# --------------------------------------------------------------------------------------
# Pin 4: closed form with all-zero keys.  Every visible score is 0, so LSE = ln|V(p)| and O
# is the plain mean of the visible value rows.  With V[j,0] = j and V[j,1] = j^2 the mean
# index and mean square index are closed-form sums, which pins the exact key ranges
# (anchor [0,a) for blocks >= 2, own block start..p) including a < b and a ragged tail.
# [SUM] 3.4 Phase 1 Steps 1, 2, 4.
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("L,b,a", [(50, 16, 16), (50, 16, 5), (64, 16, 0), (9, 4, 3), (23, 23, 7)])
def test_zero_keys_closed_form(oracle_lib, L, b, a):
    hq, hkv, d = 2, 1, 4
    rng = np.random.default_rng(4)
    q = _rand(rng, hq, L, d)
    k = np.zeros((hkv, L, d), np.float32)
    v = np.zeros((hkv, L, d), np.float32)
    j = np.arange(L, dtype=np.float64)
    v[0, :, 0] = j
    v[0, :, 1] = j * j
    o, lse = oracle_lib.phase1(q, k, v, b, a)
    for p in range(L):
        i, start = p // b, (p // b) * b
        own_n = p - start + 1
        own_s1 = (start + p) * own_n / 2.0
        own_s2 = (p * (p + 1) * (2 * p + 1) - (start - 1) * start * (2 * start - 1)) / 6.0
        if i >= 1:
            n = a + own_n
            s1 = a * (a - 1) / 2.0 + own_s1
            s2 = (a - 1) * a * (2 * a - 1) / 6.0 + own_s2
        else:
            n, s1, s2 = own_n, own_s1, own_s2
        for h in range(hq):
            assert abs(lse[h, p] - math.log(n)) < 1e-12
            assert abs(o[h, p, 0] - s1 / n) < 1e-9
            assert abs(o[h, p, 1] - s2 / n) < 1e-7 * max(1.0, s2 / n)
            assert o[h, p, 2] == 0.0 and o[h, p, 3] == 0.0


# --------------------------------------------------------------------------------------
# Pin 5: literal augmentation, brute force.  Build each augmented block [c_1 ; c_i] as an
# explicit token list (anchor first, [SUM] 3.4 Phase 1 Step 2; [README] Phase 1), run
# per-element causal softmax attention over it in pure Python, and keep only the rows of
# the block's own tokens (anchor rows and KV are discarded, Step 5).
# --------------------------------------------------------------------------------------
def _bruteforce_phase1(q, k, v, L, b, a):
    hq, _, d = q.shape
    G = hq // k.shape[0]
    out = np.zeros((hq, L, d))
    lse = np.zeros((hq, L))
    n = -(-L // b)
    for i in range(n):
        own = list(range(i * b, min(L, (i + 1) * b)))
        seq = (list(range(a)) if i >= 1 else []) + own   # the augmented sequence
        for h in range(hq):
            g = h // G
            for pos_in_seq, p in enumerate(seq):
                if p not in own or (i >= 1 and pos_in_seq < a):
                    continue                             # anchor rows are not produced
                keys = seq[:pos_in_seq + 1]              # causal inside the augmented block
                xs = [sum(float(q[h, p, e]) * float(k[g, j, e]) for e in range(d)) / math.sqrt(d)
                      for j in keys]
                mx = max(xs)
                ws = [math.exp(x - mx) for x in xs]
                den = sum(ws)
                for e in range(d):
                    out[h, p, e] = sum(w * float(v[g, j, e]) for w, j in zip(ws, keys)) / den
                lse[h, p] = mx + math.log(den)
    return out, lse


@pytest.mark.parametrize("L,b,a", [(12, 4, 4), (14, 4, 2), (10, 3, 0), (7, 7, 7)])
def test_literal_augmentation_bruteforce(oracle_lib, L, b, a):
    rng = np.random.default_rng(5)
    hq, hkv, d = 4, 2, 3
    q, k, v = _rand(rng, hq, L, d), _rand(rng, hkv, L, d), _rand(rng, hkv, L, d)
    o, lse = oracle_lib.phase1(q, k, v, b, a)
    ob, lseb = _bruteforce_phase1(q, k, v, L, b, a)
    np.testing.assert_allclose(o, ob, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lseb, atol=1e-12, rtol=0)


def test_phase1_row_sampling_matches_full(oracle_lib):
    rng = np.random.default_rng(6)
    hq, hkv, L, d, b = 4, 2, 40, 8, 10
    q, k, v = _rand(rng, hq, L, d), _rand(rng, hkv, L, d), _rand(rng, hkv, L, d)
    o, lse = oracle_lib.phase1(q, k, v, b, b)
    rows = np.array([39, 0, 10, 11, 25], dtype=np.int64)
    os_, ls_ = oracle_lib.phase1(q, k, v, b, b, rows=rows)
    np.testing.assert_array_equal(os_, o[:, rows])
    np.testing.assert_array_equal(ls_, lse[:, rows])
    os2, ls2 = oracle_lib.phase1(np.ascontiguousarray(q[:, rows]), k, v, b, b, rows=rows, q_sampled=True)
    np.testing.assert_array_equal(os2, o[:, rows])
    np.testing.assert_array_equal(ls2, lse[:, rows])


# --------------------------------------------------------------------------------------
# Pin 6: the partition identity.  [SUM] 3.4 Phase 2 "Why this decomposition works" and
# [README] Phase 2: for disjoint key partitions, sum_h (s_h / s_global) A_h equals softmax
# attention over the union, exactly.  Checked against dense softmax for several splits,
# including empty partitions; merging is associative; a single partition is the identity.
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("cuts", [[0, 61], [0, 30, 61], [0, 1, 2, 3, 61], [0, 0, 20, 20, 61, 61],
                                  [0, 7, 19, 33, 34, 50, 61]])
def test_merge_equals_dense_softmax(oracle_lib, cuts):
    rng = np.random.default_rng(7)
    hq, hkv, R, T, d = 4, 2, 5, 61, 8
    q, k, v = _rand(rng, hq, R, d), _rand(rng, hkv, T, d), _rand(rng, hkv, T, d)
    parts = [oracle_lib.partial(q, k, v, lo, hi) for lo, hi in zip(cuts[:-1], cuts[1:])]
    o, lse = oracle_lib.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]),
                              np.stack([p[2] for p in parts]))
    od, lsed = dense(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                     np.ones((R, T), bool))
    np.testing.assert_allclose(o, od, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse, lsed, atol=1e-13, rtol=0)


def test_partial_is_local_softmax_and_sum(oracle_lib):
    """A_h is normalised over the partition only and s_h = e^m l is the partition's sum of
    exponentials ([SUM] 3.4 Phase 2 Step 3 equations for A_h and s_h)."""
    rng = np.random.default_rng(8)
    hq, hkv, R, T, d = 2, 1, 3, 20, 4
    q, k, v = _rand(rng, hq, R, d), _rand(rng, hkv, T, d), _rand(rng, hkv, T, d)
    a, m, l = oracle_lib.partial(q, k, v, 5, 13)
    s = np.einsum("hrd,td->hrt", q.astype(np.float64), k[0, 5:13].astype(np.float64)) / math.sqrt(d)
    np.testing.assert_allclose(np.exp(m) * l, np.exp(s).sum(-1), rtol=1e-13)
    np.testing.assert_allclose(a, (np.exp(s) / np.exp(s).sum(-1, keepdims=True)) @ v[0, 5:13], atol=1e-13)


def test_merge_associative_and_identity(oracle_lib):
    rng = np.random.default_rng(9)
    P, n, d = 3, 6, 5
    a = rng.standard_normal((P, n, d))
    m = rng.standard_normal((P, n)) * 30
    l = rng.uniform(0.5, 40, (P, n))
    o_all, lse_all = oracle_lib.merge(a, m, l)
    o12, lse12 = oracle_lib.merge(a[:2], m[:2], l[:2])
    o_nested, lse_nested = oracle_lib.merge(np.stack([o12, a[2]]), np.stack([lse12, m[2]]),
                                            np.stack([np.ones(n), l[2]]))
    np.testing.assert_allclose(o_nested, o_all, atol=1e-12)
    np.testing.assert_allclose(lse_nested, lse_all, atol=1e-12)
    o1, lse1 = oracle_lib.merge(a[:1], m[:1], l[:1])
    np.testing.assert_allclose(o1, a[0], atol=1e-15)
    np.testing.assert_allclose(lse1, m[0] + np.log(l[0]), atol=1e-13)


def test_merge_empty_partitions(oracle_lib):
    a = np.ones((2, 3, 4))
    m = np.array([[-np.inf, 1.0, -np.inf], [-np.inf, -np.inf, 2.0]])
    l = np.array([[0.0, 2.0, 0.0], [0.0, 0.0, 3.0]])
    a[0, 1] = 5.0
    o, lse = oracle_lib.merge(a, m, l)
    assert np.all(o[0] == 0.0) and lse[0] == -np.inf
    np.testing.assert_allclose(o[1], 5.0)
    np.testing.assert_allclose(lse[1], 1.0 + math.log(2.0))
    np.testing.assert_allclose(o[2], 1.0)
    np.testing.assert_allclose(lse[2], 2.0 + math.log(3.0))


def test_merge_no_overflow_at_large_scores(oracle_lib):
    """[SUM] 3.4 Phase 2 Step 5: aggregation must not form e^{score}; e^800 overflows fp64."""
    a = np.stack([np.full((1, 2), 1.0), np.full((1, 2), 3.0)])
    m = np.array([[800.0], [800.0 + math.log(3.0)]])
    l = np.array([[1.0], [1.0]])
    o, lse = oracle_lib.merge(a, m, l)
    np.testing.assert_allclose(o, [[2.5, 2.5]], rtol=1e-14)
    np.testing.assert_allclose(lse, [800.0 + math.log(4.0)], rtol=1e-15)


def test_partial_causal_offset(oracle_lib):
    rng = np.random.default_rng(10)
    hq, hkv, R, T, d = 2, 2, 6, 15, 4
    q, k, v = _rand(rng, hq, R, d), _rand(rng, hkv, T, d), _rand(rng, hkv, T, d)
    lo, hi, off = 3, 12, 2
    a, m, l = oracle_lib.partial(q, k, v, lo, hi, off)
    vis = np.zeros((R, T), bool)
    vis[:, lo:hi] = (np.arange(lo, hi)[None, :] - lo) <= (np.arange(R)[:, None] + off)
    od, lsed = dense(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), vis)
    np.testing.assert_allclose(a, od, atol=1e-13)
    np.testing.assert_allclose(m + np.log(l), lsed, atol=1e-13)


# --------------------------------------------------------------------------------------
# Pin 7: Phase 2 query and decode rows are rows of global causal attention over the whole
# sequence [context ; query ; generated tokens], whatever the shard split.
# [SUM] 3.2 (the aggregate equals the single-device result), 3.4 Phase 2 Steps 3-5, 7.
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("bounds", [[0, 40], [0, 10, 20, 30, 40], [0, 3, 40], [0, 20, 20, 40]])
def test_phase2_equals_global_causal_rows(oracle_lib, bounds):
    rng = np.random.default_rng(11)
    hq, hkv, L, lq, T, d = 4, 2, 40, 5, 3, 8
    kc, vc = _rand(rng, hkv, L, d), _rand(rng, hkv, L, d)
    qq, kq, vq = _rand(rng, hq, lq, d), _rand(rng, hkv, lq, d), _rand(rng, hkv, lq, d)
    qd, kd, vd = _rand(rng, T, hq, d), _rand(rng, T, hkv, d), _rand(rng, T, hkv, d)
    k_all = np.concatenate([kc, kq, np.transpose(kd, (1, 0, 2))], axis=1).astype(np.float64)
    v_all = np.concatenate([vc, vq, np.transpose(vd, (1, 0, 2))], axis=1).astype(np.float64)
    N = L + lq + T
    q_rows = np.concatenate([qq, np.transpose(qd, (1, 0, 2))], axis=1).astype(np.float64)
    od, lsed = dense(q_rows, k_all, v_all, causal_mask(lq + T, N, offset=L))
    o, lse = oracle_lib.phase2_query(qq, kc, vc, bounds, kq, vq)
    np.testing.assert_allclose(o, od[:, :lq], atol=1e-12)
    np.testing.assert_allclose(lse, lsed[:, :lq], atol=1e-12)
    k_tail = np.concatenate([kq, np.transpose(kd, (1, 0, 2))], axis=1)
    v_tail = np.concatenate([vq, np.transpose(vd, (1, 0, 2))], axis=1)
    for t in range(T):
        ot, lset = oracle_lib.phase2_decode(qd[t], kc, vc, bounds, k_tail, v_tail, lq + t + 1)
        np.testing.assert_allclose(ot, od[:, lq + t], atol=1e-12)
        np.testing.assert_allclose(lset, lsed[:, lq + t], atol=1e-12)


# --------------------------------------------------------------------------------------
# Pin 8: locality.  Keys outside a row's visible set cannot change it (bitwise); the
# anchor changes every later block; permuting anchor tokens (K and V together) leaves
# later blocks unchanged up to rounding, since the anchor is fully visible to them.
# [SUM] 3.4 Phase 1 Steps 2, 4.
# --------------------------------------------------------------------------------------
def test_locality_and_anchor_effects(oracle_lib):
    rng = np.random.default_rng(12)
    hq, hkv, L, d, b, a = 2, 1, 36, 8, 12, 12
    q, k, v = _rand(rng, hq, L, d), _rand(rng, hkv, L, d), _rand(rng, hkv, L, d)
    o, lse = oracle_lib.phase1(q, k, v, b, a)
    # perturb keys of block 1 (tokens 12..23): rows of block 2 (24..35) must be bitwise unchanged
    k2, v2 = k.copy(), v.copy()
    k2[:, 12:24] += 1.0
    v2[:, 12:24] -= 2.0
    o2, lse2 = oracle_lib.phase1(q, k2, v2, b, a)
    assert np.array_equal(o2[:, 24:], o[:, 24:]) and np.array_equal(lse2[:, 24:], lse[:, 24:])
    assert np.array_equal(o2[:, :12], o[:, :12])
    # a future key inside the block does not affect earlier rows
    k3 = k.copy()
    k3[:, 30] += 5.0
    o3, _ = oracle_lib.phase1(q, k3, v, b, a)
    assert np.array_equal(o3[:, :30], o[:, :30]) and not np.array_equal(o3[:, 30:], o[:, 30:])
    # changing the anchor changes every later block
    k4 = k.copy()
    k4[:, 3] += 1.0
    _, lse4 = oracle_lib.phase1(q, k4, v, b, a)
    assert np.all(np.abs(lse4[:, 12:] - lse[:, 12:]) > 0)
    # permuting anchor tokens leaves later blocks unchanged up to rounding
    perm = rng.permutation(a)
    k5, v5 = k.copy(), v.copy()
    k5[:, :a] = k[:, perm]
    v5[:, :a] = v[:, perm]
    o5, lse5 = oracle_lib.phase1(q, k5, v5, b, a)
    np.testing.assert_allclose(o5[:, 12:], o[:, 12:], atol=1e-13)
    np.testing.assert_allclose(lse5[:, 12:], lse[:, 12:], atol=1e-13)


# --------------------------------------------------------------------------------------
# Pin 9: a planted needle makes the softmax sharply peaked: the aligned query's LSE is the
# needle score (to e^-gap) and its output is the needle's value row.  Scores near 90 make
# e^score overflow fp32, which the log-space aggregation must survive.
# --------------------------------------------------------------------------------------
def test_needle_peaked_softmax(oracle_lib):
    rng = np.random.default_rng(13)
    hq, hkv, L, d, lq = 4, 2, 256, 128, 2
    G = hq // hkv
    kc, vc = _rand(rng, hkv, L, d), _rand(rng, hkv, L, d)
    qq, kq, vq = _rand(rng, hq, lq, d), _rand(rng, hkv, lq, d), _rand(rng, hkv, lq, d)
    pos = [17, 200]
    for g in range(hkv):
        kc[g, pos[g]] = 8.0 * qq[g * G, 0]
    o, lse = oracle_lib.phase2_query(qq, kc, vc, [0, 64, 128, 192, 256], kq, vq)
    for g in range(hkv):
        h = g * G
        score = 8.0 * float(np.dot(qq[h, 0].astype(np.float64), qq[h, 0].astype(np.float64))) / math.sqrt(d)
        assert score > 60.0
        assert abs(lse[h, 0] - score) < 1e-6
        np.testing.assert_allclose(o[h, 0], vc[g, pos[g]].astype(np.float64), atol=1e-9)


# --------------------------------------------------------------------------------------
# GQA head mapping (a reading: contiguous groups, q head h uses kv head h // (Hq/Hkv)).
# --------------------------------------------------------------------------------------
def test_gqa_contiguous_groups(oracle_lib):
    rng = np.random.default_rng(14)
    hq, hkv, L, d, b = 8, 2, 20, 4, 20
    q, k, v = _rand(rng, hq, L, d), _rand(rng, hkv, L, d), _rand(rng, hkv, L, d)
    o, _ = oracle_lib.phase1(q, k, v, b, b)
    for h in range(hq):
        oh, _ = oracle_lib.phase1(q[h:h + 1], k[h // 4:h // 4 + 1], v[h // 4:h // 4 + 1], b, b)
        np.testing.assert_array_equal(o[h], oh[0])


def test_oracle_rejects_bad_arguments(oracle_lib):
    q = np.zeros((2, 8, 4), np.float32)
    k = np.zeros((1, 8, 4), np.float32)
    with pytest.raises(ValueError):
        oracle_lib.phase1(q, k, k, 4, 5)          # anchor > block
    with pytest.raises(ValueError):
        oracle_lib.phase1(q, k, k, 4, 4, rows=[8])  # row out of range
    with pytest.raises(ValueError):
        oracle_lib.partial(q, k, k, 3, 9)        # hi > tokens
