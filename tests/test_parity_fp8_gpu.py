"""GPU parity of the E4M3 context cache: scales and codes bit-exact against the oracle, and
the query phase and the decode step over an E4M3 context (codes and scales made by the
oracle) against the oracle's over the dequantised values."""
import numpy as np
import pytest
import torch

import block_sparse_long_phase1_amd as sa
import oracle
from oracle import kv_fp8 as of8
from block_sparse_long_phase1_amd import inputs as sin
from block_sparse_long_phase1_amd.configs import CONFIGS, StarConfig, shard_bounds
from tests._parity import assert_lse, assert_out, flush_print

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _cfg(hq, hkv, L, b, d=128, dtype="bf16", lq=16, T=3, S=2, seed=71):
    return StarConfig("test", hq=hq, hkv=hkv, d=d, L=L, block=b, anchor=b, lq=lq, decode_steps=T,
                      shards=S, dtype=dtype, needle=False, seed=seed)


def _oracle_cache(k, v):
    """Scales and E4M3 codes of k, v [Hkv, L, d] made by the oracle, on the device."""
    ks, vs = of8.kv_absmax_scales(k.cpu()), of8.kv_absmax_scales(v.cpu())
    k8 = np.stack([of8.kv_quantize(k[g:g + 1].cpu(), ks[g:g + 1])[0] for g in range(k.shape[0])])
    v8 = np.stack([of8.kv_quantize(v[g:g + 1].cpu(), vs[g:g + 1])[0] for g in range(v.shape[0])])
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return to(k8), to(v8), to(ks), to(vs), (k8, v8, ks, vs)


@pytest.mark.parametrize("hkv,L,d,dtype", [(3, 1000, 128, "bf16"), (2, 777, 64, "bf16"), (3, 300, 64, "f32"),
                                           (1, 1, 8, "f32")])
def test_scales_and_codes_bit_exact(hkv, L, d, dtype):
    flush_print("kv fp8 codes", hkv, L, d, dtype)
    cfg = _cfg(hkv, hkv, L, L, d=d, dtype=dtype, seed=73)
    x = sin.randn(cfg, "k_ctx", (hkv, L, d), DEV) * 3.0
    if hkv == 3:
        x[1].zero_()                     # an all-zero head takes scale 1
    s = sa.star_kv_fp8_scales(x)
    c = sa.star_kv_quantize_fp8(x, s)
    torch.cuda.synchronize()
    rs = of8.kv_absmax_scales(x.cpu())
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32)), (s.cpu().numpy(), rs)
    rc = of8.kv_quantize(x.cpu(), rs)
    got = c.cpu().numpy()
    bad = np.argwhere(got != rc)
    assert bad.size == 0, "%d codes differ, first at %s: %s vs %s" % (
        len(bad), bad[0], got[tuple(bad[0])], rc[tuple(bad[0])])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_codes_at_format_edges(dtype):
    """Every finite E4M3 value, every midpoint between neighbours (exact ties), the fp32
    neighbours of each midpoint, saturation, infinities, NaN and signed zeros, with scale 1."""
    mags = of8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (mags[:-1] + mags[1:]) / 2
    vals = [mags, mids, [448.0, 450.0, 464.0, 500.0, 2.0 ** 100, np.inf, 2.0 ** -11, 2.0 ** -10, 3 * 2.0 ** -10]]
    if dtype == "f32":
        m32 = mids.astype(np.float32)
        vals += [np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9))]
    x = np.concatenate([np.asarray(v, np.float64) for v in vals]).astype(np.float32)
    x = np.concatenate([x, -x, np.float32([np.nan, -np.nan, 0.0, -0.0])])
    x = np.concatenate([x, np.zeros((-x.size) % 8, np.float32)]).reshape(1, -1, 8)
    t = torch.from_numpy(x)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
        assert np.array_equal(t.float().numpy()[np.isfinite(x)], x[np.isfinite(x)])   # all exact in bf16
    t = t.to(DEV)
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    c = sa.star_kv_quantize_fp8(t, one)
    torch.cuda.synchronize()
    rc = of8.kv_quantize(t.cpu(), np.float32([1.0]))
    got = c.cpu().numpy()
    bad = np.argwhere(got != rc)
    assert bad.size == 0, [(float(x[tuple(i)]), hex(got[tuple(i)]), hex(rc[tuple(i)])) for i in bad[:8]]


def _scales_both_sides_of_the_fast_range():
    """Scales for the quantiser tests: max / 448 of seeded bf16 maxima, seeded fp32 scales
    over 2^-120 .. 2^120, and fixed ones at and just past 2^-90 and 2^90 (the ends of the
    kernel's reciprocal path; outside it divides), 1, 3, the smallest normal and subnormal
    and the largest finite fp32."""
    rng = np.random.default_rng(97)
    maxima = (rng.integers(1, 0x7F80, size=96).astype(np.uint32) << 16).view(np.float32)
    from_bf16 = (maxima / np.float32(448.0)).astype(np.float32)
    rand = np.exp2(rng.uniform(-120, 120, size=32)).astype(np.float32)
    lo, hi = np.float32(2.0 ** -90), np.float32(2.0 ** 90)
    fixed = np.float32([1.0, 3.0, lo, np.nextafter(lo, np.float32(0)), hi, np.nextafter(hi, np.float32(np.inf)),
                        2.0 ** -126, np.float32(2.0 ** -149), np.finfo(np.float32).max])
    return np.concatenate([from_bf16, rand, fixed]).astype(np.float32)


def test_codes_every_bf16_value_under_many_scales():
    """Every bf16 bit pattern (finite, infinite, NaN, both signs) quantised under each scale of
    the set above: codes bit-exact against the oracle's."""
    sc = _scales_both_sides_of_the_fast_range()
    flush_print("kv fp8 every bf16 value", len(sc), "scales")
    pats = np.arange(1 << 16, dtype=np.uint16).view(np.int16).reshape(1, -1, 8)
    x = torch.from_numpy(np.repeat(pats, len(sc), axis=0)).view(torch.bfloat16)
    c = sa.star_kv_quantize_fp8(x.to(DEV), torch.from_numpy(sc).to(DEV))
    torch.cuda.synchronize()
    rc = of8.kv_quantize(x, sc)
    got = c.cpu().numpy()
    bad = np.argwhere(got != rc)
    assert bad.size == 0, "%d codes differ: %s" % (len(bad), [
        (hex(int(pats.reshape(-1)[i[1] * 8 + i[2]]) & 0xFFFF), float(sc[i[0]]), hex(got[tuple(i)]), hex(rc[tuple(i)]))
        for i in bad[:8]])


def test_codes_fp32_around_every_midpoint_under_many_scales():
    """fp32 values x = RN(t * scale) for every E4M3 value and every midpoint between neighbours
    t, moved by -4 .. +4 ulps, both signs, plus zeros, infinities, NaN and values far past the
    range, under each scale of the set above: codes bit-exact against the oracle's."""
    sc = _scales_both_sides_of_the_fast_range()
    flush_print("kv fp8 fp32 midpoints", len(sc), "scales")
    mags = of8.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    t = np.concatenate([mags, (mags[:-1] + mags[1:]) / 2, [464.0, 1e3, 2.0 ** -10, 2.0 ** -11]])
    rows = []
    for s in sc:
        base = (t * np.float64(s)).astype(np.float32)
        near = (base.view(np.int32)[:, None] + np.arange(-4, 5, dtype=np.int32)[None, :]).reshape(-1)
        v = near.view(np.float32)
        v = v[np.isfinite(v) & (near >= 0)]
        extra = np.float32([0.0, np.inf, np.nan, np.finfo(np.float32).max, 1e-45])
        rows.append(np.concatenate([v, -v, extra, -extra]))
    n = max(len(r) for r in rows)
    n += (-n) % 8
    x = np.zeros((len(sc), n), np.float32)
    for g, r in enumerate(rows):
        x[g, :len(r)] = r
    x = x.reshape(len(sc), -1, 8)
    c = sa.star_kv_quantize_fp8(torch.from_numpy(x).to(DEV), torch.from_numpy(sc).to(DEV))
    torch.cuda.synchronize()
    rc = of8.kv_quantize(x, sc)
    got = c.cpu().numpy()
    bad = np.argwhere(got != rc)
    assert bad.size == 0, "%d codes differ: %s" % (len(bad), [
        (float(x[tuple(i)]), float(sc[i[0]]), hex(got[tuple(i)]), hex(rc[tuple(i)])) for i in bad[:8]])


@pytest.mark.parametrize("hq,hkv,L,bounds,lq,T,d", [
    (8, 2, 3000, [0, 800, 1600, 3000], 40, 3, 128),         # G = 4, ragged shards
    (16, 1, 2333, [0, 700, 700, 2333], 5, 3, 64),           # d = 64, G = 16, an empty shard
    (4, 4, 777, [0, 777], 1, 2, 128),                        # G = 1, one cached query token
    (16, 2, 1500, [0, 512, 1024, 1500], 20, 2, 128),        # G = 8
    (4, 2, 600, [0, 100, 600], 0, 2, 64),                    # G = 2, first token is the first cached one
])
def test_decode_kv8(hq, hkv, L, bounds, lq, T, d):
    flush_print("decode kv8", hq, hkv, L, bounds, lq, T, d)
    cfg = _cfg(hq, hkv, L, L, d=d, lq=max(lq, 1), T=T, S=len(bounds) - 1, seed=79)
    q, k, v = sin.phase1_inputs(cfg, DEV)
    p2 = sin.phase2_inputs(cfg, DEV)
    k8, v8, ks, vs, (hk8, hv8, hks, hvs) = _oracle_cache(k, v)
    k_tail = torch.zeros((hkv, lq + T, d), dtype=torch.bfloat16, device=DEV)
    v_tail = torch.zeros_like(k_tail)
    k_tail[:, :lq] = p2["k_qry"][:, :lq]
    v_tail[:, :lq] = p2["v_qry"][:, :lq]
    ws = sa.decode_workspace(L, lq + T, len(bounds) - 1, hq, hkv, d, DEV)
    for t in range(T):
        o, lse = sa.star_decode_step_kv8(p2["q_dec"][t], p2["k_dec"][t], p2["v_dec"][t], k8, v8, ks, vs, bounds,
                                         k_tail, v_tail, lq + t, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(k_tail[:, lq + t], p2["k_dec"][t]) and torch.equal(v_tail[:, lq + t], p2["v_dec"][t])
        ro, rl = of8.phase2_decode_kv8(p2["q_dec"][t].cpu(), hk8, hv8, hks, hvs, bounds, k_tail.cpu(),
                                       v_tail.cpu(), lq + t + 1)
        assert_out(o, ro, "kv8 decode O step %d" % t)
        assert_lse(lse, rl, "kv8 decode LSE step %d" % t)


@pytest.mark.parametrize("G,d", [(4, 128), (2, 64)])
def test_decode_kv8_merge_over_many_chunks(G, d):
    """The E4M3 decode step with one kv head and 159 chunks (shards of 7000, 1 and 12999
    tokens, 128-key chunks, plus the query host's): the merging workgroup folds three batches
    of partials, the last one ragged."""
    hq, hkv, L, lq, T = G, 1, 20000, 5, 1
    flush_print("decode kv8 many chunks", G, d)
    cfg = _cfg(hq, hkv, L, L, d=d, lq=lq, T=T, S=3, seed=89)
    _, k, v = sin.phase1_inputs(cfg, DEV)
    p2 = sin.phase2_inputs(cfg, DEV)
    k8, v8, ks, vs, (hk8, hv8, hks, hvs) = _oracle_cache(k, v)
    bounds = [0, 7000, 7001, 20000]
    k_tail = torch.zeros((hkv, lq + T, d), dtype=torch.bfloat16, device=DEV)
    v_tail = torch.zeros_like(k_tail)
    k_tail[:, :lq] = p2["k_qry"]
    v_tail[:, :lq] = p2["v_qry"]
    ws = sa.decode_workspace(L, lq + T, len(bounds) - 1, hq, hkv, d, DEV)
    o, lse = sa.star_decode_step_kv8(p2["q_dec"][0], p2["k_dec"][0], p2["v_dec"][0], k8, v8, ks, vs, bounds,
                                     k_tail, v_tail, lq, workspace=ws)
    torch.cuda.synchronize()
    ro, rl = of8.phase2_decode_kv8(p2["q_dec"][0].cpu(), hk8, hv8, hks, hvs, bounds, k_tail.cpu(), v_tail.cpu(),
                                   lq + 1)
    assert_out(o, ro, "kv8 decode O")
    assert_lse(lse, rl, "kv8 decode LSE")


def test_decode_kv8_equals_bf16_decode_on_representable_values():
    """With unit scales and a context whose bf16 values are E4M3 values, the E4M3 decode step
    and the bf16 decode step compute the same numbers: their outputs are bit-identical."""
    cfg = _cfg(8, 2, 2000, 2000, lq=8, T=1, S=2, seed=83)
    _, k, v = sin.phase1_inputs(cfg, DEV)
    p2 = sin.phase2_inputs(cfg, DEV)
    one = np.float32([1.0, 1.0])
    hk8 = of8.kv_quantize(k.cpu(), one)
    hv8 = of8.kv_quantize(v.cpu(), one)
    kr = torch.from_numpy(of8.e4m3_decode(hk8).astype(np.float32)).to(torch.bfloat16).to(DEV)
    vr = torch.from_numpy(of8.e4m3_decode(hv8).astype(np.float32)).to(torch.bfloat16).to(DEV)
    bounds = [0, 900, 2000]
    outs = []
    for kv8 in (False, True):
        kt = torch.zeros((2, 9, 128), dtype=torch.bfloat16, device=DEV)
        vt = torch.zeros_like(kt)
        kt[:, :8] = p2["k_qry"]
        vt[:, :8] = p2["v_qry"]
        if kv8:
            ones = torch.ones(2, dtype=torch.float32, device=DEV)
            o, l = sa.star_decode_step_kv8(p2["q_dec"][0], p2["k_dec"][0], p2["v_dec"][0],
                                           torch.from_numpy(hk8).to(DEV), torch.from_numpy(hv8).to(DEV), ones, ones,
                                           bounds, kt, vt, 8)
        else:
            o, l = sa.star_decode_step(p2["q_dec"][0], p2["k_dec"][0], p2["v_dec"][0], kr, vr, bounds, kt, vt, 8)
        outs.append((o, l))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("hq,hkv,L,bounds,rows,tail_len,tail_cap,d", [
    (8, 2, 3000, [0, 800, 1600, 3000], 40, 40, 48, 128),             # G = 4, ragged shards
    (16, 1, 2333, [0, 700, 700, 2333], 9, 30, 33, 64),               # d = 64, G = 16, an empty shard
    (4, 4, 777, [0, 777], 1, 1, 1, 128),                              # G = 1, one row, one cached token
    (16, 2, 1500, [0, 512, 1024, 1500], 20, 20, 24, 128),             # G = 8
    (8, 1, 6000, [0, 1500, 3000, 4500, 6000], 300, 300, 310, 128),    # several row tiles and key splits
    (4, 2, 100, [0, 37, 100], 70, 70, 70, 64),                        # context shorter than two tiles
])
def test_query_kv8(hq, hkv, L, bounds, rows, tail_len, tail_cap, d):
    """The query phase over an E4M3 context cache (oracle-made codes and scales) against the
    oracle's query phase over the dequantised context; the query host's cache is bf16."""
    flush_print("query kv8", hq, hkv, L, bounds, rows, tail_len, d)
    cfg = _cfg(hq, hkv, L, L, d=d, lq=tail_len, T=1, S=len(bounds) - 1, seed=89)
    q, k, v = sin.phase1_inputs(cfg, DEV)
    p2 = sin.phase2_inputs(cfg, DEV)
    k8, v8, ks, vs, (hk8, hv8, hks, hvs) = _oracle_cache(k, v)
    qr = p2["q_qry"][:, tail_len - rows:].contiguous()
    k_tail = torch.zeros((hkv, tail_cap, d), dtype=torch.bfloat16, device=DEV)
    v_tail = torch.zeros_like(k_tail)
    k_tail[:, :tail_len] = p2["k_qry"]
    v_tail[:, :tail_len] = p2["v_qry"]
    o, lse = sa.star_phase2_query_kv8(qr, k8, v8, ks, vs, bounds, k_tail, v_tail, tail_len)
    torch.cuda.synchronize()
    ro, rl = of8.phase2_query_kv8(qr.cpu(), hk8, hv8, hks, hvs, bounds, k_tail.cpu(), v_tail.cpu(), tail_len)
    assert_out(o, ro, "kv8 query O")
    assert_lse(lse, rl, "kv8 query LSE")


@pytest.mark.parametrize("hq,hkv,T,lo,hi,rows,off,d", [
    (8, 2, 3000, 0, 3000, 40, -1, 128),          # the whole cache, no mask
    (16, 1, 2333, 700, 2333, 9, -1, 64),         # a shard view of a bigger cache, d = 64, G = 16
    (4, 2, 600, 100, 420, 70, 250, 128),         # causal offset: row i sees partition tokens <= 250 + i
    (8, 2, 20000, 2000, 20000, 16, -1, 128),     # several key splits, merged into one partial
    (4, 4, 300, 150, 150, 5, -1, 128),           # an empty partition
])
def test_partial_kv8(hq, hkv, T, lo, hi, rows, off, d):
    """One partition of oracle-made E4M3 codes against the oracle's partial over the
    dequantised values: A, the log-sum-exp m + log l, and m itself."""
    flush_print("partial kv8", hq, hkv, T, lo, hi, rows, off, d)
    cfg = _cfg(hq, hkv, T, T, d=d, seed=101)
    q = sin.randn(cfg, "q_qry", (hq, rows, d), DEV)
    k = sin.randn(cfg, "k_ctx", (hkv, T, d), DEV)
    v = sin.randn(cfg, "v_ctx", (hkv, T, d), DEV)
    k8, v8, ks, vs, (hk8, hv8, hks, hvs) = _oracle_cache(k, v)
    a, m, l = sa.star_phase2_partial_kv8(q, k8[:, lo:], v8[:, lo:], ks, vs, T * d, hi - lo, off)
    torch.cuda.synchronize()
    if hi == lo:
        assert torch.all(a == 0) and torch.all(torch.isneginf(m)) and torch.all(l == 0)
        return
    ra, rm, rl = of8.partial_kv8(q.cpu(), hk8, hv8, hks, hvs, lo, hi, off)
    assert_out(a, ra, "kv8 partial A")
    assert_lse(m + torch.log(l), rm + np.log(rl), "kv8 partial LSE")
    assert_lse(m, rm, "kv8 partial m")


@pytest.mark.parametrize("d", [128, 64])
def test_query_kv8_equals_bf16_query_on_representable_values(d):
    """With unit scales and a context whose bf16 values are E4M3 values, the E4M3 query phase
    and the bf16 query phase compute the same numbers: bit-identical outputs."""
    cfg = _cfg(8, 2, 2000, 2000, d=d, lq=24, T=1, S=2, seed=97)
    _, k, v = sin.phase1_inputs(cfg, DEV)
    p2 = sin.phase2_inputs(cfg, DEV)
    one = np.float32([1.0, 1.0])
    hk8 = of8.kv_quantize(k.cpu(), one)
    hv8 = of8.kv_quantize(v.cpu(), one)
    kr = torch.from_numpy(of8.e4m3_decode(hk8).astype(np.float32)).to(torch.bfloat16).to(DEV)
    vr = torch.from_numpy(of8.e4m3_decode(hv8).astype(np.float32)).to(torch.bfloat16).to(DEV)
    ones = torch.ones(2, dtype=torch.float32, device=DEV)
    bounds = [0, 900, 2000]
    k_tail, v_tail = p2["k_qry"].contiguous(), p2["v_qry"].contiguous()
    o8, l8 = sa.star_phase2_query_kv8(p2["q_qry"], torch.from_numpy(hk8).to(DEV), torch.from_numpy(hv8).to(DEV),
                                      ones, ones, bounds, k_tail, v_tail, 24)
    ob, lb = sa.star_phase2_query(p2["q_qry"], kr, vr, bounds, k_tail, v_tail, 24)
    torch.cuda.synchronize()
    assert torch.equal(o8, ob) and torch.equal(l8, lb)


def test_quantize_and_kv8_decode_replayed_from_a_hip_graph():
    """The scales, the quantisation of K and V, the query phase and T decode steps over the
    E4M3 cache, captured in one HIP graph (the library allocates nothing and records no
    memsets), replay bit-identically to the eager calls, with eager work between the replays."""
    cfg = _cfg(8, 2, 3000, 3000, lq=16, T=3, S=3, seed=89)
    q, k, v = sin.phase1_inputs(cfg, DEV)
    p2 = sin.phase2_inputs(cfg, DEV)
    bounds = [0, 1000, 2000, 3000]
    T, lq, cap, d = cfg.decode_steps, cfg.lq, cfg.tail_cap, cfg.d

    def buffers():
        kt = torch.zeros((cfg.hkv, cap, d), dtype=torch.bfloat16, device=DEV)
        vt = torch.zeros_like(kt)
        kt[:, :lq] = p2["k_qry"]
        vt[:, :lq] = p2["v_qry"]
        return dict(ks=torch.empty(cfg.hkv, dtype=torch.float32, device=DEV),
                    vs=torch.empty(cfg.hkv, dtype=torch.float32, device=DEV),
                    k8=torch.empty(k.shape, dtype=torch.uint8, device=DEV),
                    v8=torch.empty(v.shape, dtype=torch.uint8, device=DEV), kt=kt, vt=vt,
                    ws=sa.decode_workspace(cfg.L, cap, 3, cfg.hq, cfg.hkv, d, DEV),
                    wq=torch.empty(max(16, sa.star_phase2_query_workspace_bytes(lq, 3, cfg.hq, cfg.hkv, d)),
                                   dtype=torch.uint8, device=DEV),
                    oq=torch.empty((cfg.hq, lq, d), dtype=torch.bfloat16, device=DEV),
                    lq=torch.empty((cfg.hq, lq), dtype=torch.float32, device=DEV),
                    o=[torch.empty((cfg.hq, d), dtype=torch.bfloat16, device=DEV) for _ in range(T)],
                    l=[torch.empty((cfg.hq,), dtype=torch.float32, device=DEV) for _ in range(T)])

    def run(b):
        sa.star_kv_fp8_scales(k, b["ks"])
        sa.star_kv_quantize_fp8(k, b["ks"], b["k8"])
        sa.star_kv_fp8_scales(v, b["vs"])
        sa.star_kv_quantize_fp8(v, b["vs"], b["v8"])
        sa.star_phase2_query_kv8(p2["q_qry"], b["k8"], b["v8"], b["ks"], b["vs"], bounds, b["kt"], b["vt"], lq,
                                 o=b["oq"], lse=b["lq"], workspace=b["wq"])
        for t in range(T):
            sa.star_decode_step_kv8(p2["q_dec"][t], p2["k_dec"][t], p2["v_dec"][t], b["k8"], b["v8"], b["ks"], b["vs"],
                                    bounds, b["kt"], b["vt"], lq + t, o=b["o"][t], lse=b["l"][t], workspace=b["ws"])

    eager = buffers()
    run(eager)
    g = buffers()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(g)
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for name in ("ks", "vs", "k8", "v8", "kt", "vt", "oq", "lq"):
            assert torch.equal(g[name], eager[name]), "replay %d: %s differs" % (rep, name)
        for t in range(T):
            assert torch.equal(g["o"][t], eager["o"][t]), "replay %d step %d: O differs" % (rep, t)
            assert torch.equal(g["l"][t], eager["l"][t]), "replay %d step %d: LSE differs" % (rep, t)
        # unrelated eager work between replays, and outputs cleared
        sa.star_phase1_encode(q, k, v, cfg.block, cfg.anchor)
        for name in ("ks", "vs", "k8", "v8", "oq", "lq"):
            g[name].zero_()
        for t in range(T):
            g["o"][t].zero_()
            g["l"][t].zero_()
        torch.cuda.synchronize()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["8b_32k", "8b_128k_needle"])
def test_decode_kv8_full(name):
    """A workload at full size (8b_32k: Hq=32, Hkv=8, d=128, L=32768, 4 shards; 8b_128k_needle:
    L=131072 with a planted needle key per kv head): the GPU's scales and codes of the whole
    context equal the oracle's, and the first and last of T decode steps over the oracle-made
    E4M3 cache match the oracle."""
    cfg = CONFIGS[name]
    flush_print("kv8 full", cfg.name)
    x = sin.all_inputs(cfg, DEV)
    k, v = x["k_ctx"], x["v_ctx"]
    bounds = cfg.bounds()
    k8, v8, ks, vs, (hk8, hv8, hks, hvs) = _oracle_cache(k, v)
    flush_print("  oracle cache made")
    gks = sa.star_kv_fp8_scales(k)
    gk8 = sa.star_kv_quantize_fp8(k, gks)
    gvs = sa.star_kv_fp8_scales(v)
    gv8 = sa.star_kv_quantize_fp8(v, gvs)
    torch.cuda.synchronize()
    assert torch.equal(gks, ks) and torch.equal(gvs, vs)
    assert torch.equal(gk8, k8) and torch.equal(gv8, v8)
    del gk8, gv8
    k_tail = torch.zeros((cfg.hkv, cfg.tail_cap, cfg.d), dtype=torch.bfloat16, device=DEV)
    v_tail = torch.zeros_like(k_tail)
    k_tail[:, :cfg.lq] = x["k_qry"]
    v_tail[:, :cfg.lq] = x["v_qry"]
    # the query phase over the E4M3 cache, checked on its first and last 16 rows: the first
    # rows see a cache of 16 tokens, the last ones the whole query
    oq, lq_lse = sa.star_phase2_query_kv8(x["q_qry"], k8, v8, ks, vs, bounds, k_tail, v_tail, cfg.lq)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(lq_lse).all())
    kt, vt = k_tail.cpu(), v_tail.cpu()
    for lo, tl in ((0, 16), (cfg.lq - 16, cfg.lq)):
        ro, rl = of8.phase2_query_kv8(x["q_qry"][:, lo:lo + 16].cpu(), hk8, hv8, hks, hvs, bounds, kt, vt, tl)
        assert_out(oq[:, lo:lo + 16], ro, "%s kv8 query rows %d.. O" % (name, lo))
        assert_lse(lq_lse[:, lo:lo + 16], rl, "%s kv8 query rows %d.. LSE" % (name, lo))
    flush_print("  kv8 query ok")
    T = cfg.decode_steps
    ws = sa.decode_workspace(cfg.L, cfg.tail_cap, cfg.shards, cfg.hq, cfg.hkv, cfg.d, DEV)
    od = torch.empty((T, cfg.hq, cfg.d), dtype=torch.bfloat16, device=DEV)
    ld = torch.empty((T, cfg.hq), dtype=torch.float32, device=DEV)
    for t in range(T):
        sa.star_decode_step_kv8(x["q_dec"][t], x["k_dec"][t], x["v_dec"][t], k8, v8, ks, vs, bounds, k_tail, v_tail,
                                cfg.lq + t, o=od[t], lse=ld[t], workspace=ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(ld).all())
    kt, vt = k_tail.cpu(), v_tail.cpu()
    for t in (0, T - 1):
        ro, rl = of8.phase2_decode_kv8(x["q_dec"][t].cpu(), hk8, hv8, hks, hvs, bounds, kt, vt, cfg.lq + t + 1)
        assert_out(od[t], ro, "%s kv8 decode step %d O" % (name, t))
        assert_lse(ld[t], rl, "%s kv8 decode step %d LSE" % (name, t))
    flush_print("  kv8 decode ok")
