"""star_decode_step_noalloc (chunk partials in the library's static device scratch) against
star_decode_step (the same kernels with a caller workspace), through the C ABI.

Two calls in a row on one GPU, the second on a smaller input, so the second call reuses the
scratch the first one left behind; then a shape whose q heads per kv head take the second
(merge) launch.  Outputs, LSEs and the appended cache rows must be bit-identical to the
workspace entry point's, and both within the oracle tolerances.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_phase1_amd as sa
import oracle
from block_sparse_long_phase1_amd import inputs as sin
from block_sparse_long_phase1_amd.configs import StarConfig
from tests._parity import assert_lse, assert_out, flush_print

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(cfg):
    q, k, v = sin.phase1_inputs(cfg, DEV)
    p2 = sin.phase2_inputs(cfg, DEV)
    bounds = cfg.bounds()
    tails = []
    for _ in range(2):
        kt = torch.zeros((cfg.hkv, cfg.tail_cap, cfg.d), dtype=q.dtype, device=DEV)
        vt = torch.zeros_like(kt)
        kt[:, :cfg.lq] = p2["k_qry"]
        vt[:, :cfg.lq] = p2["v_qry"]
        tails.append((kt, vt))
    return k, v, p2, bounds, tails


def _run_pair(cfg):
    flush_print("noalloc", cfg.name, "hq", cfg.hq, "hkv", cfg.hkv, "L", cfg.L, "shards", cfg.shards)
    k, v, p2, bounds, ((kt_a, vt_a), (kt_b, vt_b)) = _case(cfg)
    ws = sa.decode_workspace(cfg.L, cfg.tail_cap, len(bounds) - 1, cfg.hq, cfg.hkv, cfg.d, DEV)
    T = cfg.decode_steps
    o_ref = torch.empty((T, cfg.hq, cfg.d), dtype=k.dtype, device=DEV)
    l_ref = torch.empty((T, cfg.hq), dtype=torch.float32, device=DEV)
    o_na = torch.full_like(o_ref, float("nan"))
    l_na = torch.full_like(l_ref, float("nan"))
    for t in range(T):
        args = (p2["q_dec"][t], p2["k_dec"][t], p2["v_dec"][t], k, v, bounds)
        sa.star_decode_step(*args, kt_a, vt_a, cfg.lq + t, o=o_ref[t], lse=l_ref[t], workspace=ws)
        sa.star_decode_step_noalloc(*args, kt_b, vt_b, cfg.lq + t, o=o_na[t], lse=l_na[t])
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ref), "%s: outputs differ from star_decode_step" % cfg.name
    assert torch.equal(l_na, l_ref), "%s: LSEs differ from star_decode_step" % cfg.name
    assert torch.equal(kt_b, kt_a) and torch.equal(vt_b, vt_a), "%s: appended cache rows differ" % cfg.name
    kh, vh, kt, vt = k.cpu(), v.cpu(), kt_b.cpu(), vt_b.cpu()
    for t in sorted({0, T - 1}):
        ro, rl = oracle.phase2_decode(p2["q_dec"][t].cpu(), kh, vh, bounds, kt, vt, cfg.lq + t + 1)
        assert_out(o_na[t], ro, "%s noalloc decode step %d O" % (cfg.name, t))
        assert_lse(l_na[t], rl, "%s noalloc decode step %d LSE" % (cfg.name, t))
    flush_print("  ok")


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    big = StarConfig("noalloc_big", hq=32, hkv=8, d=128, L=32768, block=8192, anchor=8192, lq=64,
                     decode_steps=3, shards=4, dtype="bf16", seed=811)
    small = StarConfig("noalloc_small", hq=8, hkv=2, d=128, L=3000, block=1000, anchor=1000, lq=16,
                       decode_steps=2, shards=3, dtype="bf16", seed=812)
    _run_pair(big)
    _run_pair(small)


def test_noalloc_with_a_merge_launch_and_head_dim_64():
    # G = 8 runs the decode kernel without its in-kernel merge, then merge_kernel
    cfg = StarConfig("noalloc_g8_d64", hq=16, hkv=2, d=64, L=5000, block=2500, anchor=2500, lq=8,
                     decode_steps=2, shards=2, dtype="bf16", seed=813)
    _run_pair(cfg)


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """A shape whose chunk partials exceed the static scratch is refused before any launch."""
    cfg = StarConfig("noalloc_too_big", hq=1024, hkv=64, d=128, L=4096, block=4096, anchor=4096, lq=4,
                     decode_steps=1, shards=64, dtype="bf16", seed=814)
    need = sa.star_decode_workspace_bytes(cfg.L, cfg.tail_cap, 64, cfg.hq, cfg.hkv, cfg.d)
    assert need > (8 << 20)
    q = torch.zeros((cfg.hq, cfg.d), dtype=torch.bfloat16, device=DEV)
    kn = torch.zeros((cfg.hkv, cfg.d), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((cfg.hkv, cfg.L, cfg.d), dtype=torch.bfloat16, device=DEV)
    kt = torch.zeros((cfg.hkv, cfg.tail_cap, cfg.d), dtype=torch.bfloat16, device=DEV)
    o = torch.empty((cfg.hq, cfg.d), dtype=torch.bfloat16, device=DEV)
    bounds = list(np.linspace(0, cfg.L, 65).astype(np.int64))
    with pytest.raises(sa.StarError, match="static scratch"):
        sa.star_decode_step_noalloc(q, kn, kn, kc, kc, bounds, kt, kt.clone(), 0, o=o)
