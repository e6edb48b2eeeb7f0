"""The profiling build (decode timestamps, libstarattn_timeline.so) computes exactly what the
product library computes: the same decode steps through both give bit-identical outputs, and
the timestamps it records are ordered as the launch runs (start <= stream end <= stores done <=
ticket for every workgroup)."""
import ctypes
import os

import numpy as np
import pytest
import torch

import block_sparse_long_phase1_amd as sa
from block_sparse_long_phase1_amd import build as sa_build
from block_sparse_long_phase1_amd import inputs as sin
from block_sparse_long_phase1_amd.configs import StarConfig
from tests._parity import flush_print

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 128), (4, 1, 64)])
def test_timeline_build_matches_product_library(hq, hkv, d):
    flush_print("timeline build", hq, hkv, d)
    if not os.path.exists(sa_build.TIMELINE_LIB_PATH):
        pytest.fail("libstarattn_timeline.so is missing: build the package first")
    cfg = StarConfig("tl", hq=hq, hkv=hkv, d=d, L=3000, block=3000, anchor=3000, lq=7, decode_steps=2,
                     shards=3, dtype="bf16", needle=False, seed=97)
    _, k, v = sin.phase1_inputs(cfg, DEV)
    p2 = sin.phase2_inputs(cfg, DEV)
    bounds = [0, 1000, 1001, 3000]
    timeline = sa.load_library(sa_build.TIMELINE_LIB_PATH)
    timeline.star_decode_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    timeline.star_decode_timeline_read.restype = ctypes.c_int
    outs = {}
    try:
        for name, path in (("product", sa_build.LIB_PATH), ("timeline", sa_build.TIMELINE_LIB_PATH)):
            sa.load_library(path, make_default=True)
            k_tail = torch.zeros((hkv, cfg.lq + 2, d), dtype=torch.bfloat16, device=DEV)
            v_tail = torch.zeros_like(k_tail)
            k_tail[:, :cfg.lq] = p2["k_qry"]
            v_tail[:, :cfg.lq] = p2["v_qry"]
            ws = sa.decode_workspace(cfg.L, cfg.lq + 2, 3, hq, hkv, d, DEV)
            res = []
            for t in range(2):
                o, lse = sa.star_decode_step(p2["q_dec"][t], p2["k_dec"][t], p2["v_dec"][t], k, v, bounds, k_tail,
                                             v_tail, cfg.lq + t, workspace=ws)
                res.append((o.clone(), lse.clone()))
            torch.cuda.synchronize()
            outs[name] = res
    finally:
        sa.load_library(sa_build.LIB_PATH, make_default=True)   # the product library again
    for (o0, l0), (o1, l1) in zip(outs["product"], outs["timeline"]):
        assert torch.equal(o0, o1) and torch.equal(l0, l1)
    buf = np.zeros((4096, 8), dtype=np.uint64)
    assert timeline.star_decode_timeline_read(buf.ctypes.data, buf.nbytes) == 0
    grid = int((buf[:, 0] > 0).sum())
    assert grid > 0
    t = buf[:grid].astype(np.int64)
    assert (t[:, 1] >= t[:, 0]).all()
    if hq // hkv <= 4:   # the in-kernel merge: stores and tickets are timed too
        assert (t[:, 2] >= t[:, 1]).all() and (t[:, 3] >= t[:, 2]).all()
