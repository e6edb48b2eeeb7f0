"""Host-side plan: block count, shard bounds, Phase-2 message size (CPU only)."""
import json
import os

import pytest

from block_sparse_long_phase1_amd.configs import (CONFIGS, n_blocks, shard_bounds,
                                                  star_comm_elements_per_token)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "plan_cases.json")


def test_block_counts_from_pages():
    cases = json.load(open(GOLDEN))
    for c in cases["n_blocks"]:
        assert n_blocks(c["L"], c["block"]) == c["n"], c["cite"]
    cm = cases["comm_elements_per_token_head_layer"]
    assert star_comm_elements_per_token(cm["d"]) == cm["elements"]


@pytest.mark.parametrize("L,b,S", [(32768, 8192, 4), (131072, 16384, 8), (1000, 300, 3), (1000, 300, 8),
                                   (2048, 512, 2), (100, 100, 1), (7, 3, 5)])
def test_shard_bounds_cover_context_with_whole_blocks(L, b, S):
    bd = shard_bounds(L, b, S)
    assert len(bd) == S + 1 and bd[0] == 0 and bd[-1] == L
    assert all(x <= y for x, y in zip(bd, bd[1:]))
    for x in bd[1:-1]:
        assert x % b == 0 or x == L          # shards are groups of whole blocks
    n = n_blocks(L, b)
    sizes = [(y - x + b - 1) // b for x, y in zip(bd, bd[1:])]
    assert sum(sizes) == n and max(sizes) - min(sizes) <= 1


def test_config_work_counts():
    c = CONFIGS["8b_32k"]
    assert c.n_blocks == 4 and c.G == 4 and c.bounds() == [0, 8192, 16384, 24576, 32768]
    # pairs per head: 4 blocks x 8192*8193/2 causal + 3 blocks x 8192*8192 anchor = 335,560,704
    assert c.phase1_flops() == 4 * 128 * 32 * 335_560_704
    assert c.decode_step_bytes(0) == 2 * 8 * (32768 + 128 + 1) * 128 * 2
    assert CONFIGS["8b_1m"].n_blocks == 16 and CONFIGS["70b_128k"].n_blocks == 8
    assert CONFIGS["70b_128k"].G == 8


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 exits with a message before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
