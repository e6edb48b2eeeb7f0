"""Workload shapes and the host-side plan (block and shard boundaries).

Block partition: "Star Attention: Efficient LLM Inference over Long Sequences"
(paper-graph-ui summary), section 3.4, Phase 1 Step 1 -- n = ceil(L / b)
contiguous blocks, the last possibly shorter.  Host assignment: same page,
Phase 1 Step 3 -- blocks are independent units spread over the hosts; the page
leaves the policy open and this plan uses contiguous groups of blocks (host r
gets blocks [floor(r n / S), floor((r+1) n / S))).

The five workloads mirror the pages' settings: 8B-shaped (32 q / 8 kv heads)
and 70B-shaped (64 q / 8 kv heads) attention layers with head dim 128 in
bf16, block = anchor = a quarter of the context up to 128K (section 3.4
"Hyperparameters and Configuration Choices"), and a 1M-token context with 16
blocks.  The first is a tiny fp32 case the oracle finishes in a moment.
"""
from __future__ import annotations

from dataclasses import dataclass


def n_blocks(L: int, block: int) -> int:
    """Number of context blocks, ceil(L / block)."""
    if L < 1 or block < 1:
        raise ValueError("L and block must be >= 1")
    return -(-L // block)


def block_range(L: int, block: int, i: int) -> tuple[int, int]:
    return i * block, min(L, (i + 1) * block)


def shard_bounds(L: int, block: int, n_shards: int) -> list[int]:
    """Token bounds of n_shards hosts, each a contiguous group of whole blocks."""
    n = n_blocks(L, block)
    if n_shards < 1:
        raise ValueError("n_shards must be >= 1")
    out = []
    for r in range(n_shards + 1):
        first_block = (r * n) // n_shards
        out.append(min(L, first_block * block))
    out[-1] = L
    return out


def star_comm_elements_per_token(d: int) -> int:
    """Numbers a host returns per query token, head and layer in Phase 2: A_h (d values)
    plus s_h (one scalar) -- section 3.4 Phase 2 Step 4."""
    return d + 1


@dataclass(frozen=True)
class StarConfig:
    name: str
    hq: int
    hkv: int
    d: int
    L: int
    block: int
    anchor: int
    lq: int
    decode_steps: int
    shards: int
    dtype: str          # "bf16" or "f32"
    needle: bool = False
    seed: int = 0

    @property
    def G(self) -> int:
        return self.hq // self.hkv

    @property
    def n_blocks(self) -> int:
        return n_blocks(self.L, self.block)

    @property
    def tail_cap(self) -> int:
        return self.lq + self.decode_steps

    def bounds(self) -> list[int]:
        return shard_bounds(self.L, self.block, self.shards)

    def phase1_pairs_per_head(self) -> int:
        """Unmasked (query, key) pairs of Phase 1 per q head."""
        total = 0
        for i in range(self.n_blocks):
            lo, hi = block_range(self.L, self.block, i)
            r = hi - lo
            total += r * (r + 1) // 2 + (self.anchor * r if i >= 1 else 0)
        return total

    def phase1_flops(self) -> int:
        """Algorithmic Phase-1 work: 2 flops per multiply-add in QK^T and in PV, so 4*d per pair."""
        return 4 * self.d * self.hq * self.phase1_pairs_per_head()

    def phase2_query_flops(self) -> int:
        pairs = self.lq * self.L + self.lq * (self.lq + 1) // 2
        return 4 * self.d * self.hq * pairs

    def decode_step_bytes(self, t: int) -> int:
        """K and V bytes one decode step must stream: every cached token once, per kv head."""
        eb = 2 if self.dtype == "bf16" else 4
        return 2 * self.hkv * (self.L + self.lq + t + 1) * self.d * eb

    def decode_step_bytes_kv8(self, t: int) -> int:
        """The same with an E4M3 context cache (1 byte per element) and the query host's
        cache in the compute dtype."""
        eb = 2 if self.dtype == "bf16" else 4
        return 2 * self.hkv * self.d * (self.L + (self.lq + t + 1) * eb)


_BASE_SEED = 20241126

CONFIGS = {
    "tiny_f32": StarConfig("tiny_f32", hq=1, hkv=1, d=64, L=2048, block=512, anchor=512, lq=16,
                           decode_steps=4, shards=2, dtype="f32", seed=_BASE_SEED + 0),
    "8b_32k": StarConfig("8b_32k", hq=32, hkv=8, d=128, L=32768, block=8192, anchor=8192, lq=128,
                         decode_steps=32, shards=4, dtype="bf16", seed=_BASE_SEED + 1),
    "8b_128k_needle": StarConfig("8b_128k_needle", hq=32, hkv=8, d=128, L=131072, block=32768, anchor=32768,
                                 lq=128, decode_steps=64, shards=4, dtype="bf16", needle=True,
                                 seed=_BASE_SEED + 2),
    "70b_128k": StarConfig("70b_128k", hq=64, hkv=8, d=128, L=131072, block=16384, anchor=16384, lq=256,
                           decode_steps=64, shards=8, dtype="bf16", seed=_BASE_SEED + 3),
    "8b_1m": StarConfig("8b_1m", hq=32, hkv=8, d=128, L=1048576, block=65536, anchor=65536, lq=128,
                        decode_steps=32, shards=16, dtype="bf16", seed=_BASE_SEED + 4),
}
