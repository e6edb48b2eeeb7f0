"""Seeded synthetic inputs shared by the GPU path, the tests and the benchmark.

Holds no attention arithmetic: only random draws and their placement.  Every
tensor has its own generator stream derived from the workload's seed, so any
subset can be regenerated on its own.  Values are standard normal fp32 draws,
rounded to nearest-even when the workload is bf16; they stand in for one
attention layer's post-rotary activations.

Needle workloads plant, for every kv head g, one context key at a seeded
position p_g equal to 8x the query vector of token 0 of q head g*G, so the
aligned query's softmax is sharply peaked (score near 8 |q|^2 / sqrt(d)).
"""
from __future__ import annotations

import torch

from .configs import StarConfig

_STREAMS = {"q_ctx": 1, "k_ctx": 2, "v_ctx": 3, "q_qry": 4, "k_qry": 5, "v_qry": 6,
            "q_dec": 7, "k_dec": 8, "v_dec": 9, "needle": 10}


def torch_dtype(cfg: StarConfig):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def _gen(cfg: StarConfig, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed * 1000 + _STREAMS[name])
    return g


def randn(cfg: StarConfig, name: str, shape, device, chunk_rows: int = 1 << 27) -> torch.Tensor:
    """N(0,1) draws of `shape` in the workload dtype, generated in slices along dim 0 so the
    fp32 staging buffer stays bounded."""
    dt = torch_dtype(cfg)
    gen = _gen(cfg, name, device)
    out = torch.empty(shape, dtype=dt, device=device)
    per = 1
    for s in shape[1:]:
        per *= s
    step = max(1, chunk_rows // max(per, 1))
    for i in range(0, shape[0], step):
        j = min(shape[0], i + step)
        out[i:j] = torch.randn((j - i,) + tuple(shape[1:]), generator=gen, device=device,
                               dtype=torch.float32).to(dt)
    return out


def needle_positions(cfg: StarConfig, device="cpu") -> list[int]:
    g = _gen(cfg, "needle", "cpu")
    return [int(x) for x in torch.randint(0, cfg.L, (cfg.hkv,), generator=g)]


def phase1_inputs(cfg: StarConfig, device):
    q = randn(cfg, "q_ctx", (cfg.hq, cfg.L, cfg.d), device)
    k = randn(cfg, "k_ctx", (cfg.hkv, cfg.L, cfg.d), device)
    v = randn(cfg, "v_ctx", (cfg.hkv, cfg.L, cfg.d), device)
    return q, k, v


def phase2_inputs(cfg: StarConfig, device):
    """Query-token Q/K/V and per-step decode q/k/v (the pages' model and sampler are replaced
    by seeded draws, one per generated token)."""
    T = cfg.decode_steps
    return {
        "q_qry": randn(cfg, "q_qry", (cfg.hq, cfg.lq, cfg.d), device),
        "k_qry": randn(cfg, "k_qry", (cfg.hkv, cfg.lq, cfg.d), device),
        "v_qry": randn(cfg, "v_qry", (cfg.hkv, cfg.lq, cfg.d), device),
        "q_dec": randn(cfg, "q_dec", (T, cfg.hq, cfg.d), device),
        "k_dec": randn(cfg, "k_dec", (T, cfg.hkv, cfg.d), device),
        "v_dec": randn(cfg, "v_dec", (T, cfg.hkv, cfg.d), device),
    }


def plant_needles(cfg: StarConfig, k_ctx: torch.Tensor, q_qry: torch.Tensor) -> list[int]:
    """Set K[g, p_g] = 8 * q_qry[g*G, 0] for every kv head; returns the positions."""
    pos = needle_positions(cfg)
    for g, p in enumerate(pos):
        k_ctx[g, p] = (8.0 * q_qry[g * cfg.G, 0].float()).to(k_ctx.dtype)
    return pos


def all_inputs(cfg: StarConfig, device):
    q, k, v = phase1_inputs(cfg, device)
    p2 = phase2_inputs(cfg, device)
    needles = plant_needles(cfg, k, p2["q_qry"]) if cfg.needle else []
    out = {"q_ctx": q, "k_ctx": k, "v_ctx": v, "needles": needles}
    out.update(p2)
    return out
