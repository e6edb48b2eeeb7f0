"""Where the time of one decode launch goes, from the profiling build of the library.

    python -m block_sparse_long_phase1_amd.decode_timeline [--config 8b_32k,8b_128k_needle] [--reps 4] [--kv8]

libstarattn_timeline.so (built next to libstarattn.so) is the same library with the decode
kernel recording, per workgroup, the constant 100 MHz clock at fixed points: start, stream done
(waves combined into the chunk partial), partial stores complete, ticket drawn, and for the
workgroup that merges a kv head: past its acquire fence and merge done.  This tool runs decode
step 0 of each workload on seeded synthetic inputs of its shapes (as bench.py does) in three ways:
steady (the last of 16 launches issued back to back, as in a decode loop), warm (one launch after
the same step ran and the GPU went idle) and cold (one launch after 1 GiB was overwritten and read
back), and prints one JSON line per launch and a table of medians.  Times are microseconds from
the first workgroup's start.  The in-kernel merge exists for hq/hkv <= 4; other shapes report the
stream part only.  With --kv8 the context cache is first quantised to E4M3 (per-kv-head scales)
and the decode step over it is timed instead (workload names get a "_kv8" suffix).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics

import numpy as np

from . import build as _build

SLOTS = 8
GROUPS = 4096
MODES = ("steady", "warm", "cold")


def _load():
    import block_sparse_long_phase1_amd as sa
    path = _build.TIMELINE_LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError("%s not found; build it with `python -m block_sparse_long_phase1_amd.build`" % path)
    lib = sa.load_library(path, make_default=True)   # every binding now calls the profiling build
    lib.star_decode_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.star_decode_timeline_read.restype = ctypes.c_int
    return sa, lib


def _summary(ts: np.ndarray, grid: int) -> dict:
    t = ts[:grid].astype(np.float64)
    t0 = t[:, 0].min()
    us = lambda col: (t[:, col] - t0) / 100.0
    start, stream_end = us(0), us(1)
    stream = stream_end - start
    r = {"workgroups": grid, "start_spread": float(start.max()),
         "stream_median": float(np.median(stream)), "stream_max": float(stream.max()),
         "stream_end": float(stream_end.max())}
    if (t[:, 2] > 0).all():
        stored, ticket = us(2), us(3)
        r.update({"store_wait_median": float(np.median(stored - stream_end)),
                  "store_wait_max": float((stored - stream_end).max()),
                  "ticket_median": float(np.median(ticket - stored)), "last_ticket": float(ticket.max())})
        # the workgroups that drew a kv head's last ticket in this launch (slot 6 holds every
        # workgroup's ticket, so merge slots left by earlier launches are not mistaken for them)
        merger = (t[:, 6] == t[:, 6].max()) & (t[:, 5] > 0)
        if merger.any():
            r.update({"mergers": int(merger.sum()),
                      "merge_acquire": float(np.max(us(4)[merger] - ticket[merger])),
                      "merge": float(np.max(us(5)[merger] - ticket[merger])),
                      "end": float(us(5)[merger].max())})
    return r


def run(configs: list[str], reps: int, kv8: bool = False) -> list[dict]:
    import torch
    sa, lib = _load()
    from .configs import CONFIGS
    from . import inputs as sin

    dev = "cuda:0"
    buf = np.zeros((GROUPS, SLOTS), dtype=np.uint64)
    out = []
    for name in configs:
        cfg = CONFIGS[name]
        k = sin.randn(cfg, "k_ctx", (cfg.hkv, cfg.L, cfg.d), dev)
        v = sin.randn(cfg, "v_ctx", (cfg.hkv, cfg.L, cfg.d), dev)
        p2 = sin.phase2_inputs(cfg, dev)
        bounds = cfg.bounds()
        kt = torch.zeros((cfg.hkv, cfg.tail_cap, cfg.d), dtype=k.dtype, device=dev)
        vt = torch.zeros_like(kt)
        kt[:, :cfg.lq] = p2["k_qry"]
        vt[:, :cfg.lq] = p2["v_qry"]
        ws = sa.decode_workspace(cfg.L, cfg.tail_cap, len(bounds) - 1, cfg.hq, cfg.hkv, cfg.d, dev)
        o = torch.empty((cfg.hq, cfg.d), dtype=k.dtype, device=dev)
        lse = torch.empty((cfg.hq,), dtype=torch.float32, device=dev)
        st = torch.cuda.current_stream()
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        sink = torch.empty((), dtype=torch.float32, device=dev)

        if kv8:
            ks, vs = sa.star_kv_fp8_scales(k), sa.star_kv_fp8_scales(v)
            k8, v8 = sa.star_kv_quantize_fp8(k, ks), sa.star_kv_quantize_fp8(v, vs)

            def step():
                sa.star_decode_step_kv8(p2["q_dec"][0], p2["k_dec"][0], p2["v_dec"][0], k8, v8, ks, vs, bounds, kt,
                                        vt, cfg.lq, o=o, lse=lse, workspace=ws, stream=st)
        else:
            def step():
                sa.star_decode_step(p2["q_dec"][0], p2["k_dec"][0], p2["v_dec"][0], k, v, bounds, kt, vt, cfg.lq,
                                    o=o, lse=lse, workspace=ws, stream=st)
        label = name + ("_kv8" if kv8 else "")

        for _ in range(3):
            step()
        torch.cuda.synchronize()
        for rep in range(reps):
            for mode in MODES:
                if mode == "cold":
                    flush.fill_(float(rep))
                    torch.sum(flush, dim=0, out=sink)
                else:
                    step()
                torch.cuda.synchronize()
                assert lib.star_decode_timeline_read(None, 0) == 0
                if mode == "steady":
                    for _ in range(15):
                        step()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(st)
                step()
                b.record(st)
                torch.cuda.synchronize()
                assert lib.star_decode_timeline_read(buf.ctypes.data, buf.nbytes) == 0
                grid = int((buf[:, 0] > 0).sum())
                r = {"config": label, "mode": mode, "rep": rep, "event_us": a.elapsed_time(b) * 1e3}
                r.update(_summary(buf, grid))
                print(json.dumps({k2: (round(x, 2) if isinstance(x, float) else x) for k2, x in r.items()}),
                      flush=True)
                out.append(r)
        del k, v, flush
        if kv8:
            del k8, v8
        torch.cuda.empty_cache()
    return out


def table(rows: list[dict]) -> str:
    keys = ["event_us", "start_spread", "stream_median", "stream_max", "stream_end", "store_wait_median",
            "ticket_median", "last_ticket", "merge_acquire", "merge", "end"]
    lines = ["| workload | launch | " + " | ".join(keys) + " |", "|---|---|" + "---|" * len(keys)]
    for name in dict.fromkeys(r["config"] for r in rows):
        for mode in MODES:
            sel = [r for r in rows if r["config"] == name and r["mode"] == mode]
            if not sel:
                continue
            cells = []
            for k in keys:
                vals = [r[k] for r in sel if k in r]
                cells.append("%.2f" % statistics.median(vals) if vals else "-")
            lines.append("| %s | %s | %s |" % (name, mode, " | ".join(cells)))
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", default="8b_32k,8b_128k_needle,8b_1m")
    ap.add_argument("--reps", type=int, default=4)
    ap.add_argument("--kv8", action="store_true", help="time the decode step over an E4M3 context cache")
    args = ap.parse_args()
    rows = run(args.config.split(","), args.reps, args.kv8)
    print("medians over %d launches of each kind (us):" % args.reps)
    print(table(rows))


if __name__ == "__main__":
    main()
