"""Benchmark of the Star Attention two-phase hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input, inputs already
resident in HBM:
  Phase 1  star_phase1_encode over the whole context (one kernel launch),
  Phase 2  query encoding: star_phase2_query (the partials of every context shard and of
           the query host's own cache, then their merge),
           then decode_steps x star_decode_step (append + split-KV partials + merge).

Prints ONE JSON line.  `value` is context tokens per second of the whole step
(L / step time, `value_is` says so); `phase1.context_tokens_per_s` is the Phase-1 rate alone.  `roofline` describes the dominant kernel (the Phase-1 MFMA kernel):
algorithmic flops per launch / its average launch time measured with HIP events on the
launch stream, against the bf16 dense MFMA peak.  `decode` reports the decode step's
K/V stream rate (warm: inside the step; cold: after overwriting 1 GiB and reading it back,
so the 256 MB last-level cache holds no K/V and no dirty lines).  `decode_kv8` reports the
same decode steps over an E4M3 context cache (quantised once, after the step; its time is
reported too) against the same bytes model with 1-byte context elements, and the query
phase over that cache (star_phase2_query_kv8).  `cpu_baseline`
times the fp64 oracle on a bounded sample of the same step on the host's cores: seeded
Phase-1 rows, sampled query rows and whole decode steps.

The default workload is the largest one, 8b_1m (L = 1,048,576, block = anchor = 65,536,
16 shards); `--config` selects another.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Phase-1 context tokens/s + MFMA %peak; Phase-2 decode KV GB/s (%HBM), 1 GPU"
PEAK_BF16_FLOPS = 2.5e15     # MI355X dense bf16 MFMA
PEAK_HBM_BYTES = 8.0e12      # MI355X HBM3E
PHASE1_KERNEL = "attn_mfma_kernel<0, 128, false>"
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "block_sparse_long_phase1_amd", "csrc", f)
                  for f in ("prefill.hip", "common.h", "internal.h")]


def code_text(text: str) -> str:
    """C++ source with comments removed and white space collapsed: what the compiler sees."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """sha256 prefix of the Phase-1 kernel's sources without comments, so that the committed
    counter profile stays valid across comment edits and no longer after a code change."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p) as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_profile_path(workload: str) -> str:
    """The committed rocprofv3 counter summary of the Phase-1 kernel on one workload."""
    return os.path.join(PROFILE_DIR, "phase1_%s_traffic.txt" % workload)


def read_traffic(workload: str):
    """HBM bytes per Phase-1 launch on `workload` from the committed rocprofv3 counter
    summary, if one was taken on that workload and on the current kernel source; else None."""
    path = traffic_profile_path(workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not b or m.group(1) != kernel_source_hash():
        return None
    return float(b.group(1))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="8b_1m")
    ap.add_argument("--block", type=int, default=None, help="override the workload's block size")
    ap.add_argument("--anchor", type=int, default=None, help="override the workload's anchor size")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=24.0,
                    help="host CPU time budget of the oracle baseline (split between the two phases)")
    ap.add_argument("--cold-reps", type=int, default=8)
    ap.add_argument("--no-kv8", action="store_true", help="skip the E4M3 context-cache decode leg")
    ap.add_argument("--only", choices=["all", "phase1", "decode"], default="all",
                    help="restrict the timed step (for profiling runs); the JSON line is always the full step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 1 GiB device copy (counter calibration) and exit")
    return ap.parse_args()


def calibrate_copy():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the whole path runs on a single MI355X and no "
              "multi-GPU sharding is implemented (--gpus %d requested)" % args.gpus)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    import numpy as np
    import torch

    import block_sparse_long_phase1_amd as sa
    from block_sparse_long_phase1_amd import inputs as sin
    from block_sparse_long_phase1_amd.configs import CONFIGS

    cfg = CONFIGS[args.config]
    if args.block is not None or args.anchor is not None:
        import dataclasses
        blk = args.block if args.block is not None else cfg.block
        anc = args.anchor if args.anchor is not None else min(cfg.anchor, blk)
        cfg = dataclasses.replace(cfg, name="%s_b%d_a%d" % (cfg.name, blk, anc), block=blk, anchor=anc)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    print("bench: config %s, generating inputs" % cfg.name, file=sys.stderr, flush=True)
    x = sin.all_inputs(cfg, dev)
    q, k, v = x["q_ctx"], x["k_ctx"], x["v_ctx"]
    bounds = cfg.bounds()
    dt = q.dtype
    o = torch.empty_like(q)
    lse = torch.empty((cfg.hq, cfg.L), dtype=torch.float32, device=dev)
    k_tail = torch.zeros((cfg.hkv, cfg.tail_cap, cfg.d), dtype=dt, device=dev)
    v_tail = torch.zeros_like(k_tail)
    k_tail[:, :cfg.lq] = x["k_qry"]
    v_tail[:, :cfg.lq] = x["v_qry"]
    S = len(bounds) - 1
    ws_q = torch.empty(max(sa.star_phase2_query_workspace_bytes(cfg.lq, S, cfg.hq, cfg.hkv, cfg.d), 16),
                       dtype=torch.uint8, device=dev)
    ws_dec = sa.decode_workspace(cfg.L, cfg.tail_cap, S, cfg.hq, cfg.hkv, cfg.d, dev)
    oq = torch.empty((cfg.hq, cfg.lq, cfg.d), dtype=dt, device=dev)
    lq_lse = torch.empty((cfg.hq, cfg.lq), dtype=torch.float32, device=dev)
    od = torch.empty((cfg.decode_steps, cfg.hq, cfg.d), dtype=dt, device=dev)
    ld = torch.empty((cfg.decode_steps, cfg.hq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def phase1():
        sa.star_phase1_encode(q, k, v, cfg.block, cfg.anchor, o=o, lse=lse, stream=stream)

    def query_phase():
        sa.star_phase2_query(x["q_qry"], k, v, bounds, k_tail, v_tail, cfg.lq, o=oq, lse=lq_lse,
                             workspace=ws_q, stream=stream)

    def decode(t):
        sa.star_decode_step(x["q_dec"][t], x["k_dec"][t], x["v_dec"][t], k, v, bounds, k_tail, v_tail,
                            cfg.lq + t, o=od[t], lse=ld[t], workspace=ws_dec, stream=stream)

    ev = lambda: torch.cuda.Event(enable_timing=True)
    p1_ms, q_ms, dec_ms = [], [], []

    def step(timed):
        if args.only in ("all", "phase1"):
            e0, e1 = ev(), ev()
            e0.record(stream)
            phase1()
            e1.record(stream)
        if args.only == "all":
            e2 = ev()
            query_phase()
            e2.record(stream)
        if args.only in ("all", "decode"):
            e3 = ev()
            e3.record(stream)
            for t in range(cfg.decode_steps):
                decode(t)
            e4 = ev()
            e4.record(stream)
        if timed:
            return (e0, e1, e2, e3, e4) if args.only == "all" else None
        return None

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    evs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        evs.append(step(True))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    print("bench: %d timed steps, %.3f ms/step" % (args.steps, ms_per_step), file=sys.stderr, flush=True)
    if args.only != "all":
        return
    for e0, e1, e2, e3, e4 in evs:
        p1_ms.append(e0.elapsed_time(e1))
        q_ms.append(e1.elapsed_time(e2))
        dec_ms.append(e3.elapsed_time(e4))

    # ---- cold-cache decode: overwrite 1 GiB, then read it back, before each timed step
    # (untimed).  The read-back leaves the last-level cache holding clean lines of the
    # flush buffer, so the timed step neither finds K/V cached nor pays for writing back
    # the flush's dirty lines.  Nothing synchronises between these launches and the timed
    # step, so the GPU is busy until the step starts and host launch time is not counted.
    print("bench: cold-cache decode steps", file=sys.stderr, flush=True)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    cold = []
    for r in range(args.cold_reps):
        flush.fill_(float(r))
        torch.sum(flush, dim=0, out=sink)
        t = r % cfg.decode_steps
        a, b = ev(), ev()
        a.record(stream)
        decode(t)
        b.record(stream)
        torch.cuda.synchronize()
        cold.append((a.elapsed_time(b), cfg.decode_step_bytes(t)))

    # ---- E4M3 context cache: quantise the context once, then the decode steps over it
    kv8 = None
    if cfg.dtype == "bf16" and not args.no_kv8:
        print("bench: E4M3 context cache leg", file=sys.stderr, flush=True)
        ks = torch.empty((cfg.hkv,), dtype=torch.float32, device=dev)
        vs = torch.empty_like(ks)
        k8 = torch.empty((cfg.hkv, cfg.L, cfg.d), dtype=torch.uint8, device=dev)
        v8 = torch.empty_like(k8)

        def quantize():
            sa.star_kv_fp8_scales(k, ks, stream=stream)
            sa.star_kv_quantize_fp8(k, ks, k8, stream=stream)
            sa.star_kv_fp8_scales(v, vs, stream=stream)
            sa.star_kv_quantize_fp8(v, vs, v8, stream=stream)

        def decode8(t):
            sa.star_decode_step_kv8(x["q_dec"][t], x["k_dec"][t], x["v_dec"][t], k8, v8, ks, vs, bounds, k_tail,
                                    v_tail, cfg.lq + t, o=od[t], lse=ld[t], workspace=ws_dec, stream=stream)

        def query8():
            sa.star_phase2_query_kv8(x["q_qry"], k8, v8, ks, vs, bounds, k_tail, v_tail, cfg.lq, o=oq, lse=lq_lse,
                                     workspace=ws_q, stream=stream)

        quantize()
        qz = []
        for _ in range(3):
            a, b = ev(), ev()
            a.record(stream)
            quantize()
            b.record(stream)
            qz.append((a, b))
        for _ in range(args.warmup):
            query8()
            for t in range(cfg.decode_steps):
                decode8(t)
        qreps = []
        for _ in range(args.steps):
            a, b = ev(), ev()
            a.record(stream)
            query8()
            b.record(stream)
            qreps.append((a, b))
        reps = []
        for _ in range(args.steps):
            a, b = ev(), ev()
            a.record(stream)
            for t in range(cfg.decode_steps):
                decode8(t)
            b.record(stream)
            reps.append((a, b))
        torch.cuda.synchronize()
        q8_ms = float(np.mean([a.elapsed_time(b) for a, b in qz]))
        d8_ms = float(np.mean([a.elapsed_time(b) for a, b in reps]))
        qq8_ms = float(np.mean([a.elapsed_time(b) for a, b in qreps]))
        cold8 = []
        for r in range(args.cold_reps):
            flush.fill_(float(r))
            torch.sum(flush, dim=0, out=sink)
            t = r % cfg.decode_steps
            a, b = ev(), ev()
            a.record(stream)
            decode8(t)
            b.record(stream)
            torch.cuda.synchronize()
            cold8.append((a.elapsed_time(b), cfg.decode_step_bytes_kv8(t)))
        b8 = sum(cfg.decode_step_bytes_kv8(t) for t in range(cfg.decode_steps))
        w8 = b8 / (d8_ms * 1e-3)
        c8 = sum(bb for _, bb in cold8) / (sum(ms for ms, _ in cold8) * 1e-3)
        qbytes = 2 * cfg.hkv * cfg.L * cfg.d * (2 * 2 + 1)   # two reads of bf16 K and V, one E4M3 write
        kv8 = {"ms_per_token": d8_ms / cfg.decode_steps, "bytes_per_token": b8 / cfg.decode_steps,
               "warm_GBps": w8 / 1e9, "warm_hbm_frac": w8 / PEAK_HBM_BYTES,
               "cold_GBps": c8 / 1e9, "cold_hbm_frac": c8 / PEAK_HBM_BYTES,
               "cold_ms_per_token": float(np.mean([ms for ms, _ in cold8])),
               "quantize_ms": q8_ms, "quantize_GBps": qbytes / (q8_ms * 1e-3) / 1e9,
               "query_ms": qq8_ms, "query_tflops": cfg.phase2_query_flops() / (qq8_ms * 1e-3) / 1e12}
        del k8, v8
    del flush

    flops = cfg.phase1_flops()
    p1_avg = float(np.mean(p1_ms))
    achieved = flops / (p1_avg * 1e-3)
    dec_bytes = sum(cfg.decode_step_bytes(t) for t in range(cfg.decode_steps))
    dec_avg = float(np.mean(dec_ms))
    warm_bw = dec_bytes / (dec_avg * 1e-3)
    cold_bw = sum(bb for _, bb in cold) / (sum(ms for ms, _ in cold) * 1e-3)
    traffic = read_traffic(cfg.name)

    result = {
        "metric": METRIC,
        "value": cfg.L / (ms_per_step * 1e-3),
        "unit": "context tokens/s",
        "value_is": "context tokens per second of the whole step: L / (Phase 1 + query phase + every "
                    "decode step); the Phase-1 rate alone is phase1.context_tokens_per_s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) post-rotary Q/K/V, one attention layer)",
        "config": {"workload": "%s: Hq=%d Hkv=%d d=%d L=%d block=anchor=%d, %d shards, lq=%d, %d decode steps"
                               % (cfg.name, cfg.hq, cfg.hkv, cfg.d, cfg.L, cfg.block, cfg.shards, cfg.lq,
                                  cfg.decode_steps),
                   "L": cfg.L, "block": cfg.block, "anchor": cfg.anchor, "hq": cfg.hq, "hkv": cfg.hkv,
                   "head_dim": cfg.d, "lq": cfg.lq, "decode_steps": cfg.decode_steps, "shards": cfg.shards},
        "roofline": {"bound": "mfma", "kernel": PHASE1_KERNEL, "achieved": achieved / 1e12,
                     "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_FLOPS,
                     "traffic": traffic, "flops_per_launch": flops, "launch_ms": p1_avg},
        "phase1": {"ms": p1_avg, "context_tokens_per_s": cfg.L / (p1_avg * 1e-3),
                   "tflops": achieved / 1e12, "mfma_frac": achieved / PEAK_BF16_FLOPS},
        "query_phase": {"ms": float(np.mean(q_ms)), "tflops": cfg.phase2_query_flops() / (np.mean(q_ms) * 1e-3) / 1e12},
        "decode": {"steps": cfg.decode_steps, "ms_per_token": dec_avg / cfg.decode_steps,
                   "bytes_per_token": dec_bytes / cfg.decode_steps,
                   "warm_GBps": warm_bw / 1e9, "warm_hbm_frac": warm_bw / PEAK_HBM_BYTES,
                   "cold_GBps": cold_bw / 1e9, "cold_hbm_frac": cold_bw / PEAK_HBM_BYTES,
                   "cold_ms_per_token": float(np.mean([ms for ms, _ in cold]))},
        "decode_kv8": kv8,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("bench: CPU oracle baseline (about %.0f s)" % args.cpu_seconds, file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, x, bounds, k_tail, v_tail, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def host_threads() -> tuple[int, int]:
    """(CPUs this process may run on, oracle threads).  The oracle takes at most 16 threads,
    one GPU's share of a host, whatever the machine reports."""
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count() or 1
    return avail, max(1, min(16, avail))


def cpu_baseline(cfg, x, bounds, k_tail, v_tail, seconds):
    """The fp64 oracle on the host over a bounded sample of one bench step, scaled to the
    whole step: about half of `seconds` on seeded-random Phase-1 rows (all q heads each), then
    sampled query rows (every partition, all q heads) and whole decode steps (all q heads over
    every context token and the query host's cache).  Each leg takes at least one unit."""
    import numpy as np
    import torch

    import oracle

    avail, threads = host_threads()
    q, k, v = x["q_ctx"], x["k_ctx"], x["v_ctx"]
    kh, vh = k.cpu(), v.cpu()
    kt, vt = k_tail.cpu(), v_tail.cpu()
    rng = np.random.default_rng(cfg.seed)

    # Phase 1: seeded-random context rows, batches doubling until the budget is spent
    p1_rows, p1_s, batch = 0, 0.0, 8
    while p1_s < 0.5 * seconds:
        rows = np.sort(rng.choice(cfg.L, size=min(batch, cfg.L), replace=False)).astype(np.int64)
        qs = q[:, torch.from_numpy(rows).to(q.device)].cpu()
        t0 = time.perf_counter()
        oracle.phase1(qs, kh, vh, cfg.block, cfg.anchor, rows=rows, q_sampled=True, threads=threads)
        p1_s += time.perf_counter() - t0
        p1_rows += rows.size
        batch = min(batch * 2, 1024)

    # Phase 2 query phase: one query row at a time (its partial over every context shard, its
    # causal partial over the query tokens before it, the merge), rows in seeded order
    kq, vq = kt[:, :cfg.lq], vt[:, :cfg.lq]
    qq = x["q_qry"].cpu()
    q_rows, q_s = 0, 0.0
    for i in rng.permutation(cfg.lq):
        qi = qq[:, int(i):int(i) + 1]
        t0 = time.perf_counter()
        parts = [oracle.partial(qi, kh, vh, lo, hi, -1, threads=threads) for lo, hi in zip(bounds[:-1], bounds[1:])]
        parts.append(oracle.partial(qi, kq, vq, 0, cfg.lq, int(i), threads=threads))
        oracle.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]),
                     np.stack([p[2] for p in parts]))
        q_s += time.perf_counter() - t0
        q_rows += 1
        if q_s >= 0.15 * seconds:
            break

    # Phase 2 decode: whole steps t = 0, 1, ... (the query host's cache as the step saw it)
    dec_steps, dec_s = 0, 0.0
    for t in range(cfg.decode_steps):
        qt = x["q_dec"][t].cpu()
        t0 = time.perf_counter()
        oracle.phase2_decode(qt, kh, vh, bounds, kt, vt, cfg.lq + t + 1, threads=threads)
        dec_s += time.perf_counter() - t0
        dec_steps += 1
        if dec_s >= 0.35 * seconds:
            break

    p1_row_s = p1_s / p1_rows
    q_row_s = q_s / q_rows
    dec_step_s = dec_s / dec_steps
    step_s = p1_row_s * cfg.L + q_row_s * cfg.lq + dec_step_s * cfg.decode_steps
    return {"value": cfg.L / step_s, "unit": "context tokens/s", "cores": threads, "kind": "oracle",
            "threads": threads, "host_cpus": avail, "host_cpus_reported": os.cpu_count(),
            "cpu_model": cpu_model(),
            "sample": "%s, fp64 C oracle on %d threads (%s; %d CPUs available, os.cpu_count() %s): %d "
                      "seeded-random Phase-1 context rows x all %d q heads (%.1f s), %d of %d query rows "
                      "(%.1f s), %d of %d decode steps (%.1f s); value = L / (per-row Phase-1 time x L + "
                      "per-row query time x lq + per-step decode time x T), i.e. the whole step extrapolated "
                      "from the sample (uniformly drawn rows carry the context's mean cost per row)"
                      % (cfg.name, threads, cpu_model(), avail, os.cpu_count(), p1_rows, cfg.hq, p1_s, q_rows,
                         cfg.lq, q_s, dec_steps, cfg.decode_steps, dec_s),
            "phase1": {"rows": p1_rows, "seconds": p1_s, "context_tokens_per_s": 1.0 / p1_row_s,
                       "extrapolated_s": p1_row_s * cfg.L},
            "query_phase": {"rows": q_rows, "seconds": q_s, "extrapolated_s": q_row_s * cfg.lq},
            "decode": {"steps": dec_steps, "seconds": dec_s, "s_per_token": dec_step_s,
                       "kv_GBps": cfg.decode_step_bytes(0) / dec_step_s / 1e9,
                       "extrapolated_s": dec_step_s * cfg.decode_steps},
            "step_s_extrapolated": step_s}


def cpu_model() -> str:
    """The host CPU's model name (Linux), for the CPU-baseline record."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


if __name__ == "__main__":
    main()
