#!/usr/bin/env python3
"""Benchmark of the HGA forward hot path on one MI355X.

Step = one pass of hga_summarize (append the active segment's 32 chunk
summaries per kv head) -> hga_route -> hga_attend_fwd over one Qwen3-8B
attention layer: 32 query heads, 8 kv heads, head dim 128, bf16, 2048 active
queries at positions 14336..16383 over 14336 history tokens resident in HBM,
chunk 64, top-16 plus the causal local block. Inputs are seeded synthetic
draws (sparse_long_context_summarize_amd.inputs), resident in HBM before the
timed region; the history summaries are built before it as well.

Prints one JSON line: query tokens/s of that layer (value), the attention
kernel's roofline position (algorithmic flops over its HIP-event-timed
duration against the bf16 MFMA peak) and the CPU oracle's rate on a bounded
sample of the same workload. The backward (hga_attend_bwd at the same shape)
and the 36-layer x 8-segment loop are timed separately and reported under
"extra"; they are not part of the step.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
C = 64

# HBM bytes the attention kernel moved per launch, from rocprofv3 --pmc
# FETCH_SIZE / WRITE_SIZE at this workload (KiB per dispatch, scaled by the
# copy-kernel calibration factor); None until measured for the current kernel.
MEASURED_TRAFFIC_BYTES = None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the backward and segment-loop timings")
    return ap.parse_args()


def attend_flops(ids: np.ndarray, n_q: int, G: int, D: int, p0: int) -> float:
    """Algorithmic flops of hga_attend_fwd: 4*D per attended (query, key) pair
    (2*D for q.k, 2*D for p*v), summed over every query of every head."""
    Hkv, nb, k = ids.shape
    P = p0 + np.arange(nb) * C
    valid = ((ids >= 0) & (ids < (P // C)[None, :, None])).sum(axis=2)      # [Hkv][nb]
    routed_pairs = valid.sum() * C * C * G                                   # 64 queries x 64 keys
    local_pairs = Hkv * G * nb * (C * (C + 1) // 2)
    return 4.0 * D * float(routed_pairs + local_pairs)


def attend_bytes(ids: np.ndarray, n_q: int, Hq: int, D: int, p0: int) -> float:
    """Algorithmic HBM bytes of hga_attend_fwd: each (block, kv head) gathers
    its routed chunks' and local block's K and V once (bf16), reads Q once,
    writes O (bf16) and lse (fp32)."""
    Hkv, nb, k = ids.shape
    P = p0 + np.arange(nb) * C
    valid = ((ids >= 0) & (ids < (P // C)[None, :, None])).sum(axis=2)
    gathered = (valid.sum() + Hkv * nb) * C * D * 2 * 2
    return float(gathered + Hq * n_q * D * 2 * 2 + Hq * n_q * 4)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "this library has no multi-GPU path to measure", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_long_context_summarize_amd import hga, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    hga.lib()    # raises if libhga.so is missing: no fallback

    w = inputs.LAYER16K
    x = inputs.generate(w)
    dev = torch.device("cuda:0")

    def up(a):
        return torch.from_numpy(a).to(torch.bfloat16).to(dev)

    Q, K, V = up(x["Q"]), up(x["K"]), up(x["V"])
    cfg = hga.make_config(w.Hq, w.Hkv, w.k)
    nb = w.n_q // C
    n_cap = w.T // C
    S = torch.zeros((w.Hkv, n_cap, w.D), device=dev)
    ids = torch.empty((w.Hkv, nb, w.k), dtype=torch.int32, device=dev)
    O = torch.empty((w.Hq, w.n_q, w.D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.Hq, w.n_q), device=dev)
    hga.hga_summarize(cfg, K, 0, w.p0, S)          # history summaries: outside the step
    n_valid = (w.p0 + w.n_q) // C

    ev = {name: [] for name in ("summarize", "route", "attend")}

    def step(record=False):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if record else None
        if record: e[0].record()
        hga.hga_summarize(cfg, K, w.p0, w.n_q, S)
        if record: e[1].record()
        hga.hga_route(cfg, Q, w.p0, S, n_valid, ids)
        if record: e[2].record()
        hga.hga_attend_fwd(cfg, Q, K, V, w.p0, ids, O, lse)
        if record:
            e[3].record()
            ev["summarize"].append((e[0], e[1]))
            ev["route"].append((e[1], e[2]))
            ev["attend"].append((e[2], e[3]))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(record=True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    ms = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in ev.items()}
    ids_np = ids.cpu().numpy()
    flops = attend_flops(ids_np, w.n_q, w.G, w.D, w.p0)
    abytes = attend_bytes(ids_np, w.n_q, w.Hq, w.D, w.p0)
    achieved = flops / (ms["attend"] * 1e-3) / 1e12
    ms_per_step = elapsed / args.steps * 1e3
    value = w.n_q * args.steps / elapsed

    out = {
        "metric": "HGA attention query tokens/sec per layer at 16K history; % bf16 MFMA peak",
        "value": value,
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V with per-chunk key offsets N(0,0.5^2))",
        "config": {"workload": w.name, "n_q_heads": w.Hq, "n_kv_heads": w.Hkv,
                   "head_dim": w.D, "history": w.p0, "active_queries": w.n_q,
                   "chunk": C, "q_block": C, "top_k": w.k},
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": MEASURED_TRAFFIC_BYTES,
        },
        "kernels_ms": ms,
        "attend_algorithmic": {"flops": flops, "bytes": abytes,
                               "gathered_GBps": abytes / (ms["attend"] * 1e-3) / 1e9,
                               "hbm_frac_of_algorithmic_bytes":
                                   abytes / (ms["attend"] * 1e-3) / 1e9 / PEAK_HBM_GBS},
    }

    if not args.no_extra:
        out["extra"] = extra_timings(torch, hga, inputs, dev)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inputs, w, x)

    print(json.dumps(out), flush=True)


def extra_timings(torch, hga, inputs, dev):
    """Backward at the 16K layer shape, timed with HIP events (median of 20)."""
    res = {}
    w = inputs.BWD16K
    x = inputs.generate(w)

    def up(a):
        return torch.from_numpy(a).to(torch.bfloat16).to(dev)

    Q, K, V, dO = up(x["Q"]), up(x["K"]), up(x["V"]), up(x["dO"])
    cfg = hga.make_config(w.Hq, w.Hkv, w.k)
    nb = w.n_q // C
    S = torch.zeros((w.Hkv, w.T // C, w.D), device=dev)
    ids = torch.empty((w.Hkv, nb, w.k), dtype=torch.int32, device=dev)
    O = torch.empty((w.Hq, w.n_q, w.D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.Hq, w.n_q), device=dev)
    hga.hga_summarize(cfg, K, 0, w.T, S)
    hga.hga_route(cfg, Q, w.p0, S, w.T // C, ids)
    hga.hga_attend_fwd(cfg, Q, K, V, w.p0, ids, O, lse)
    dQ = torch.empty((w.Hq, w.n_q, w.D), device=dev)
    dK = torch.empty((w.Hkv, w.n_q, w.D), device=dev)
    dV = torch.empty((w.Hkv, w.n_q, w.D), device=dev)
    ws = torch.empty(hga.hga_attend_bwd_workspace_bytes(cfg, w.n_q), dtype=torch.uint8,
                     device=dev)
    try:
        times = []
        for i in range(25):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            hga.hga_attend_bwd(cfg, Q, K, V, w.p0, ids, O, lse, dO, dQ, dK, dV, ws)
            b.record()
            times.append((a, b))
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in times[5:])
        res["bwd16k_ms"] = t[len(t) // 2]
    except hga.HGAError as e:
        res["bwd16k_ms"] = None
        res["bwd16k_error"] = str(e)
    return res


def cpu_baseline(inputs, w, x):
    """The CPU oracle (plain C, fp64, OpenMP) on a bounded sample of the same
    workload: summaries of the active segment, routing of every block, and
    attention for the first n_blk query blocks of every head."""
    import oracle
    threads = min(16, os.cpu_count() or 1)
    oracle.set_threads(threads)
    n_blk = 8
    mask = np.zeros((w.Hq, w.n_blocks), np.uint8)
    mask[:, :n_blk] = 1
    n_cap = w.T // C
    S = oracle.summarize(x["K"], C, 0, w.p0 // C, n_cap=n_cap)
    t0 = time.perf_counter()
    oracle.summarize(x["K"], C, w.p0 // C, n_cap, out=S)
    ids = oracle.route(x["Q"], S, w.p0, w.k, w.Hkv)
    oracle.attend_fwd(x["Q"], x["K"], x["V"], ids, w.p0, unit_mask=mask)
    dt = time.perf_counter() - t0
    return {"value": n_blk * C / dt, "unit": "query tokens/s", "cores": oracle.get_threads(),
            "kind": "oracle",
            "sample": f"{n_blk} of {w.n_blocks} query blocks (all 32 heads) of {w.name}, "
                      f"plus the active segment's summaries and all blocks' routing; "
                      f"{dt:.1f} s"}


if __name__ == "__main__":
    main()
