#!/usr/bin/env python3
"""Benchmark of the HGA forward hot path on one MI355X.

Step = one pass of hga_summarize (append the active segment's 32 chunk
summaries per kv head) -> hga_route_attend_fwd (routing, then attention over
the routed chunks, in one launch) over one Qwen3-8B attention layer: 32 query heads, 8 kv heads, head dim 128, bf16, 2048 active
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

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--no-cpu-baseline]
                    [--no-extra] [--kernel-loop NAME]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import re
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
C = 64
# untimed steps enqueued before the W warm-up steps, about 150 ms of work at
# the 16K layer: after a host wait the GPU runs its first few hundred
# launches up to ~10 % slower while its clocks settle, and a training or
# serving loop runs in the settled state
SETUP_STEPS = 3000

# HBM bytes the routing + attention kernel moves per launch at this
# workload, from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB
# per dispatch) scaled by what the same counters read for an x*1 elementwise
# copy of 256 MiB (`bench.py --copy-calibration 256`: FETCH_SIZE reads half
# the bytes moved, factor 2.0; WRITE_SIZE reads them exactly, factor 1.0).
# The figure belongs to the kernel sources whose combined sha256 prefix is
# recorded; for any other source the traffic is reported as null.
MEASURED_TRAFFIC = {"sources": ["sparse_long_context_summarize_amd/csrc/attend_fwd.hip",
                                "sparse_long_context_summarize_amd/csrc/attend_tiles.h",
                                "sparse_long_context_summarize_amd/csrc/route_core.h"],
                    "sha256_prefix": "d5175c7b24748d8e",
                    "fetch_kib": 30709.4, "fetch_factor": 2.0,
                    "write_kib": 16691.2, "write_factor": 1.0}


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for src in MEASURED_TRAFFIC["sources"]:
        with open(os.path.join(root, src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic_bytes():
    m = MEASURED_TRAFFIC
    if m["sha256_prefix"] is None or kernel_source_hash() != m["sha256_prefix"]:
        return None
    return 1024.0 * (m["fetch_kib"] * m["fetch_factor"] + m["write_kib"] * m["write_factor"])


class HipTimer:
    """HIP timing events of the runtime this process already uses (torch's),
    created with hipEventDisableSystemFence: a default event's system-scope
    release writes back and invalidates the caches when it is recorded,
    which lengthens the interval it brackets by a few microseconds; these
    events only take timestamps."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        maps = open("/proc/self/maps").read()
        path = sorted(set(re.findall(r"/\S*libamdhip64\.so[.0-9]*", maps)))
        if not path:
            raise RuntimeError("the HIP runtime is not loaded")
        self.L = ctypes.CDLL(path[0])
        self.L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def event(self):
        e = ctypes.c_void_p()
        self._ok(self.L.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE),
                 "hipEventCreateWithFlags")
        return e

    def record(self, e, stream: int):
        self._ok(self.L.hipEventRecord(e, ctypes.c_void_p(stream)), "hipEventRecord")

    def elapsed_ms(self, a, b) -> float:
        t = ctypes.c_float()
        self._ok(self.L.hipEventElapsedTime(ctypes.byref(t), a, b), "hipEventElapsedTime")
        return t.value


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the backward and segment-loop timings")
    ap.add_argument("--kernel-loop", default=None, choices=sorted(KERNEL_LOOPS),
                    help="only launch one call N times back to back at one workload (for "
                         "rocprofv3 kernel traces and counter passes) and exit")
    ap.add_argument("--loop-launches", type=int, default=50)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy (x*1 elementwise) of MIB MiB five times (to scale HBM "
                         "byte counters against a kernel of known traffic) and exit")
    return ap.parse_args()


def _n_valid_units(ids: np.ndarray, p0: int, unit: int) -> int:
    """Distinct ids u with 0 <= u < P/unit, summed over (kv head, block) rows."""
    Hkv, nb, _ = ids.shape
    n = 0
    for b in range(nb):
        lim = (p0 + b * C) // unit
        for g in range(Hkv):
            row = ids[g, b]
            n += np.unique(row[(row >= 0) & (row < lim)]).size
    return n


def attend_flops(ids: np.ndarray, n_q: int, G: int, D: int, p0: int, unit: int = C) -> float:
    """Algorithmic flops of hga_attend_fwd (unit = 64, chunk ids) or
    hga_attend_fwd_groups (unit = 8, group ids): 4*D per attended (query, key)
    pair (2*D for q.k, 2*D for p*v), summed over every query of every head."""
    Hkv, nb, k = ids.shape
    routed_pairs = _n_valid_units(ids, p0, unit) * unit * C * G   # unit keys x 64 queries
    local_pairs = Hkv * G * nb * (C * (C + 1) // 2)
    return 4.0 * D * float(routed_pairs + local_pairs)


def attend_flops_executed(ids: np.ndarray, G: int, D: int, p0: int) -> float:
    """Flops the attention kernel executes: every tile is a full 64 x 64 block,
    the masked half of the local (diagonal) tile included."""
    Hkv, nb, k = ids.shape
    tiles = _n_valid_units(ids, p0, C) + Hkv * nb
    return 4.0 * D * G * C * C * float(tiles)


def attend_bytes(ids: np.ndarray, n_q: int, Hq: int, D: int, p0: int, unit: int = C) -> float:
    """Algorithmic HBM bytes of the attention call: each (block, kv head)
    gathers its routed units' and local block's K and V once (bf16), reads Q
    once, writes O (bf16) and lse (fp32)."""
    Hkv, nb, k = ids.shape
    gathered = (_n_valid_units(ids, p0, unit) * unit + Hkv * nb * C) * D * 2 * 2
    return float(gathered + Hq * n_q * D * 2 * 2 + Hq * n_q * 4)


_TIMER = None


def _median_ms(torch, fn, pre=None, n=20):
    """Median time of fn over n launches after 300 untimed ones (the first few
    hundred launches after a host wait run at lower clocks), each between a
    pair of fence-free HIP events on the launch stream (a default event's
    system-scope release adds a few microseconds to the interval it
    brackets); pre runs before each launch, outside the events."""
    global _TIMER
    if _TIMER is None:
        _TIMER = HipTimer()
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(300):
        if pre is not None:
            pre()
        fn()
    ts = []
    for _ in range(n):
        if pre is not None:
            pre()
        a, b = _TIMER.event(), _TIMER.event()
        _TIMER.record(a, stream)
        fn()
        _TIMER.record(b, stream)
        ts.append((a, b))
    torch.cuda.synchronize()
    t = sorted(_TIMER.elapsed_ms(a, b) for a, b in ts)
    return t[len(t) // 2]


def bwd_flops(ids: np.ndarray, n_q: int, G: int, D: int, p0: int, unit: int = C) -> float:
    """Algorithmic flops of hga_attend_bwd (unit = 64, chunk ids) or
    hga_attend_bwd_groups (unit = 8): per attended (query, key) pair 2*D each
    for S, dP and dQ, plus 2*D each for dK and dV where the key is in the
    active segment (history is detached)."""
    Hkv, nb, k = ids.shape
    P = p0 + np.arange(nb) * C
    hist = act = 0
    for b in range(nb):
        for g in range(Hkv):
            row = ids[g, b]
            ok = np.unique(row[(row >= 0) & (row < P[b] // unit)])
            a = int((ok * unit >= p0).sum())
            act += a * unit * C
            hist += (len(ok) - a) * unit * C
        act += Hkv * (C * (C + 1) // 2)
    return float(G * (6 * D * hist + 10 * D * act))


KERNEL_LOOPS = {
    "attend16k": "hga_attend_fwd at the 16K layer (ids from hga_route)",
    "attend128k": "hga_attend_fwd at the 128K-history workload (ids from hga_route)",
    "route_attend16k": "hga_route_attend_fwd at the 16K layer",
    "summarize16k": "hga_summarize of the 16K layer's active segment",
    "bwd16k": "hga_attend_bwd at the 16K backward workload",
    "decode128k": "hga_route_decode + hga_attend_decode, one token after the 128K history",
    "decode128k_fused": "hga_route_attend_decode, one token after the 128K history",
}


def kernel_loop(torch, hga, inputs, name, n):
    """Launch one call n times back to back (after 5 untimed launches and a
    synchronize) and print what ran: a short program for rocprofv3."""
    dev = torch.device("cuda:0")

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(dev)

    w = {"attend128k": inputs.LAYER128K, "decode128k": inputs.LAYER128K,
         "decode128k_fused": inputs.LAYER128K, "bwd16k": inputs.BWD16K}.get(name,
                                                                          inputs.LAYER16K)
    x = inputs.generate(w)
    Q, K, V = up(x["Q"]), up(x["K"]), up(x["V"])
    cfg = hga.make_config(w.Hq, w.Hkv, w.k)
    nb = w.n_q // C
    S = torch.zeros((w.Hkv, w.T // C, w.D), device=dev)
    ids = torch.empty((w.Hkv, nb, w.k), dtype=torch.int32, device=dev)
    O = torch.empty((w.Hq, w.n_q, w.D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.Hq, w.n_q), device=dev)
    if name == "summarize16k":
        hga.hga_summarize(cfg, K, 0, w.p0, S)
        run = hga.prepare("hga_summarize", cfg, K, w.p0, w.n_q, S)
    elif name in ("decode128k", "decode128k_fused"):
        p0 = w.T - 1
        n_closed = p0 // C
        Qd = up(x["Q"][:, :1])
        hga.hga_summarize(cfg, K, 0, n_closed * C, S)
        dids = torch.empty((w.Hkv, 1, w.k), dtype=torch.int32, device=dev)
        Od = torch.empty((w.Hq, 1, w.D), dtype=torch.bfloat16, device=dev)
        lsed = torch.empty((w.Hq, 1), device=dev)
        if name == "decode128k_fused":
            ws = torch.empty(hga.hga_route_attend_decode_workspace_bytes(cfg, p0, 1),
                             dtype=torch.uint8, device=dev)
            run = hga.prepare("hga_route_attend_decode", cfg, Qd, K, V, p0, S, n_closed, dids,
                              Od, lsed, ws)
        else:
            ws = torch.empty(hga.hga_decode_workspace_bytes(cfg, p0, 1), dtype=torch.uint8,
                             device=dev)
            r = hga.prepare("hga_route_decode", cfg, Qd, p0, S, n_closed, dids, ws)
            a = hga.prepare("hga_attend_decode", cfg, Qd, K, V, p0, dids, Od, lsed, ws)

            def run():
                r()
                a()
    else:
        hga.hga_summarize(cfg, K, 0, w.T, S)
        hga.hga_route(cfg, Q, w.p0, S, w.T // C, ids)
        if name in ("attend16k", "attend128k"):
            run = hga.prepare("hga_attend_fwd", cfg, Q, K, V, w.p0, ids, O, lse)
        elif name == "route_attend16k":
            run = hga.prepare("hga_route_attend_fwd", cfg, Q, K, V, w.p0, S, w.T // C, ids, O,
                              lse)
        else:   # bwd16k
            hga.hga_attend_fwd(cfg, Q, K, V, w.p0, ids, O, lse)
            dO = up(x["dO"])
            dQ = torch.empty((w.Hq, w.n_q, w.D), device=dev)
            dK = torch.empty((w.Hkv, w.n_q, w.D), device=dev)
            dV = torch.empty((w.Hkv, w.n_q, w.D), device=dev)
            ws = torch.empty(hga.hga_attend_bwd_workspace_bytes(cfg, w.n_q), dtype=torch.uint8,
                             device=dev)
            run = hga.prepare("hga_attend_bwd", cfg, Q, K, V, w.p0, ids, O, lse, dO, dQ, dK,
                              dV, ws)
    for _ in range(5):
        run()
    torch.cuda.synchronize()
    for _ in range(n):
        run()
    torch.cuda.synchronize()
    print(json.dumps({"kernel_loop": name, "what": KERNEL_LOOPS[name], "workload": w.name,
                      "launches": n}), flush=True)


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
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)      # an elementwise kernel: n*4 bytes in, n*4 out
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4}))
        return
    hga.lib()    # raises if libhga.so is missing: no fallback
    if args.kernel_loop:
        kernel_loop(torch, hga, inputs, args.kernel_loop, args.loop_launches)
        return

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

    # Arguments are marshalled once; each step makes the two C calls.
    run_sum = hga.prepare("hga_summarize", cfg, K, w.p0, w.n_q, S)
    run_fused = hga.prepare("hga_route_attend_fwd", cfg, Q, K, V, w.p0, S, n_valid, ids, O, lse)
    timer = HipTimer()
    stream = torch.cuda.current_stream().cuda_stream      # the stream the calls launch on

    def step():
        run_sum()
        run_fused()

    # Code objects load on the first launches; after this synchronize the
    # rest of the run is enqueued without a host wait, so the GPU never idles
    # (an idle GPU lowers its clocks, and they take about a millisecond to
    # return): set-up steps, then the W warm-up steps, then the K timed steps
    # between two in-stream events, then the kernel-timing steps.
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    for _ in range(SETUP_STEPS):
        step()
    for _ in range(args.warmup):
        step()
    e_begin, e_end = timer.event(), timer.event()
    timer.record(e_begin, stream)
    for _ in range(args.steps):
        step()
    timer.record(e_end, stream)
    # Kernel durations: HIP event pairs around each kernel of the next
    # max(K, 16) steps (enqueued right behind the timed ones; an event pair
    # costs step time, so none sits inside the timed region).
    n_kern = max(args.steps, 16)
    pairs = [((timer.event(), timer.event()), (timer.event(), timer.event()))
             for _ in range(n_kern)]
    for (es, ef) in pairs:
        timer.record(es[0], stream)
        run_sum()
        timer.record(es[1], stream)
        timer.record(ef[0], stream)
        run_fused()
        timer.record(ef[1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    elapsed = timer.elapsed_ms(e_begin, e_end) * 1e-3
    ms = {"summarize": float(np.mean([timer.elapsed_ms(a, b) for (a, b), _ in pairs])),
          "route_attend": float(np.mean([timer.elapsed_ms(a, b) for _, (a, b) in pairs]))}
    ms_per_step = elapsed / args.steps * 1e3
    if ms["route_attend"] > ms_per_step:
        print(f"bench.py: the routing + attention kernel's mean duration "
              f"({ms['route_attend'] * 1e3:.2f} us over {n_kern} launches) exceeds the measured "
              f"step ({ms_per_step * 1e3:.2f} us): the timing is inconsistent, no result printed",
              file=sys.stderr)
        sys.exit(3)
    ids_np = ids.cpu().numpy()
    flops = attend_flops(ids_np, w.n_q, w.G, w.D, w.p0)
    abytes = attend_bytes(ids_np, w.n_q, w.Hq, w.D, w.p0)
    launch_ms = ms["route_attend"]
    achieved = flops / (launch_ms * 1e-3) / 1e12
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
            "traffic": measured_traffic_bytes(),
        },
        "kernels_ms": ms,
        "timing": {"step": "in-stream HIP events around the K timed steps, enqueued right "
                           "behind the warm-up steps with no host wait in between",
                   "kernels": f"HIP event pairs around each kernel of {n_kern} further steps",
                   "setup_steps": SETUP_STEPS,
                   "wall_s_setup_warmup_timed_kernel_steps": wall},
        "attend_algorithmic": {"flops": flops, "bytes": abytes,
                               "executed_flops": attend_flops_executed(ids_np, w.G, w.D, w.p0),
                               "gathered_GBps": abytes / (launch_ms * 1e-3) / 1e9,
                               "hbm_frac_of_algorithmic_bytes":
                                   abytes / (launch_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
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
    res.update(segloop_timing(torch, hga, inputs, dev))
    res.update(group_timings(torch, hga, inputs, dev))
    res.update(decode_timings(torch, hga, inputs, dev))
    res.update(variant_timings(torch, hga, inputs, dev))
    res.update(attend_timings(torch, hga, inputs, dev))
    try:
        bwd = hga.prepare("hga_attend_bwd", cfg, Q, K, V, w.p0, ids, O, lse, dO, dQ, dK, dV, ws)
        res["bwd16k_ms"] = _median_ms(torch, bwd)
        fl = bwd_flops(ids.cpu().numpy(), w.n_q, w.G, w.D, w.p0)
        res["bwd16k_algorithmic_gflop"] = fl / 1e9
        res["bwd16k_tflops"] = fl / (res["bwd16k_ms"] * 1e-3) / 1e12
        n2, nw = hga.hga_diag_bwd_second_pass(cfg, w.n_q, ws)
        res["bwd16k_dq_second_pass_workgroups"] = f"{n2} of {nw}"
    except hga.HGAError as e:
        res["bwd16k_ms"] = None
        res["bwd16k_error"] = str(e)
    return res


def attend_timings(torch, hga, inputs, dev):
    """hga_attend_fwd alone, HIP-event timed (median of 20 after 300 warm-up
    launches): at the 128K-history workload (k = 32), and at the 16K layer
    with L2 and the Infinity Cache flushed before every launch (a 512 MiB
    write) beside the same launches warm."""
    res = {}

    def up(a):
        return torch.from_numpy(a).to(torch.bfloat16).to(dev)

    def med(fn, pre=None, n=20):
        return _median_ms(torch, fn, pre, n)

    for w, tag in ((inputs.LAYER128K, "layer128k"), (inputs.LAYER16K, "layer16k")):
        x = inputs.generate(w)
        Q, K, V = up(x["Q"]), up(x["K"]), up(x["V"])
        cfg = hga.make_config(w.Hq, w.Hkv, w.k)
        S = torch.zeros((w.Hkv, w.T // C, w.D), device=dev)
        ids = torch.empty((w.Hkv, w.n_q // C, w.k), dtype=torch.int32, device=dev)
        O = torch.empty((w.Hq, w.n_q, w.D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.Hq, w.n_q), device=dev)
        hga.hga_summarize(cfg, K, 0, w.T, S)
        hga.hga_route(cfg, Q, w.p0, S, w.T // C, ids)
        run = hga.prepare("hga_attend_fwd", cfg, Q, K, V, w.p0, ids, O, lse)
        flops = attend_flops(ids.cpu().numpy(), w.n_q, w.G, w.D, w.p0)
        abytes = attend_bytes(ids.cpu().numpy(), w.n_q, w.Hq, w.D, w.p0)
        if tag == "layer128k":
            ms = med(run)
            res["layer128k_attend_us"] = ms * 1e3
            res["layer128k_attend_tflops"] = flops / (ms * 1e-3) / 1e12
            res["layer128k_attend_gathered_GBps"] = abytes / (ms * 1e-3) / 1e9
        else:
            res["layer16k_route_us"] = med(hga.prepare("hga_route", cfg, Q, w.p0, S, w.T // C,
                                                       ids)) * 1e3
            # routing + attention with a one-chunk sink window (64 more keys per query)
            cfg_s = hga.make_config(w.Hq, w.Hkv, w.k, sink_chunks=1)
            ids_s = torch.empty_like(ids)
            res["layer16k_sink1_route_attend_us"] = med(hga.prepare(
                "hga_route_attend_fwd", cfg_s, Q, K, V, w.p0, S, w.T // C, ids_s, O, lse)) * 1e3
            res["layer16k_attend_us"] = med(run) * 1e3
            flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
            ms_cold = med(run, pre=lambda: flush.fill_(1))
            ms_warm = med(run, pre=lambda: flush[:1].fill_(1))
            res["layer16k_attend_cold_us"] = ms_cold * 1e3
            res["layer16k_attend_warm_us"] = ms_warm * 1e3
            res["layer16k_attend_cold_gathered_GBps"] = abytes / (ms_cold * 1e-3) / 1e9
            # the gather alone (hga_diag_gather: the same rows, no arithmetic)
            sink = torch.empty(hga.hga_diag_gather_sink_words(cfg, w.n_q), dtype=torch.int32,
                               device=dev)
            gat = hga.prepare("hga_diag_gather", cfg, K, V, w.p0, w.n_q, ids, sink)
            gbytes = abytes - (w.Hq * w.n_q * w.D * 2 * 2 + w.Hq * w.n_q * 4)
            g_cold = med(gat, pre=lambda: flush.fill_(1))
            g_warm = med(gat, pre=lambda: flush[:1].fill_(1))
            res["layer16k_gather_only_cold_us"] = g_cold * 1e3
            res["layer16k_gather_only_warm_us"] = g_warm * 1e3
            res["layer16k_gather_only_cold_GBps"] = gbytes / (g_cold * 1e-3) / 1e9
            del flush
        del Q, K, V, S, ids, O, lse
    return res


def group_timings(torch, hga, inputs, dev):
    """The second routing level at the 16K layer (16 routed chunks, best 64
    of their 128 groups per block): each call HIP-event timed alone (median
    of 10), and the whole group-level forward of one layer (chunk and group
    summaries of the active segment, both routers, group attention)."""
    w = inputs.LAYER16K_GROUPS
    x = inputs.generate(w)

    def up(a):
        return torch.from_numpy(a).to(torch.bfloat16).to(dev)

    Q, K, V = up(x["Q"]), up(x["K"]), up(x["V"])
    cfg = hga.make_config(w.Hq, w.Hkv, w.k)
    nb = w.n_q // C
    S = torch.zeros((w.Hkv, w.T // C, w.D), device=dev)
    SG = torch.zeros((w.Hkv, w.T // hga.HGA_GROUP, w.D), device=dev)
    ids = torch.empty((w.Hkv, nb, w.k), dtype=torch.int32, device=dev)
    gids = torch.empty((w.Hkv, nb, w.m), dtype=torch.int32, device=dev)
    O = torch.empty((w.Hq, w.n_q, w.D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.Hq, w.n_q), device=dev)
    hga.hga_summarize(cfg, K, 0, w.T, S)
    hga.hga_summarize_groups(cfg, K, 0, w.T, SG)
    calls = {
        "summarize": hga.prepare("hga_summarize", cfg, K, w.p0, w.n_q, S),
        "summarize_groups": hga.prepare("hga_summarize_groups", cfg, K, w.p0, w.n_q, SG),
        "route": hga.prepare("hga_route", cfg, Q, w.p0, S, w.T // C, ids),
        "route_groups": hga.prepare("hga_route_groups", cfg, Q, w.p0, SG, ids, gids),
        "attend_fwd_groups": hga.prepare("hga_attend_fwd_groups", cfg, Q, K, V, w.p0, gids,
                                         O, lse),
    }
    for fn in calls.values():
        fn()
    res = {}
    for name, fn in calls.items():
        if name != "summarize":
            res[f"groups16k_{name}_us"] = _median_ms(torch, fn) * 1e3

    def layer():
        for fn in calls.values():
            fn()

    # both routing levels and the group attention in one call
    fused = hga.prepare("hga_route_attend_fwd_groups", cfg, Q, K, V, w.p0, S, w.T // C, SG, ids,
                        gids, O, lse)
    fused()
    res["groups16k_route_attend_fwd_groups_us"] = _median_ms(torch, fused) * 1e3

    def layer_fused():
        calls["summarize"]()
        calls["summarize_groups"]()
        fused()

    # backward of the group attention at the same layer (dO ~ N(0, 1))
    dO = up(np.random.default_rng(5).standard_normal((w.Hq, w.n_q, w.D), dtype=np.float32))
    dQ = torch.empty((w.Hq, w.n_q, w.D), device=dev)
    dK = torch.empty((w.Hkv, w.n_q, w.D), device=dev)
    dV = torch.empty((w.Hkv, w.n_q, w.D), device=dev)
    ws = torch.empty(hga.hga_attend_bwd_workspace_bytes(cfg, w.n_q), dtype=torch.uint8,
                     device=dev)
    bwd = hga.prepare("hga_attend_bwd_groups", cfg, Q, K, V, w.p0, gids, O, lse, dO, dQ, dK,
                      dV, ws)

    ms = _median_ms(torch, layer)
    ms_fused = _median_ms(torch, layer_fused)
    ms_bwd = _median_ms(torch, bwd)
    n2, nw = hga.hga_diag_bwd_second_pass(cfg, w.n_q, ws)
    res["groups16k_bwd_dq_second_pass_workgroups"] = f"{n2} of {nw}"
    g = gids.cpu().numpy()
    fl_bwd = bwd_flops(g, w.n_q, w.G, w.D, w.p0, unit=hga.HGA_GROUP)
    fl = attend_flops(g, w.n_q, w.G, w.D, w.p0, unit=hga.HGA_GROUP)
    ab = attend_bytes(g, w.n_q, w.Hq, w.D, w.p0, unit=hga.HGA_GROUP)
    t_att = res["groups16k_attend_fwd_groups_us"] * 1e-6
    res.update({
        "groups16k_layer_fwd_us": ms * 1e3,
        "groups16k_query_tokens_per_s": w.n_q / (ms * 1e-3),
        "groups16k_fused_layer_fwd_us": ms_fused * 1e3,
        "groups16k_fused_query_tokens_per_s": w.n_q / (ms_fused * 1e-3),
        "groups16k_group_top_k": w.m,
        "groups16k_attend_algorithmic_gflop": fl / 1e9,
        "groups16k_attend_tflops": fl / t_att / 1e12,
        "groups16k_attend_gathered_GBps": ab / t_att / 1e9,
        "groups16k_bwd_us": ms_bwd * 1e3,
        "groups16k_bwd_algorithmic_gflop": fl_bwd / 1e9,
        "groups16k_bwd_tflops": fl_bwd / (ms_bwd * 1e-3) / 1e12,
    })
    return res


def variant_timings(torch, hga, inputs, dev):
    """The routing variants at the 16K layer, each call HIP-event timed alone
    (median of 20): per-query-head routing (one id row per query head, so the
    G heads of a kv head gather their chunks separately) through the fused
    route + attention, the routing alone, the attention alone and the
    backward; strictly causal routing (hga_route_causal) beside the default
    router."""
    w = inputs.LAYER16K
    x = inputs.generate(w)

    def up(a):
        return torch.from_numpy(a).to(torch.bfloat16).to(dev)

    Q, K, V = up(x["Q"]), up(x["K"]), up(x["V"])
    nb = w.n_q // C
    cfg_h = hga.make_config(w.Hq, w.Hkv, w.k, route_heads=hga.HGA_ROUTE_PER_Q_HEAD)
    cfg = hga.make_config(w.Hq, w.Hkv, w.k)
    S = torch.empty((w.Hkv, w.T // C, w.D), device=dev)
    hga.hga_summarize(cfg, K, 0, w.T, S)
    ids_h = torch.empty((w.Hq, nb, w.k), dtype=torch.int32, device=dev)
    ids = torch.empty((w.Hkv, nb, w.k), dtype=torch.int32, device=dev)
    O = torch.empty((w.Hq, w.n_q, w.D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.Hq, w.n_q), device=dev)
    dO = up(np.random.default_rng(6).standard_normal((w.Hq, w.n_q, w.D), dtype=np.float32))
    Q_prev = up(np.random.default_rng(7).standard_normal((w.Hq, C, w.D), dtype=np.float32))
    dQ = torch.empty((w.Hq, w.n_q, w.D), device=dev)
    dK = torch.empty((w.Hkv, w.n_q, w.D), device=dev)
    dV = torch.empty((w.Hkv, w.n_q, w.D), device=dev)
    ws = torch.empty(hga.hga_attend_bwd_workspace_bytes(cfg_h, w.n_q), dtype=torch.uint8,
                     device=dev)
    calls = {
        "perhead16k_route_attend": hga.prepare("hga_route_attend_fwd", cfg_h, Q, K, V, w.p0, S,
                                               w.T // C, ids_h, O, lse),
        "perhead16k_route": hga.prepare("hga_route", cfg_h, Q, w.p0, S, w.T // C, ids_h),
        "perhead16k_attend": hga.prepare("hga_attend_fwd", cfg_h, Q, K, V, w.p0, ids_h, O, lse),
        "perhead16k_bwd": hga.prepare("hga_attend_bwd", cfg_h, Q, K, V, w.p0, ids_h, O, lse, dO,
                                      dQ, dK, dV, ws),
        "causal16k_route": hga.prepare("hga_route_causal", cfg, Q, Q_prev, w.p0, S, w.T // C,
                                       ids),
        "default16k_route": hga.prepare("hga_route", cfg, Q, w.p0, S, w.T // C, ids),
    }
    res = {}
    for name, fn in calls.items():
        fn()
        res[f"{name}_us"] = _median_ms(torch, fn) * 1e3
    calls["perhead16k_route_attend"]()
    calls["perhead16k_bwd"]()
    n2, nw = hga.hga_diag_bwd_second_pass(cfg_h, w.n_q, ws)
    res["perhead16k_bwd_dq_second_pass_workgroups"] = f"{n2} of {nw}"
    torch.cuda.synchronize()
    g = ids_h.cpu().numpy()                    # one row per query head: G = 1 per unit
    fl = attend_flops(g, w.n_q, 1, w.D, w.p0)
    ab = attend_bytes(g, w.n_q, w.Hq, w.D, w.p0)
    fl_bwd = bwd_flops(g, w.n_q, 1, w.D, w.p0)
    t_att = res["perhead16k_attend_us"] * 1e-6
    res.update({
        "perhead16k_query_tokens_per_s": w.n_q / (res["perhead16k_route_attend_us"] * 1e-6),
        "perhead16k_attend_algorithmic_gflop": fl / 1e9,
        "perhead16k_attend_tflops": fl / t_att / 1e12,
        "perhead16k_attend_gathered_GBps": ab / t_att / 1e9,
        "perhead16k_attend_hbm_frac": ab / t_att / 8e12,
        "perhead16k_bwd_algorithmic_gflop": fl_bwd / 1e9,
        "perhead16k_bwd_tflops": fl_bwd / (res["perhead16k_bwd_us"] * 1e-6) / 1e12,
    })
    return res


def decode_timings(torch, hga, inputs, dev):
    """Routed decode at batch 1: one token after the 128K-history workload's
    last position (k = 32) and 8 tokens after the 16K layer's (k = 16), each
    call HIP-event timed (median of 20): the routing and the attention calls,
    the two in turn, and the step as one hga_route_attend_decode call.
    Algorithmic bytes: the summaries each token scores, its routed and open
    chunks' K and V (bf16), Q read and O written."""
    res = {}

    def up(a):
        return torch.from_numpy(a).to(torch.bfloat16).to(dev)

    for w, n_q, tag in ((inputs.LAYER128K, 1, "decode128k_1tok"),
                        (inputs.LAYER16K, 8, "decode16k_8tok")):
        x = inputs.generate(w)
        K, V = up(x["K"]), up(x["V"])
        Q = up(np.ascontiguousarray(x["Q"][:, :n_q]))
        p0 = w.T - n_q
        cfg = hga.make_config(w.Hq, w.Hkv, w.k)
        n_closed = (p0 + n_q - 1) // C
        S = torch.empty((w.Hkv, n_closed, w.D), device=dev)
        hga.hga_summarize(cfg, K, 0, n_closed * C, S)
        ids = torch.empty((w.Hkv, n_q, w.k), dtype=torch.int32, device=dev)
        O = torch.empty((w.Hq, n_q, w.D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.Hq, n_q), device=dev)
        ws = torch.empty(hga.hga_decode_workspace_bytes(cfg, p0, n_q), dtype=torch.uint8,
                         device=dev)
        route = hga.prepare("hga_route_decode", cfg, Q, p0, S, n_closed, ids, ws)
        attend = hga.prepare("hga_attend_decode", cfg, Q, K, V, p0, ids, O, lse, ws)
        ws_f = torch.empty(hga.hga_route_attend_decode_workspace_bytes(cfg, p0, n_q),
                           dtype=torch.uint8, device=dev)
        step = hga.prepare("hga_route_attend_decode", cfg, Q, K, V, p0, S, n_closed, ids, O,
                           lse, ws_f)

        def two_calls():
            route()
            attend()

        t_route = _median_ms(torch, route)
        t_att = _median_ms(torch, attend)
        t_two = _median_ms(torch, two_calls)
        t_step = _median_ms(torch, step)
        toks = p0 + np.arange(n_q)
        n_sum = float(sum(t // C for t in toks)) * w.Hkv
        n_tiles = float((ids.cpu().numpy() >= 0).sum() + w.Hkv * n_q)
        route_bytes = n_sum * w.D * 4 + w.Hq * n_q * w.D * 2
        att_bytes = n_tiles * C * w.D * 2 * 2 + w.Hq * n_q * w.D * 2 * 2
        res.update({
            f"{tag}_route_us": t_route * 1e3,
            f"{tag}_attend_us": t_att * 1e3,
            f"{tag}_two_calls_us": t_two * 1e3,
            f"{tag}_step_us": t_step * 1e3,
            f"{tag}_tokens_per_s": n_q / (t_step * 1e-3),
            f"{tag}_algorithmic_MB": (route_bytes + att_bytes) / 1e6,
            f"{tag}_attend_GBps": att_bytes / (t_att * 1e-3) / 1e9,
            f"{tag}_step_GBps": (route_bytes + att_bytes) / (t_step * 1e-3) / 1e9,
        })
        del K, V, S
    return res


def segloop_timing(torch, hga, inputs, dev):
    """36 layers x 8 segments of the segment loop (append the segment's
    summaries, then route and attend in one call), HIP-event timed. For timing only, every layer
    reuses layer 0's draw (the loop's cost depends on shapes and on how many
    chunks each block routes to, not on the values)."""
    w = inputs.seg_layer_workload(0)
    x = inputs.generate(w)

    def up(a):
        return torch.from_numpy(a).to(torch.bfloat16).to(dev)

    K, V, Qall = up(x["K"]), up(x["V"]), up(x["Q"])
    seg = inputs.SEGLOOP_SEG_LEN
    Qs = [Qall[:, s * seg:(s + 1) * seg].contiguous() for s in range(inputs.SEGLOOP_SEGMENTS)]
    cfg = hga.make_config(w.Hq, w.Hkv, w.k)
    S = torch.zeros((w.Hkv, w.T // C, w.D), device=dev)
    ids = torch.empty((w.Hkv, seg // C, w.k), dtype=torch.int32, device=dev)
    O = torch.empty((w.Hq, seg, w.D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.Hq, seg), device=dev)

    def loop():
        for _layer in range(inputs.SEGLOOP_LAYERS):
            for s in range(inputs.SEGLOOP_SEGMENTS):
                p0 = s * seg
                hga.hga_summarize(cfg, K, p0, seg, S)
                hga.hga_route_attend_fwd(cfg, Qs[s], K, V, p0, S, (p0 + seg) // C, ids, O, lse)

    loop()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    loop()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    # every one of the 36 layers processes all 16384 query tokens once
    return {"segloop_36x8_ms": ms,
            "segloop_query_tokens_per_s_per_layer": w.T * inputs.SEGLOOP_LAYERS / (ms * 1e-3),
            "segloop_query_tokens_per_s_whole_stack": w.T / (ms * 1e-3)}


def host_cpu():
    """What the host offers: its logical CPU count (nproc), the CPUs this
    process may run on, and the CPU model."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS"), "model": model}


def cpu_baseline(inputs, w, x):
    """The CPU oracle (plain C, fp64, OpenMP over output rows) on the same
    workload: summaries of the active segment, routing of every block and
    attention of every query, repeated for about 10 s; the median pass gives
    the rate. Threads: every CPU this process may use, capped by
    OMP_NUM_THREADS when the host sets it (GPU hosts that share their CPUs
    between GPUs set it to each GPU's share)."""
    import oracle
    cpu = host_cpu()
    threads = cpu["affinity_cpus"]
    if cpu["omp_num_threads_env"]:
        try:
            threads = min(threads, int(cpu["omp_num_threads_env"]))
        except ValueError:
            pass
    oracle.set_threads(threads)
    n_cap = w.T // C
    S = oracle.summarize(x["K"], C, 0, w.p0 // C, n_cap=n_cap)

    def one_pass():
        t0 = time.perf_counter()
        oracle.summarize(x["K"], C, w.p0 // C, n_cap, out=S)
        ids = oracle.route(x["Q"], S, w.p0, w.k, w.Hkv)
        oracle.attend_fwd(x["Q"], x["K"], x["V"], ids, w.p0)
        return time.perf_counter() - t0

    times = [one_pass()]
    reps = max(2, min(30, int(10.0 / max(times[0], 1e-3))))
    times += [one_pass() for _ in range(reps)]
    t = float(np.median(times))
    return {"value": w.n_q / t, "unit": "query tokens/s", "cores": oracle.get_threads(),
            "kind": "oracle",
            "sample": f"the full {w.name} forward (active-segment summaries, routing of all "
                      f"{w.n_blocks} blocks, attention of all {w.n_q} queries x {w.Hq} heads), "
                      f"median of {len(times)} passes, {sum(times):.1f} s in total",
            "host": cpu,
            "context": {"note": "the pages' end-to-end QLoRA training throughput of Qwen3-8B "
                                "at 2,048 tokens on one Quadro RTX 5000 (gist.science "
                                "technical summary 4.2; the authors' abstract); another "
                                "machine and another measure, quoted for context only",
                        "hga_training_tokens_per_s": 217.75,
                        "dense_training_tokens_per_s": 207.02}}


if __name__ == "__main__":
    main()
