"""GPU parity of the sink window (the first sink_chunks chunks, attended by
every later block and kept out of the routing candidates) across the hot
path: routing, attention (chunk and group level, fused and separate) and the
backward, against the CPU oracle with the same sink, through the C ABI."""
import os

import numpy as np
import pytest
import torch

import oracle
from parity import (check_close, check_group_ids, check_ids, from_dev, group_candidates,
                    to_dev_bf16)
from sparse_long_context_summarize_amd import hga, inputs

pytestmark = pytest.mark.gpu

C = 64
U = hga.HGA_GROUP


@pytest.fixture(scope="module", autouse=True)
def _setup():
    oracle.set_threads(min(16, os.cpu_count() or 1))
    torch.cuda.init()
    yield


def log(msg):
    print(msg, flush=True)


def run(x, p0, k, s, m=0, fused=False, bwd=False):
    """Summaries, routing and attention with sink_chunks = s on the GPU (and
    the group level when m > 0); the backward when bwd."""
    Hq, n_q, D = x["Q"].shape
    Hkv, T, _ = x["K"].shape
    nb = n_q // C
    cfg = hga.make_config(Hq, Hkv, k, sink_chunks=s)
    Q, K, V = to_dev_bf16(x["Q"]), to_dev_bf16(x["K"]), to_dev_bf16(x["V"])
    n_valid = (p0 + n_q) // C
    S = torch.empty((Hkv, n_valid, D), device="cuda")
    hga.hga_summarize(cfg, K, 0, p0 + n_q, S)
    ids = torch.full((Hkv, nb, k), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((Hkv, nb, k), float("nan"), device="cuda")
    O = torch.full((Hq, n_q, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((Hq, n_q), float("nan"), device="cuda")
    out = {}
    if m:
        SG = torch.empty((Hkv, n_valid * (C // U), D), device="cuda")
        hga.hga_summarize_groups(cfg, K, 0, p0 + n_q, SG)
        hga.hga_route(cfg, Q, p0, S, n_valid, ids, sc)
        gids = torch.full((Hkv, nb, m), -7, dtype=torch.int32, device="cuda")
        hga.hga_route_groups(cfg, Q, p0, SG, ids, gids)
        hga.hga_attend_fwd_groups(cfg, Q, K, V, p0, gids, O, lse)
        out["gids"] = gids.cpu().numpy()
        out["SG"] = from_dev(SG)
        units = gids
    elif fused:
        hga.hga_route_attend_fwd(cfg, Q, K, V, p0, S, n_valid, ids, O, lse, sc)
        units = ids
    else:
        hga.hga_route(cfg, Q, p0, S, n_valid, ids, sc)
        hga.hga_attend_fwd(cfg, Q, K, V, p0, ids, O, lse)
        units = ids
    if bwd:
        dO = to_dev_bf16(x["dO"])
        dQ = torch.full((Hq, n_q, D), float("nan"), device="cuda")
        dK = torch.full((Hkv, n_q, D), float("nan"), device="cuda")
        dV = torch.full((Hkv, n_q, D), float("nan"), device="cuda")
        ws = torch.full((hga.hga_attend_bwd_workspace_bytes(cfg, n_q),), 255, dtype=torch.uint8,
                        device="cuda")
        if m:
            hga.hga_attend_bwd_groups(cfg, Q, K, V, p0, units, O, lse, dO, dQ, dK, dV, ws)
        else:
            hga.hga_attend_bwd(cfg, Q, K, V, p0, units, O, lse, dO, dQ, dK, dV, ws)
        out.update(dQ=dQ, dK=dK, dV=dV)
    torch.cuda.synchronize()
    out.update(ids=ids.cpu().numpy(), scores=from_dev(sc), O=from_dev(O), lse=from_dev(lse),
               S=from_dev(S))
    for n in ("dQ", "dK", "dV"):
        if n in out:
            out[n] = from_dev(out[n])
    return out


def check(x, p0, k, s, res, where, m=0):
    Hkv = x["K"].shape[0]
    S_ref = oracle.summarize(x["K"], C, 0, (p0 + x["Q"].shape[1]) // C)
    ids_ref, sig = oracle.route(x["Q"], S_ref, p0, k, Hkv, want_scores=True, sink=s * C)
    ties = check_ids(res["ids"], ids_ref, sig, p0, where=where, sink_chunks=s)
    units, unit = res["ids"], C
    if m:
        SG_ref = oracle.summarize(x["K"], U, 0, res["SG"].shape[1])
        g_ref, gsig = oracle.route_groups(x["Q"], SG_ref, p0, res["ids"], m, Hkv,
                                          want_scores=True, sink=s * C)
        check_group_ids(res["gids"], g_ref, gsig, res["ids"], p0, where=where, sink_chunks=s)
        units, unit = res["gids"], U
    O_ref, lse_ref = oracle.attend_fwd(x["Q"], x["K"], x["V"], units, p0, unit, C, sink=s * C)
    st = check_close(f"{where} O", res["O"], O_ref)
    check_close(f"{where} lse", res["lse"], lse_ref, atol=1e-3, rtol=0, rel_l2=None)
    if "dQ" in res:
        grads = oracle.attend_bwd(x["Q"], x["K"], x["V"], x["dO"], units, p0, unit, C,
                                  sink=s * C)
        for name, ref in zip(("dQ", "dK", "dV"), grads):
            check_close(f"{where} {name}", res[name], ref)
    log(f"{where}: near ties {ties}; O {st}")


@pytest.mark.parametrize("s", [1, 4])
@pytest.mark.parametrize("fused", [False, True])
def test_forward(s, fused):
    T, n_q, k = 1024, 256, 5
    x = inputs.small_random(500 + s, 8, 2, 128, T, n_q, bf16=True)
    res = run(x, T - n_q, k, s, fused=fused)
    check(x, T - n_q, k, s, res, f"sink {s} fused={fused}")
    assert np.all((res["ids"] == -1) | (res["ids"] >= s))


def test_fused_equals_separate_with_sink():
    T, n_q, k, s = 2048, 512, 7, 2
    x = inputs.small_random(510, 8, 2, 128, T, n_q, bf16=True)
    a = run(x, T - n_q, k, s)
    b = run(x, T - n_q, k, s, fused=True)
    for name in ("ids", "scores", "O", "lse"):
        np.testing.assert_array_equal(a[name], b[name], err_msg=name)


def test_sink_beyond_the_history():
    # s = 20 chunks: blocks with P/C <= 20 attend their whole history as sink
    T, n_q, k, s = 1536, 512, 3, 20
    x = inputs.small_random(511, 4, 1, 128, T, n_q, bf16=True)
    res = run(x, T - n_q, k, s)
    check(x, T - n_q, k, s, res, "sink past P")


def test_layer16k_with_one_sink_chunk():
    w = inputs.LAYER16K
    x = inputs.generate(w)
    res = run(x, w.p0, w.k, 1, fused=True)
    check(x, w.p0, w.k, 1, res, "layer16k sink 1")


@pytest.mark.parametrize("p0", [0, 768])
def test_backward(p0):
    # p0 = 0: the sink chunks are active keys attended by every later block
    T, n_q, k, s = 1024, 1024 - p0, 4, 3
    x = inputs.small_random(520 + p0, 4, 2, 128, T, n_q, bf16=True, with_dO=True)
    res = run(x, p0, k, s, bwd=True)
    check(x, p0, k, s, res, f"bwd sink p0={p0}")


@pytest.mark.parametrize("p0", [0, 768])
def test_group_level(p0):
    T, n_q, k, m, s = 1024, 1024 - p0, 4, 19, 2
    x = inputs.small_random(530 + p0, 4, 2, 128, T, n_q, bf16=True, with_dO=True)
    res = run(x, p0, k, s, m=m, bwd=True)
    check(x, p0, k, s, res, f"groups sink p0={p0}", m=m)
    for g in range(2):
        for b in range(n_q // C):
            cand = group_candidates(res["ids"][g, b], p0 + b * C, sink_chunks=s)
            row = res["gids"][g, b]
            assert np.all(np.isin(row[row >= 0], cand))


def test_gather_diagnostic_reads_the_sink():
    # the diagnostic runs with the sink and touches its rows (smoke: it returns
    # and differs from the run without the sink)
    T, n_q, k = 1024, 256, 3
    x = inputs.small_random(540, 4, 1, 128, T, n_q, bf16=True)
    K, V = to_dev_bf16(x["K"]), to_dev_bf16(x["V"])
    ids = torch.full((1, n_q // C, k), -1, dtype=torch.int32, device="cuda")
    words = []
    for s in (0, 2):
        cfg = hga.make_config(4, 1, k, sink_chunks=s)
        sink = torch.empty(hga.hga_diag_gather_sink_words(cfg, n_q), dtype=torch.int32,
                           device="cuda")
        hga.hga_diag_gather(cfg, K, V, T - n_q, n_q, ids, sink)
        torch.cuda.synchronize()
        words.append(sink.cpu().numpy())
    assert not np.array_equal(words[0], words[1])
