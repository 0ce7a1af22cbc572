"""GPU edge cases through the C ABI: empty calls (no queries, no tokens)
return without touching any buffer; the largest sink window (64 chunks); the
largest candidate count the router takes (24576 chunks) for block routing
and for decode routing."""
import os

import numpy as np
import pytest
import torch

import oracle
from parity import check_close, check_ids, from_dev, to_dev_bf16
from sparse_long_context_summarize_amd import hga, inputs

pytestmark = pytest.mark.gpu

C = 64


@pytest.fixture(scope="module", autouse=True)
def _setup():
    oracle.set_threads(min(16, os.cpu_count() or 1))
    torch.cuda.init()
    yield


def log(msg):
    print(msg, flush=True)


def test_empty_calls_touch_nothing():
    Hq, Hkv, D, T, k = 4, 2, 128, 1024, 4
    x = inputs.small_random(800, Hq, Hkv, D, T, 64, bf16=True)
    cfg = hga.make_config(Hq, Hkv, k, sink_chunks=1)
    K, V = to_dev_bf16(x["K"]), to_dev_bf16(x["V"])
    S = torch.full((Hkv, T // C, D), float("nan"), device="cuda")
    SG = torch.full((Hkv, T // 8, D), float("nan"), device="cuda")
    hga.hga_summarize(cfg, K, 512, 0, S)
    hga.hga_summarize_groups(cfg, K, 512, 0, SG)
    Q0 = torch.empty((Hq, 0, D), dtype=torch.bfloat16, device="cuda")
    ids0 = torch.empty((Hkv, 0, k), dtype=torch.int32, device="cuda")
    O0 = torch.empty((Hq, 0, D), dtype=torch.bfloat16, device="cuda")
    lse0 = torch.empty((Hq, 0), device="cuda")
    hga.hga_route(cfg, Q0, 512, S, 0, ids0)
    hga.hga_route_causal(cfg, Q0, None, 0, S, 0, ids0)
    hga.hga_attend_fwd(cfg, Q0, K, V, 512, ids0, O0, lse0)
    hga.hga_route_attend_fwd(cfg, Q0, K, V, 512, S, 0, ids0, O0, lse0)
    ws = torch.empty(max(1, hga.hga_attend_bwd_workspace_bytes(cfg, 0)), dtype=torch.uint8,
                     device="cuda")
    dQ0 = torch.empty((Hq, 0, D), device="cuda")
    dK0 = torch.empty((Hkv, 0, D), device="cuda")
    hga.hga_attend_bwd(cfg, Q0, K, V, 512, ids0, O0, lse0, O0, dQ0, dK0, dK0.clone(), ws)
    gids0 = torch.empty((Hkv, 0, 8), dtype=torch.int32, device="cuda")
    hga.hga_route_groups(cfg, Q0, 512, SG, ids0, gids0)
    hga.hga_attend_fwd_groups(cfg, Q0, K, V, 512, gids0, O0, lse0)
    wsd = torch.empty(max(1, hga.hga_decode_workspace_bytes(cfg, 700, 0)), dtype=torch.uint8,
                      device="cuda")
    dids0 = torch.empty((Hkv, 0, k), dtype=torch.int32, device="cuda")
    hga.hga_route_decode(cfg, Q0, 700, S, 10, dids0, wsd)
    hga.hga_attend_decode(cfg, Q0, K, V, 700, dids0, O0, lse0, wsd)
    torch.cuda.synchronize()
    assert torch.isnan(S).all() and torch.isnan(SG).all()


def test_largest_sink_window():
    s, T, n_q, k = hga.HGA_MAX_SINK_CHUNKS, 64 * 80, 512, 4
    x = inputs.small_random(801, 4, 2, 128, T, n_q, bf16=True)
    p0 = T - n_q
    cfg = hga.make_config(4, 2, k, sink_chunks=s)
    Q, K, V = to_dev_bf16(x["Q"]), to_dev_bf16(x["K"]), to_dev_bf16(x["V"])
    S = torch.empty((2, T // C, 128), device="cuda")
    hga.hga_summarize(cfg, K, 0, T, S)
    ids = torch.full((2, n_q // C, k), -7, dtype=torch.int32, device="cuda")
    O = torch.empty((4, n_q, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((4, n_q), device="cuda")
    hga.hga_route_attend_fwd(cfg, Q, K, V, p0, S, T // C, ids, O, lse)
    torch.cuda.synchronize()
    S_ref = oracle.summarize(x["K"], C, 0, T // C)
    ids_ref, sig = oracle.route(x["Q"], S_ref, p0, k, 2, want_scores=True, sink=s * C)
    g_ids = ids.cpu().numpy()
    check_ids(g_ids, ids_ref, sig, p0, sink_chunks=s, where="sink 64")
    O_ref, lse_ref = oracle.attend_fwd(x["Q"], x["K"], x["V"], g_ids, p0, sink=s * C)
    st = check_close("sink 64 O", from_dev(O), O_ref)
    check_close("sink 64 lse", from_dev(lse), lse_ref, atol=1e-3, rtol=0, rel_l2=None)
    log(f"sink 64: O {st}")
    # one chunk past the limit is refused before any launch
    with pytest.raises(hga.HGAError):
        hga.hga_route(hga.make_config(4, 2, k, sink_chunks=s + 1), Q, p0, S, T // C, ids)


@pytest.fixture(scope="module")
def huge():
    # 24576 candidate chunks before the block at p0, one kv head
    n_c = 24576
    T = C * (n_c + 1)
    x = inputs.small_random(802, 2, 1, 128, T, C, bf16=True)
    K = to_dev_bf16(x["K"])
    cfg = hga.make_config(2, 1, 32)
    S = torch.empty((1, T // C, 128), device="cuda")
    hga.hga_summarize(cfg, K, 0, T, S)
    S_ref = oracle.summarize(x["K"], C, 0, T // C)
    return x, K, S, S_ref, n_c


def test_route_with_the_most_candidates(huge):
    x, K, S, S_ref, n_c = huge
    p0 = C * n_c
    cfg = hga.make_config(2, 1, 32)
    ids = torch.full((1, 1, 32), -7, dtype=torch.int32, device="cuda")
    hga.hga_route(cfg, to_dev_bf16(x["Q"]), p0, S, n_c, ids)
    torch.cuda.synchronize()
    ids_ref, sig = oracle.route(x["Q"], S_ref, p0, 32, 1, want_scores=True)
    check_ids(ids.cpu().numpy(), ids_ref, sig, p0, where="24576 candidates")
    # one candidate more than the router keeps is refused
    T2 = C * (n_c + 2)
    with pytest.raises(hga.HGAError):
        S2 = torch.empty((1, T2 // C, 128), device="cuda")
        hga.hga_route(cfg, to_dev_bf16(x["Q"]), p0 + C, S2, n_c + 1, ids)


def test_decode_route_with_the_most_candidates(huge):
    x, K, S, S_ref, n_c = huge
    p0 = C * n_c + 5                                # open chunk n_c: candidates 0 .. n_c-1
    Q = x["Q"][:, :1]
    cfg = hga.make_config(2, 1, 32)
    ids = torch.full((1, 1, 32), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(hga.hga_decode_workspace_bytes(cfg, p0, 1), dtype=torch.uint8,
                     device="cuda")
    hga.hga_route_decode(cfg, to_dev_bf16(Q), p0, S, n_c, ids, ws)
    torch.cuda.synchronize()
    ids_ref, sig = oracle.route_decode(Q, S_ref, p0, 32, 1, want_scores=True)
    check_ids(ids.cpu().numpy(), ids_ref, sig, p0, Bq=1, where="decode 24576 candidates")


@pytest.mark.parametrize("gain", [6.0, 24.0])
def test_peaked_softmax_forward_and_backward(gain):
    """Queries scaled up: logits spread over tens of units, so the running max
    keeps growing (rescales) and single keys take almost all the weight (the
    backward's high/low split of large probabilities)."""
    Hq, Hkv, D, T, n_q, k = 8, 2, 128, 1024, 256, 5
    x = inputs.small_random(810 + int(gain), Hq, Hkv, D, T, n_q, bf16=True, with_dO=True)
    x["Q"] = inputs.round_bf16(x["Q"] * np.float32(gain))
    p0 = T - n_q
    cfg = hga.make_config(Hq, Hkv, k)
    Q, K, V = to_dev_bf16(x["Q"]), to_dev_bf16(x["K"]), to_dev_bf16(x["V"])
    S = torch.empty((Hkv, T // C, D), device="cuda")
    hga.hga_summarize(cfg, K, 0, T, S)
    ids = torch.empty((Hkv, n_q // C, k), dtype=torch.int32, device="cuda")
    O = torch.empty((Hq, n_q, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((Hq, n_q), device="cuda")
    hga.hga_route_attend_fwd(cfg, Q, K, V, p0, S, T // C, ids, O, lse)
    dO = to_dev_bf16(x["dO"])
    dQ = torch.empty((Hq, n_q, D), device="cuda")
    dK = torch.empty((Hkv, n_q, D), device="cuda")
    dV = torch.empty((Hkv, n_q, D), device="cuda")
    ws = torch.empty(hga.hga_attend_bwd_workspace_bytes(cfg, n_q), dtype=torch.uint8,
                     device="cuda")
    hga.hga_attend_bwd(cfg, Q, K, V, p0, ids, O, lse, dO, dQ, dK, dV, ws)
    torch.cuda.synchronize()
    g_ids = ids.cpu().numpy()
    O_ref, lse_ref = oracle.attend_fwd(x["Q"], x["K"], x["V"], g_ids, p0)
    st = check_close(f"gain {gain} O", from_dev(O), O_ref)
    check_close(f"gain {gain} lse", from_dev(lse), lse_ref, atol=1e-3, rtol=0, rel_l2=None)
    grads = oracle.attend_bwd(x["Q"], x["K"], x["V"], x["dO"], g_ids, p0)
    for name, got, ref in zip(("dQ", "dK", "dV"), (dQ, dK, dV), grads):
        check_close(f"gain {gain} {name}", from_dev(got), ref)
    log(f"gain {gain}: O {st}")
