"""Seeded random shapes through the fused entry points against the oracle:
hga_summarize + hga_route_attend_fwd (chunk routing, then attention),
hga_summarize_groups + hga_route_attend_fwd_groups (both routing levels,
then group attention) and hga_attend_bwd after the fused forward (per kv
head and per query head), with mixed head layouts (G = 1, 2, 4, 8), budgets,
sink windows, history lengths and segment lengths. Ids pass under the gap
rule, outputs under the bf16 bar (tests/parity.py)."""
import os

import numpy as np
import pytest
import torch

import oracle
from parity import check_close, check_group_ids, check_ids, from_dev, to_dev_bf16
from sparse_long_context_summarize_amd import hga, inputs

pytestmark = pytest.mark.gpu

C = 64
U = hga.HGA_GROUP


@pytest.fixture(scope="module", autouse=True)
def _setup():
    oracle.set_threads(min(16, os.cpu_count() or 1))
    torch.cuda.init()
    yield


def _shape(seed):
    r = np.random.default_rng(seed)
    Hkv = int(r.choice([1, 2, 4, 8]))
    G = int(r.choice([1, 2, 4, 8]))
    while Hkv * G > 32:
        G //= 2
    n_q = C * int(r.integers(1, 5))
    p0 = C * int(r.integers(0, 24))
    sink = int(r.integers(0, 3))
    k = int(r.integers(1, 21))
    m = int(r.integers(1, 8 * k + 1))
    return Hkv * G, Hkv, n_q, p0, sink, k, m


def _inputs(seed, Hq, Hkv, n_q, p0):
    x = inputs.small_random(9000 + seed, Hq, Hkv, 128, p0 + n_q, n_q, bf16=True)
    return x, to_dev_bf16(x["Q"]), to_dev_bf16(x["K"]), to_dev_bf16(x["V"])


def _check_chunk_ids(x, ids, p0, k, sink, where):
    Hkv = x["K"].shape[0]
    n_valid = (p0 + x["Q"].shape[1]) // C
    S_ref = oracle.summarize(x["K"], C, 0, n_valid)
    ids_ref, sigma = oracle.route(x["Q"], S_ref, p0, k, Hkv, want_scores=True, sink=sink * C)
    check_ids(ids, ids_ref, sigma, p0, where=where, sink_chunks=sink)


@pytest.mark.parametrize("seed", range(12))
def test_random_shape_route_attend(seed):
    Hq, Hkv, n_q, p0, sink, k, _ = _shape(seed)
    where = f"seed {seed}: Hq={Hq} Hkv={Hkv} n_q={n_q} p0={p0} sink={sink} k={k}"
    print(where, flush=True)
    x, Qd, Kd, Vd = _inputs(seed, Hq, Hkv, n_q, p0)
    cfg = hga.make_config(Hq, Hkv, k, sink_chunks=sink)
    n_valid = (p0 + n_q) // C
    S = torch.zeros((Hkv, n_valid, 128), device="cuda")
    hga.hga_summarize(cfg, Kd, 0, p0 + n_q, S)
    ids = torch.full((Hkv, n_q // C, k), -7, dtype=torch.int32, device="cuda")
    O = torch.full((Hq, n_q, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((Hq, n_q), float("nan"), device="cuda")
    hga.hga_route_attend_fwd(cfg, Qd, Kd, Vd, p0, S, n_valid, ids, O, lse)
    torch.cuda.synchronize()
    ids = ids.cpu().numpy()
    _check_chunk_ids(x, ids, p0, k, sink, where)
    O_ref, lse_ref = oracle.attend_fwd(x["Q"], x["K"], x["V"], ids, p0, sink=sink * C)
    check_close(f"{where} O", from_dev(O), O_ref)
    check_close(f"{where} lse", from_dev(lse), lse_ref, atol=1e-3, rtol=0, rel_l2=None)


@pytest.mark.parametrize("seed", range(8))
def test_random_shape_route_attend_groups(seed):
    Hq, Hkv, n_q, p0, sink, k, m = _shape(100 + seed)
    where = f"seed {seed}: Hq={Hq} Hkv={Hkv} n_q={n_q} p0={p0} sink={sink} k={k} m={m}"
    print(where, flush=True)
    x, Qd, Kd, Vd = _inputs(100 + seed, Hq, Hkv, n_q, p0)
    cfg = hga.make_config(Hq, Hkv, k, sink_chunks=sink)
    n_valid = (p0 + n_q) // C
    S = torch.zeros((Hkv, n_valid, 128), device="cuda")
    SG = torch.zeros((Hkv, n_valid * (C // U), 128), device="cuda")
    hga.hga_summarize(cfg, Kd, 0, p0 + n_q, S)
    hga.hga_summarize_groups(cfg, Kd, 0, p0 + n_q, SG)
    nb = n_q // C
    ids = torch.full((Hkv, nb, k), -7, dtype=torch.int32, device="cuda")
    gids = torch.full((Hkv, nb, m), -7, dtype=torch.int32, device="cuda")
    O = torch.full((Hq, n_q, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((Hq, n_q), float("nan"), device="cuda")
    hga.hga_route_attend_fwd_groups(cfg, Qd, Kd, Vd, p0, S, n_valid, SG, ids, gids, O, lse)
    torch.cuda.synchronize()
    ids, gids = ids.cpu().numpy(), gids.cpu().numpy()
    _check_chunk_ids(x, ids, p0, k, sink, where)
    SG_ref = oracle.summarize(x["K"], U, 0, n_valid * (C // U))
    gids_ref, gsig = oracle.route_groups(x["Q"], SG_ref, p0, ids, m, Hkv, want_scores=True,
                                         sink=sink * C)
    check_group_ids(gids, gids_ref, gsig, ids, p0, where=where, sink_chunks=sink)
    O_ref, lse_ref = oracle.attend_fwd(x["Q"], x["K"], x["V"], gids, p0, C=U, sink=sink * C)
    check_close(f"{where} O", from_dev(O), O_ref)
    check_close(f"{where} lse", from_dev(lse), lse_ref, atol=1e-3, rtol=0, rel_l2=None)


@pytest.mark.parametrize("seed", range(8))
def test_random_shape_backward(seed):
    # odd seeds route per query head (one id row per query head)
    Hq, Hkv, n_q, p0, sink, k, _ = _shape(200 + seed)
    per_q = seed % 2 == 1
    where = (f"seed {seed}: Hq={Hq} Hkv={Hkv} n_q={n_q} p0={p0} sink={sink} k={k} "
             f"per_q_head={per_q}")
    print(where, flush=True)
    x = inputs.small_random(9200 + seed, Hq, Hkv, 128, p0 + n_q, n_q, bf16=True, with_dO=True)
    Qd, Kd, Vd, dOd = (to_dev_bf16(x[n]) for n in ("Q", "K", "V", "dO"))
    cfg = hga.make_config(Hq, Hkv, k, sink_chunks=sink,
                          route_heads=hga.HGA_ROUTE_PER_Q_HEAD if per_q else
                          hga.HGA_ROUTE_PER_KV_HEAD)
    n_valid = (p0 + n_q) // C
    S = torch.zeros((Hkv, n_valid, 128), device="cuda")
    hga.hga_summarize(cfg, Kd, 0, p0 + n_q, S)
    ids = torch.full(((Hq if per_q else Hkv), n_q // C, k), -7, dtype=torch.int32, device="cuda")
    O = torch.empty((Hq, n_q, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((Hq, n_q), device="cuda")
    hga.hga_route_attend_fwd(cfg, Qd, Kd, Vd, p0, S, n_valid, ids, O, lse)
    nan = float("nan")
    dQ = torch.full((Hq, n_q, 128), nan, device="cuda")
    dK = torch.full((Hkv, n_q, 128), nan, device="cuda")
    dV = torch.full((Hkv, n_q, 128), nan, device="cuda")
    ws = torch.full((hga.hga_attend_bwd_workspace_bytes(cfg, n_q),), 255, dtype=torch.uint8,
                    device="cuda")
    hga.hga_attend_bwd(cfg, Qd, Kd, Vd, p0, ids, O, lse, dOd, dQ, dK, dV, ws)
    torch.cuda.synchronize()
    ids = ids.cpu().numpy()
    refs = oracle.attend_bwd(x["Q"], x["K"], x["V"], x["dO"], ids, p0, sink=sink * C,
                             per_q_head=per_q)
    for name, got, ref in zip(("dQ", "dK", "dV"), (dQ, dK, dV), refs):
        got = from_dev(got)
        assert np.all(np.isfinite(got)), f"{where} {name}: unwritten or non-finite"
        check_close(f"{where} {name}", got, ref)
