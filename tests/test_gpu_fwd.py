"""GPU parity of the forward hot path (hga_summarize -> hga_route ->
hga_attend_fwd) against the CPU oracle on identical seeded inputs, through the
C ABI. Attention parity is measured on the GPU's own ids once those pass the
id rule (tests/parity.py)."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from parity import (GAP, check_close, check_ids, from_dev, summary_bound, to_dev_bf16)
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


def gpu_forward(x, p0, k, *, T_cap=None, n_cap=None, ids_override=None, split_summarize=True):
    """Run the three calls on the GPU. x holds bf16-representable float32
    arrays Q [Hq][n_q][D], K/V [Hkv][T][D] with T >= p0 + n_q."""
    Hq, n_q, D = x["Q"].shape
    Hkv, T, _ = x["K"].shape
    T_cap = T if T_cap is None else T_cap
    n_valid = (p0 + n_q) // C
    n_cap = n_valid if n_cap is None else n_cap
    nb = n_q // C
    cfg = hga.make_config(Hq, Hkv, k)
    Qd = to_dev_bf16(x["Q"])
    Kd = torch.zeros((Hkv, T_cap, D), dtype=torch.bfloat16, device="cuda")
    Vd = torch.zeros((Hkv, T_cap, D), dtype=torch.bfloat16, device="cuda")
    Kd[:, :T] = to_dev_bf16(x["K"])
    Vd[:, :T] = to_dev_bf16(x["V"])
    S = torch.full((Hkv, n_cap, D), float("nan"), device="cuda")
    if split_summarize:
        hga.hga_summarize(cfg, Kd, 0, p0, S)           # history
        hga.hga_summarize(cfg, Kd, p0, n_q, S)         # append the active segment
    else:
        hga.hga_summarize(cfg, Kd, 0, p0 + n_q, S)
    ids = torch.full((Hkv, nb, k), -7, dtype=torch.int32, device="cuda")
    scores = torch.full((Hkv, nb, k), float("nan"), device="cuda")
    hga.hga_route(cfg, Qd, p0, S, n_valid, ids, scores)
    if ids_override is not None:
        ids = torch.from_numpy(np.ascontiguousarray(ids_override, dtype=np.int32)).cuda()
        cfg = hga.make_config(Hq, Hkv, ids.shape[2])
    O = torch.full((Hq, n_q, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((Hq, n_q), float("nan"), device="cuda")
    hga.hga_attend_fwd(cfg, Qd, Kd, Vd, p0, ids, O, lse)
    torch.cuda.synchronize()
    return dict(S=from_dev(S), ids=ids.cpu().numpy(), scores=from_dev(scores),
                O=from_dev(O), lse=from_dev(lse), dev=dict(Q=Qd, K=Kd, V=Vd, ids=ids, cfg=cfg))


def check_summaries(x, res, p0, n_q, where=""):
    n_valid = (p0 + n_q) // C
    S_ref = oracle.summarize(x["K"], C, 0, n_valid)
    err = np.abs(res["S"][:, :n_valid] - S_ref)
    bound = summary_bound(x["K"], 0, n_valid)
    assert np.all(err <= bound), f"{where} summaries: max err {err.max()} (bound {bound.min()})"
    assert np.isnan(res["S"][:, n_valid:]).all(), f"{where}: rows past the range were written"
    return S_ref


def check_route(x, res, S_ref, p0, k, where=""):
    Hkv = x["K"].shape[0]
    ids_ref, sigma = oracle.route(x["Q"], S_ref, p0, k, Hkv, want_scores=True)
    ties = check_ids(res["ids"], ids_ref, sigma, p0, where=where)
    # the GPU's fp32 score of each id it wrote, against the oracle's fp64 score
    Hkv, nb, _ = res["ids"].shape
    for g in range(Hkv):
        for b in range(nb):
            row = res["ids"][g, b]
            n = int((row >= 0).sum())
            nE = (p0 + b * C) // C
            if nE == 0:
                assert np.all(np.isneginf(res["scores"][g, b])), where
                continue
            M = np.max(np.abs(sigma[g, b, :nE]))
            ref = sigma[g, b, row[:n]]
            assert np.all(np.abs(res["scores"][g, b, :n] - ref) <= GAP * M), (where, g, b)
            assert np.all(np.isneginf(res["scores"][g, b, n:])), (where, g, b)
    return ids_ref, ties


def check_attend(x, res, p0, unit_mask=None, where=""):
    O_ref, lse_ref = oracle.attend_fwd(x["Q"], x["K"], x["V"], res["ids"], p0,
                                       unit_mask=unit_mask)
    s1 = check_close(f"{where} O", res["O"], O_ref)
    check_close(f"{where} lse", res["lse"], lse_ref)
    s2 = check_close(f"{where} lse (tight)", res["lse"], lse_ref, atol=1e-3, rtol=0, rel_l2=None)
    return s1, s2


def full_check(x, p0, k, res, unit_mask=None, where=""):
    S_ref = check_summaries(x, res, p0, x["Q"].shape[1], where)
    _, ties = check_route(x, res, S_ref, p0, k, where)
    stats = check_attend(x, res, p0, unit_mask, where)
    log(f"{where}: near-tie id rows {ties}; O {stats[0]}; lse {stats[1]}")


# ------------------------------------------------------------------ workloads

def test_tiny_k4():
    w = inputs.TINY
    x = inputs.generate(w, bf16=True)       # the GPU consumes bf16 copies
    log(f"tiny k=4: {w}")
    res = gpu_forward(x, w.p0, 4)
    full_check(x, w.p0, 4, res, where="tiny k=4")


def test_tiny_k_all_is_dense_causal():
    w = inputs.TINY
    x = inputs.generate(w, bf16=True)
    res = gpu_forward(x, w.p0, 31)
    full_check(x, w.p0, 31, res, where="tiny k=31")
    assert np.all(res["ids"][0, -1] == np.arange(31))
    # against dense causal attention (torch float64, explicit bottom-right mask)
    q = torch.from_numpy(x["Q"].astype(np.float64))
    kk = torch.from_numpy(x["K"].astype(np.float64))
    vv = torch.from_numpy(x["V"].astype(np.float64))
    M = torch.from_numpy(np.arange(w.T)[None, :] <= (w.p0 + np.arange(w.n_q))[:, None])
    O_dense = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, attn_mask=M,
                                                               scale=1 / math.sqrt(w.D))
    check_close("tiny dense O", res["O"], O_dense.numpy())


def test_layer16k():
    w = inputs.LAYER16K
    log(f"layer16k: {w}")
    x = inputs.generate(w)
    res = gpu_forward(x, w.p0, w.k)
    full_check(x, w.p0, w.k, res, where="layer16k")


def test_layer128k():
    """The 128K-history workload: summaries, every id row, and every output
    row of every (block, query head) unit against the oracle."""
    w = inputs.LAYER128K
    log(f"layer128k: {w}")
    x = inputs.generate(w)
    res = gpu_forward(x, w.p0, w.k)
    full_check(x, w.p0, w.k, res, where="layer128k")


def test_determinism_layer16k():
    w = inputs.LAYER16K
    x = inputs.generate(w)
    a = gpu_forward(x, w.p0, w.k)
    b = gpu_forward(x, w.p0, w.k)
    for name in ("S", "ids", "scores", "O", "lse"):
        np.testing.assert_array_equal(a[name], b[name], err_msg=name)


# ------------------------------------------------------------- segment loop

def _segment_layers(layers):
    for layer in layers:
        w = inputs.seg_layer_workload(layer)
        x = inputs.generate(w)
        Hq, Hkv, D = w.Hq, w.Hkv, w.D
        cfg = hga.make_config(Hq, Hkv, w.k)
        Kd, Vd = to_dev_bf16(x["K"]), to_dev_bf16(x["V"])
        Qd = to_dev_bf16(x["Q"])
        n_cap = w.T // C
        S = torch.full((Hkv, n_cap, D), float("nan"), device="cuda")
        S_ref = oracle.summarize(x["K"], C, 0, n_cap)
        rng = np.random.default_rng(layer)
        for s in range(inputs.SEGLOOP_SEGMENTS):
            p0 = s * inputs.SEGLOOP_SEG_LEN
            n_q = inputs.SEGLOOP_SEG_LEN
            nb = n_q // C
            Qs = Qd[:, p0:p0 + n_q].contiguous()
            # append this segment's keys first: its blocks route over them too
            hga.hga_summarize(cfg, Kd, p0, n_q, S)
            ids = torch.empty((Hkv, nb, w.k), dtype=torch.int32, device="cuda")
            scores = torch.empty((Hkv, nb, w.k), device="cuda")
            hga.hga_route(cfg, Qs, p0, S, (p0 + n_q) // C, ids, scores)
            O = torch.empty((Hq, n_q, D), dtype=torch.bfloat16, device="cuda")
            lse = torch.empty((Hq, n_q), device="cuda")
            hga.hga_attend_fwd(cfg, Qs, Kd, Vd, p0, ids, O, lse)
            torch.cuda.synchronize()
            where = f"segloop layer {layer} seg {s}"
            Sg = from_dev(S)
            rows = slice(p0 // C, (p0 + n_q) // C)
            err = np.abs(Sg[:, rows] - S_ref[:, rows])
            assert np.all(err <= summary_bound(x["K"], rows.start, rows.stop)), where
            assert np.isnan(Sg[:, (p0 + n_q) // C:]).all(), where
            xs = dict(Q=x["Q"][:, p0:p0 + n_q], K=x["K"], V=x["V"])
            res = dict(ids=ids.cpu().numpy(), scores=from_dev(scores), O=from_dev(O),
                       lse=from_dev(lse))
            check_route(xs, res, S_ref, p0, w.k, where)
            mask = np.zeros((Hq, nb), np.uint8)
            for h, b in zip(rng.integers(0, Hq, 3), rng.integers(0, nb, 3)):
                mask[h, b] = 1
            mask[rng.integers(Hq), nb - 1] = 1
            check_attend(xs, res, p0, mask, where)
        log(f"segloop layer {layer}: 8 segments ok")


@pytest.mark.parametrize("group", range(6))
def test_segment_loop(group):
    _segment_layers(range(6 * group, 6 * group + 6))


@pytest.mark.parametrize("layer", [0, 35])
def test_segment_loop_fused_every_unit(layer):
    """One layer of the segment loop through the calls the benchmark times:
    hga_summarize appends the segment's chunks, then hga_route_attend_fwd
    routes and attends in one launch; summaries, ids, scores and every row of
    O and lse of all 8 segments are compared with the oracle."""
    w = inputs.seg_layer_workload(layer)
    x = inputs.generate(w)
    Hq, Hkv, D = w.Hq, w.Hkv, w.D
    cfg = hga.make_config(Hq, Hkv, w.k)
    Kd, Vd, Qd = to_dev_bf16(x["K"]), to_dev_bf16(x["V"]), to_dev_bf16(x["Q"])
    n_cap = w.T // C
    S = torch.full((Hkv, n_cap, D), float("nan"), device="cuda")
    S_ref = oracle.summarize(x["K"], C, 0, n_cap)
    for s in range(inputs.SEGLOOP_SEGMENTS):
        p0 = s * inputs.SEGLOOP_SEG_LEN
        n_q = inputs.SEGLOOP_SEG_LEN
        nb = n_q // C
        Qs = Qd[:, p0:p0 + n_q].contiguous()
        where = f"segloop fused layer {layer} seg {s}"
        log(where)
        hga.hga_summarize(cfg, Kd, p0, n_q, S)
        ids = torch.full((Hkv, nb, w.k), -7, dtype=torch.int32, device="cuda")
        scores = torch.full((Hkv, nb, w.k), float("nan"), device="cuda")
        O = torch.full((Hq, n_q, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((Hq, n_q), float("nan"), device="cuda")
        hga.hga_route_attend_fwd(cfg, Qs, Kd, Vd, p0, S, (p0 + n_q) // C, ids, O, lse, scores)
        torch.cuda.synchronize()
        Sg = from_dev(S)
        rows = slice(p0 // C, (p0 + n_q) // C)
        err = np.abs(Sg[:, rows] - S_ref[:, rows])
        assert np.all(err <= summary_bound(x["K"], rows.start, rows.stop)), where
        xs = dict(Q=x["Q"][:, p0:p0 + n_q], K=x["K"], V=x["V"])
        res = dict(ids=ids.cpu().numpy(), scores=from_dev(scores), O=from_dev(O),
                   lse=from_dev(lse))
        check_route(xs, res, S_ref, p0, w.k, where)
        check_attend(xs, res, p0, None, where)


# ----------------------------------------------------------------- edge cases

@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (2, 1), (8, 2), (8, 1), (16, 8)])
@pytest.mark.parametrize("k", [0, 1, 7])
def test_head_layouts_and_budgets(Hq, Hkv, k):
    T, n_q = 1024, 256
    x = inputs.small_random(100 + Hq * 10 + k, Hq, Hkv, 128, T, n_q, bf16=True)
    p0 = T - n_q
    log(f"edge Hq={Hq} Hkv={Hkv} k={k}")
    res = gpu_forward(x, p0, k)
    full_check(x, p0, k, res, where=f"Hq={Hq} Hkv={Hkv} k={k}")


def test_first_segment_and_full_budget():
    # p0 = 0: block 0 has no candidates, block b has b; k = 256 > any |E|
    T = n_q = 512
    x = inputs.small_random(7, 4, 1, 128, T, n_q, bf16=True)
    res = gpu_forward(x, 0, 256)
    full_check(x, 0, 256, res, where="p0=0 k=256")
    assert np.all(res["ids"][0, 0] == -1)


def test_max_top_k_with_many_candidates():
    T, n_q = 64 * 300, 128          # 298 and 299 candidates, k = 256
    x = inputs.small_random(8, 4, 2, 128, T, n_q, bf16=True)
    res = gpu_forward(x, T - n_q, 256)
    full_check(x, T - n_q, 256, res, where="k=256 of ~300")


def test_capacity_beyond_the_segment():
    # K/V buffer and summary buffer larger than needed; one summarize call
    T, n_q = 1024, 128
    x = inputs.small_random(9, 8, 2, 128, T, n_q, bf16=True)
    res = gpu_forward(x, T - n_q, 5, T_cap=T + 4096, n_cap=200, split_summarize=False)
    full_check(x, T - n_q, 5, res, where="T_cap > p0+n_q")


def test_single_block_segment():
    T, n_q = 640, 64
    x = inputs.small_random(10, 4, 1, 128, T, n_q, bf16=True)
    res = gpu_forward(x, T - n_q, 3)
    full_check(x, T - n_q, 3, res, where="n_q=64")


def test_ids_outside_the_causal_range_are_skipped():
    T, n_q = 1024, 256
    x = inputs.small_random(11, 4, 1, 128, T, n_q, bf16=True)
    p0 = T - n_q
    ids = np.array([[[-1, 2, 5, -1, 9, 11],       # P/C = 12 for block 0
                     [0, -5, 12, 13, 40, 10 ** 6],  # block 1: 12 eligible, 13 = P/C is not
                     [-1, -1, -1, -1, -1, -1],
                     [1, 3, 14, 15, 16, 2 ** 30]]], dtype=np.int32)
    res = gpu_forward(x, p0, 6, ids_override=ids)
    # the oracle skips ids outside [0, P/C) by the same definition (the local
    # chunk listed again, e.g. 15 in block 3, must not be counted twice)
    O_ref, lse_ref = oracle.attend_fwd(x["Q"], x["K"], x["V"], ids, p0)
    check_close("skip O", res["O"], O_ref)
    check_close("skip lse", res["lse"], lse_ref, atol=1e-3, rtol=0, rel_l2=None)


def test_route_beyond_2048_candidates():
    # 2198 / 2199 eligible chunks per block: the wave-level two-stage selection
    T, n_q = 64 * 2200, 128
    x = inputs.small_random(12, 4, 1, 128, T, n_q, bf16=True)
    res = gpu_forward(x, T - n_q, 32)
    full_check(x, T - n_q, 32, res, where="2200 candidates")


@pytest.mark.parametrize("n_chunks", [32, 2200])
def test_route_exact_ties_take_lowest_ids(n_chunks):
    """Chunks repeated bit for bit give equal scores on both sides, so the
    tie rule alone (higher score, then lower chunk id) fixes every id: the
    GPU must reproduce the oracle's ids exactly (register selection for 32
    chunks, the two-stage selection for 2200)."""
    rng = np.random.default_rng(n_chunks)
    Hq, Hkv, D, n_q, k = 4, 2, 128, 256, 7
    T = n_chunks * C
    p0 = T - n_q
    x = inputs.small_random(13, Hq, Hkv, D, T, n_q, bf16=True)
    # five key patterns with well separated offsets; chunk c repeats pattern c % 5
    pats = rng.standard_normal((Hkv, 5, C, D)).astype(np.float32)
    pats += (0.4 * np.arange(5, dtype=np.float32))[None, :, None, None]
    pats = inputs.round_bf16(pats)
    K = np.empty((Hkv, T, D), np.float32)
    for c in range(n_chunks):
        K[:, c * C:(c + 1) * C] = pats[:, c % 5]
    x["K"] = K
    res = gpu_forward(x, p0, k)
    S_ref = check_summaries(x, res, p0, n_q, "ties")
    ids_ref = oracle.route(x["Q"], S_ref, p0, k, Hkv)
    np.testing.assert_array_equal(res["ids"], ids_ref)
    check_attend(x, res, p0, where="ties")


def test_repeated_and_unsorted_ids_count_once():
    """A caller's id row is a set: repeats are attended once, in any order
    (the oracle takes the same definition); k = 80 also exercises rows longer
    than one wave's 64 lanes."""
    T, n_q, k = 1024, 256, 80
    x = inputs.small_random(14, 4, 1, 128, T, n_q, bf16=True)
    p0 = T - n_q
    rng = np.random.default_rng(5)
    ids = np.full((1, n_q // C, k), -1, np.int32)
    ids[0, 0] = rng.integers(0, 12, k)                    # 80 draws of 12 ids
    ids[0, 1, :6] = [9, 2, 9, 7, 2, 2]                    # unsorted with repeats
    ids[0, 2, :4] = [3, 3, 3, 3]
    ids[0, 3] = np.arange(k) % 15                         # 0..14, each >= 5 times
    res = gpu_forward(x, p0, k, ids_override=ids)
    O_ref, lse_ref = oracle.attend_fwd(x["Q"], x["K"], x["V"], ids, p0)
    check_close("repeats O", res["O"], O_ref)
    check_close("repeats lse", res["lse"], lse_ref, atol=1e-3, rtol=0, rel_l2=None)


@pytest.mark.parametrize("sink", [0, 2])
def test_zero_query_block_over_2200_candidates(sink):
    """A query block of zeros scores every chunk exactly 0, so every candidate
    ties and the tie rule alone fixes the ids (the lowest candidates past the
    sink). With 2198-2199 candidates this runs the two-stage selection, whose
    threshold search must then take exactly k keys; both the routing kernel
    and the fused routing + attention kernel are checked against the oracle."""
    Hq, Hkv, D, n_q, k = 4, 2, 128, 128, 16
    T = 64 * 2200
    p0 = T - n_q
    x = inputs.small_random(21, Hq, Hkv, D, T, n_q, bf16=True)
    x["Q"][:, :C] = 0.0                            # block 0 of every head
    n_valid = T // C
    cfg = hga.make_config(Hq, Hkv, k, sink_chunks=sink)
    Qd, Kd, Vd = to_dev_bf16(x["Q"]), to_dev_bf16(x["K"]), to_dev_bf16(x["V"])
    S = torch.empty((Hkv, n_valid, D), device="cuda")
    hga.hga_summarize(cfg, Kd, 0, T, S)
    S_ref = oracle.summarize(x["K"], C, 0, n_valid)
    ids_ref, sigma = oracle.route(x["Q"], S_ref, p0, k, Hkv, want_scores=True, sink=64 * sink)
    assert np.array_equal(ids_ref[:, 0], np.tile(np.arange(sink, sink + k), (Hkv, 1)))
    for fused in (False, True):
        ids = torch.full((Hkv, n_q // C, k), -7, dtype=torch.int32, device="cuda")
        O = torch.full((Hq, n_q, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((Hq, n_q), float("nan"), device="cuda")
        log(f"zero block, 2200 candidates, sink {sink}, fused {fused}")
        if fused:
            hga.hga_route_attend_fwd(cfg, Qd, Kd, Vd, p0, S, n_valid, ids, O, lse)
        else:
            hga.hga_route(cfg, Qd, p0, S, n_valid, ids)
            hga.hga_attend_fwd(cfg, Qd, Kd, Vd, p0, ids, O, lse)
        torch.cuda.synchronize()
        got = ids.cpu().numpy()
        np.testing.assert_array_equal(got[:, 0], ids_ref[:, 0])
        check_ids(got, ids_ref, sigma, p0, sink_chunks=sink, where="zero block")
        O_ref, lse_ref = oracle.attend_fwd(x["Q"], x["K"], x["V"], got, p0, sink=64 * sink)
        check_close("zero block O", from_dev(O), O_ref)
        check_close("zero block lse", from_dev(lse), lse_ref, atol=1e-3, rtol=0, rel_l2=None)
