"""GPU parity of the second routing level (hga_summarize_groups ->
hga_route_groups -> hga_attend_fwd_groups) against the CPU oracle on the
same seeded inputs, through the C ABI. Group routing runs on the GPU's own
chunk ids once those pass the chunk id rule, and attention on the GPU's own
group ids once those pass the group id rule (tests/parity.py)."""
import os

import numpy as np
import pytest
import torch

import oracle
from parity import (GAP, check_close, check_group_ids, check_ids, from_dev,
                    group_candidates, summary_bound, to_dev_bf16)
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


def gpu_group_forward(x, p0, k, m, *, ids_override=None, gids_override=None,
                      n_gcap=None, T_cap=None):
    """Chunk summaries, chunk routing, group summaries, group routing and
    group attention on the GPU. x holds bf16-representable float32 arrays."""
    Hq, n_q, D = x["Q"].shape
    Hkv, T, _ = x["K"].shape
    T_cap = T if T_cap is None else T_cap
    nb = n_q // C
    n_valid = (p0 + n_q) // C
    n_gcap = n_valid * (C // U) if n_gcap is None else n_gcap
    cfg = hga.make_config(Hq, Hkv, k)
    Qd = to_dev_bf16(x["Q"])
    Kd = torch.zeros((Hkv, T_cap, D), dtype=torch.bfloat16, device="cuda")
    Vd = torch.zeros((Hkv, T_cap, D), dtype=torch.bfloat16, device="cuda")
    Kd[:, :T] = to_dev_bf16(x["K"])
    Vd[:, :T] = to_dev_bf16(x["V"])
    S = torch.full((Hkv, n_valid, D), float("nan"), device="cuda")
    hga.hga_summarize(cfg, Kd, 0, p0 + n_q, S)
    SG = torch.full((Hkv, n_gcap, D), float("nan"), device="cuda")
    hga.hga_summarize_groups(cfg, Kd, 0, p0, SG)        # history
    hga.hga_summarize_groups(cfg, Kd, p0, n_q, SG)      # the active segment
    ids = torch.full((Hkv, nb, k), -7, dtype=torch.int32, device="cuda")
    hga.hga_route(cfg, Qd, p0, S, n_valid, ids)
    if ids_override is not None:
        ids = torch.from_numpy(np.ascontiguousarray(ids_override, dtype=np.int32)).cuda()
        cfg = hga.make_config(Hq, Hkv, ids.shape[2])
    gids = torch.full((Hkv, nb, m), -7, dtype=torch.int32, device="cuda")
    gsc = torch.full((Hkv, nb, m), float("nan"), device="cuda")
    hga.hga_route_groups(cfg, Qd, p0, SG, ids, gids, gsc)
    if gids_override is not None:
        gids = torch.from_numpy(np.ascontiguousarray(gids_override, dtype=np.int32)).cuda()
    O = torch.full((Hq, n_q, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((Hq, n_q), float("nan"), device="cuda")
    hga.hga_attend_fwd_groups(cfg, Qd, Kd, Vd, p0, gids, O, lse)
    torch.cuda.synchronize()
    return dict(S=from_dev(S), SG=from_dev(SG), ids=ids.cpu().numpy(),
                gids=gids.cpu().numpy(), gscores=from_dev(gsc), O=from_dev(O),
                lse=from_dev(lse), dev=dict(Q=Qd, K=Kd, V=Vd, S=S, SG=SG, ids=ids, gids=gids))


def check_group_summaries(x, res, p0, n_q, where=""):
    n_g = (p0 + n_q) // U
    SG_ref = oracle.summarize(x["K"], U, 0, n_g)
    err = np.abs(res["SG"][:, :n_g] - SG_ref)
    bound = summary_bound(x["K"], 0, n_g, C=U)
    assert np.all(err <= bound), f"{where} group summaries: max err {err.max()}"
    assert np.isnan(res["SG"][:, n_g:]).all(), f"{where}: groups past the range were written"
    return SG_ref


def check_group_route(x, res, SG_ref, p0, m, where=""):
    """Group ids against the oracle's, both given the GPU's chunk ids; the
    GPU's fp32 score of each group it wrote against the oracle's fp64 one."""
    Hkv = x["K"].shape[0]
    gids_ref, sigma = oracle.route_groups(x["Q"], SG_ref, p0, res["ids"], m, Hkv,
                                          want_scores=True)
    ties = check_group_ids(res["gids"], gids_ref, sigma, res["ids"], p0, where=where)
    _, nb, _ = res["gids"].shape
    for g in range(Hkv):
        for b in range(nb):
            row = res["gids"][g, b]
            n = int((row >= 0).sum())
            cand = group_candidates(res["ids"][g, b], p0 + b * C)
            if cand.size == 0:
                assert n == 0 and np.all(np.isneginf(res["gscores"][g, b])), (where, g, b)
                continue
            M = np.max(np.abs(sigma[g, b, cand]))
            assert np.all(np.abs(res["gscores"][g, b, :n] - sigma[g, b, row[:n]]) <= GAP * M), \
                (where, g, b)
            assert np.all(np.isneginf(res["gscores"][g, b, n:])), (where, g, b)
    return gids_ref, ties


def check_group_attend(x, res, p0, unit_mask=None, where=""):
    O_ref, lse_ref = oracle.attend_fwd(x["Q"], x["K"], x["V"], res["gids"], p0, C=U, Bq=C,
                                       unit_mask=unit_mask)
    s1 = check_close(f"{where} O", res["O"], O_ref)
    check_close(f"{where} lse", res["lse"], lse_ref)
    s2 = check_close(f"{where} lse (tight)", res["lse"], lse_ref, atol=1e-3, rtol=0,
                     rel_l2=None)
    return s1, s2


def full_group_check(x, p0, k, m, res, unit_mask=None, where=""):
    n_q = x["Q"].shape[1]
    Hkv = x["K"].shape[0]
    S_ref = oracle.summarize(x["K"], C, 0, (p0 + n_q) // C)
    err = np.abs(res["S"] - S_ref)
    assert np.all(err <= summary_bound(x["K"], 0, (p0 + n_q) // C)), where
    ids_ref, sigma = oracle.route(x["Q"], S_ref, p0, k, Hkv, want_scores=True)
    chunk_ties = check_ids(res["ids"], ids_ref, sigma, p0, where=where)
    SG_ref = check_group_summaries(x, res, p0, n_q, where)
    _, ties = check_group_route(x, res, SG_ref, p0, m, where)
    stats = check_group_attend(x, res, p0, unit_mask, where)
    log(f"{where}: near-tie rows chunk {chunk_ties} group {ties}; O {stats[0]}; "
        f"lse {stats[1]}")


# ------------------------------------------------------------------ workloads

@pytest.mark.parametrize("m", [0, 1, 13, 16, 31])
def test_tiny_budgets(m):
    w = inputs.TINY
    x = inputs.generate(w, bf16=True)
    log(f"tiny groups k={w.k} m={m}")
    res = gpu_group_forward(x, w.p0, w.k, m)
    full_group_check(x, w.p0, w.k, m, res, where=f"tiny m={m}")


def test_every_group_is_chunk_attention():
    """m = 8k keeps every group of the routed chunks: the attended set equals
    hga_attend_fwd's on the same chunk ids, so the two kernels must agree."""
    w = inputs.TINY
    x = inputs.generate(w, bf16=True)
    m = U * w.k
    res = gpu_group_forward(x, w.p0, w.k, m)
    full_group_check(x, w.p0, w.k, m, res, where="tiny all groups")
    for b in range(w.n_blocks):
        assert np.array_equal(res["gids"][0, b], group_candidates(res["ids"][0, b],
                                                                  w.p0 + b * C)), b
    d = res["dev"]
    cfg = hga.make_config(w.Hq, w.Hkv, w.k)
    O = torch.empty_like(d["Q"])
    lse = torch.empty((w.Hq, w.n_q), device="cuda")
    hga.hga_attend_fwd(cfg, d["Q"], d["K"], d["V"], w.p0, d["ids"], O, lse)
    torch.cuda.synchronize()
    check_close("groups vs chunks O", res["O"], from_dev(O), atol=4e-3, rtol=1e-2)
    check_close("groups vs chunks lse", res["lse"], from_dev(lse), atol=1e-4, rtol=0,
                rel_l2=None)


def test_layer16k_groups():
    w = inputs.LAYER16K_GROUPS
    log(f"layer16k groups: {w}")
    x = inputs.generate(w)
    res = gpu_group_forward(x, w.p0, w.k, w.m)
    full_group_check(x, w.p0, w.k, w.m, res, where="layer16k groups")


def test_layer16k_groups_deterministic():
    w = inputs.LAYER16K_GROUPS
    x = inputs.generate(w)
    a = gpu_group_forward(x, w.p0, w.k, w.m)
    b = gpu_group_forward(x, w.p0, w.k, w.m)
    for name in ("SG", "gids", "gscores", "O", "lse"):
        np.testing.assert_array_equal(a[name], b[name], err_msg=name)


# ----------------------------------------------------------------- edge cases

@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (2, 1), (8, 2), (8, 1), (16, 8)])
@pytest.mark.parametrize("k,m", [(1, 3), (3, 8), (7, 27), (7, 56)])
def test_head_layouts_and_budgets(Hq, Hkv, k, m):
    T, n_q = 1024, 256
    x = inputs.small_random(200 + Hq * 10 + k, Hq, Hkv, 128, T, n_q, bf16=True)
    p0 = T - n_q
    log(f"groups Hq={Hq} Hkv={Hkv} k={k} m={m}")
    res = gpu_group_forward(x, p0, k, m)
    full_group_check(x, p0, k, m, res, where=f"Hq={Hq} Hkv={Hkv} k={k} m={m}")


def test_first_segment_and_largest_budgets():
    # p0 = 0: block 0 has no candidate chunk, so no candidate group
    T = n_q = 512
    x = inputs.small_random(21, 4, 1, 128, T, n_q, bf16=True)
    res = gpu_group_forward(x, 0, 256, 2048)
    full_group_check(x, 0, 256, 2048, res, where="p0=0 k=256 m=2048")
    assert np.all(res["gids"][0, 0] == -1)


def test_2048_candidate_groups():
    # 256 routed chunks of ~300: 2048 candidate groups per block, m = 200
    T, n_q = 64 * 300, 128
    x = inputs.small_random(22, 4, 2, 128, T, n_q, bf16=True)
    res = gpu_group_forward(x, T - n_q, 256, 200)
    full_group_check(x, T - n_q, 256, 200, res, where="2048 candidate groups")


def test_capacity_beyond_the_segment():
    T, n_q = 1024, 128
    x = inputs.small_random(23, 8, 2, 128, T, n_q, bf16=True)
    res = gpu_group_forward(x, T - n_q, 5, 19, n_gcap=T // U + 300, T_cap=T + 4096)
    full_group_check(x, T - n_q, 5, 19, res, where="capacity")


def test_exact_ties_take_lowest_group_ids():
    """Repeated key patterns give bit-equal group scores on both sides, so the
    tie rule alone (higher score, then lower group id) fixes every group id."""
    rng = np.random.default_rng(24)
    Hq, Hkv, D, n_q, k, m = 4, 2, 128, 256, 7, 20
    n_chunks = 40
    T = n_chunks * C
    p0 = T - n_q
    x = inputs.small_random(24, Hq, Hkv, D, T, n_q, bf16=True)
    # chunk c repeats chunk pattern c % 5; inside a pattern, groups 0-3 and
    # 4-7 repeat each other, so ties occur across and within chunks
    pats = rng.standard_normal((Hkv, 5, C // 2, D)).astype(np.float32)
    pats += (0.4 * np.arange(5, dtype=np.float32))[None, :, None, None]
    pats = inputs.round_bf16(np.concatenate([pats, pats], axis=2))
    K = np.empty((Hkv, T, D), np.float32)
    for c in range(n_chunks):
        K[:, c * C:(c + 1) * C] = pats[:, c % 5]
    x["K"] = K
    res = gpu_group_forward(x, p0, k, m)
    S_ref = oracle.summarize(x["K"], C, 0, (p0 + n_q) // C)
    np.testing.assert_array_equal(res["ids"], oracle.route(x["Q"], S_ref, p0, k, Hkv))
    SG_ref = check_group_summaries(x, res, p0, n_q, "ties")
    gids_ref = oracle.route_groups(x["Q"], SG_ref, p0, res["ids"], m, Hkv)
    np.testing.assert_array_equal(res["gids"], gids_ref)
    check_group_attend(x, res, p0, where="ties")


def test_messy_chunk_rows():
    """Chunk rows are sets: repeats, unsorted order, -1 and ids outside
    [0, P/C) (the local chunk included) add no candidates."""
    T, n_q, k, m = 1024, 256, 9, 20
    x = inputs.small_random(25, 4, 1, 128, T, n_q, bf16=True)
    p0 = T - n_q
    ids = np.array([[[3, 3, 11, -1, 0, 12, 3, 5, 99],        # P/C = 12
                     [12, 13, 2, 2, 2, -4, 7, 7, 1],           # 12 valid, 13 is the local
                     [-1] * 9,
                     [14, 15, 0, 1, 2, 3, 4, 5, 6]]], dtype=np.int32)
    res = gpu_group_forward(x, p0, k, m, ids_override=ids)
    SG_ref = check_group_summaries(x, res, p0, n_q, "messy")
    check_group_route(x, res, SG_ref, p0, m, "messy")
    assert np.all(res["gids"][0, 2] == -1)
    check_group_attend(x, res, p0, where="messy")


def test_messy_group_rows():
    """Group rows are sets too: repeats, any order, -1, and ids outside
    [0, P/8) are skipped; counts that are not multiples of 8 leave a partial
    last tile (the 8-group tile is padded and masked)."""
    T, n_q = 1024, 256
    x = inputs.small_random(26, 4, 1, 128, T, n_q, bf16=True)
    p0 = T - n_q                                       # P/8 = 96 for block 0
    rng = np.random.default_rng(3)
    m = 70
    g = np.full((1, n_q // C, m), -1, np.int32)
    g[0, 0] = rng.integers(0, 96, m)                   # repeats, unsorted
    g[0, 1, :9] = [104, 103, 96, 0, 0, 5, -3, 2 ** 30, 103]   # P/8 = 104
    g[0, 2, :3] = [111, 1, 111]
    g[0, 3] = np.arange(m) * 1 + 50                    # 70 distinct, last tile 6 of 8
    res = gpu_group_forward(x, p0, 4, 8, gids_override=g)
    check_group_attend(x, res, p0, where="messy groups")


# ------------------------------------------------ both routing levels fused

def _fused_and_separate(x, p0, k, m, sink=0):
    """hga_route_attend_fwd_groups against hga_route + hga_route_groups +
    hga_attend_fwd_groups on the same device inputs."""
    Hq, n_q, D = x["Q"].shape
    Hkv, T, _ = x["K"].shape
    nb = n_q // C
    n_valid = (p0 + n_q) // C
    n_gcap = n_valid * (C // U)
    cfg = hga.make_config(Hq, Hkv, k, sink_chunks=sink)
    Qd, Kd, Vd = to_dev_bf16(x["Q"]), to_dev_bf16(x["K"]), to_dev_bf16(x["V"])
    S = torch.zeros((Hkv, n_valid, D), device="cuda")
    SG = torch.zeros((Hkv, n_gcap, D), device="cuda")
    hga.hga_summarize(cfg, Kd, 0, p0 + n_q, S)
    hga.hga_summarize_groups(cfg, Kd, 0, p0 + n_q, SG)
    out = {}
    for tag in ("separate", "fused"):
        fill = -7 if tag == "separate" else -9
        ids = torch.full((Hkv, nb, k), fill, dtype=torch.int32, device="cuda")
        gids = torch.full((Hkv, nb, m), fill, dtype=torch.int32, device="cuda")
        gsc = torch.full((Hkv, nb, m), float(fill), device="cuda")
        O = torch.full((Hq, n_q, D), float(fill), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((Hq, n_q), float(fill), device="cuda")
        if tag == "separate":
            hga.hga_route(cfg, Qd, p0, S, n_valid, ids)
            hga.hga_route_groups(cfg, Qd, p0, SG, ids, gids, gsc)
            hga.hga_attend_fwd_groups(cfg, Qd, Kd, Vd, p0, gids, O, lse)
        else:
            hga.hga_route_attend_fwd_groups(cfg, Qd, Kd, Vd, p0, S, n_valid, SG, ids, gids, O,
                                            lse, gsc)
        torch.cuda.synchronize()
        out[tag] = dict(ids=ids.cpu().numpy(), gids=gids.cpu().numpy(), gscores=from_dev(gsc),
                        O=from_dev(O), lse=from_dev(lse))
    return out["separate"], out["fused"]


def _assert_same(a, b, where):
    for name in ("ids", "gids", "gscores", "O", "lse"):
        np.testing.assert_array_equal(b[name], a[name], err_msg=f"{where}: {name}")


@pytest.mark.parametrize("sink", [0, 2])
def test_layer16k_groups_fused(sink):
    # top_k = 16 <= 32: one launch, both routing levels in each workgroup
    w = inputs.LAYER16K_GROUPS
    x = inputs.generate(w)
    log(f"layer16k groups fused, sink {sink}")
    a, b = _fused_and_separate(x, w.p0, w.k, w.m, sink=sink)
    _assert_same(a, b, f"layer16k fused sink={sink}")
    assert (b["gids"] >= 0).sum() > 0


@pytest.mark.parametrize("Hq,Hkv,k,m,p0,sink", [
    (1, 1, 3, 20, 768, 0),      # G = 1
    (8, 4, 5, 40, 768, 1),      # G = 2, sink window
    (16, 4, 32, 256, 3840, 0),  # G = 4, the largest fused chunk budget, every group kept
    (8, 1, 7, 33, 768, 0),      # G = 8: two workgroups per unit
    (4, 1, 8, 16, 0, 0),        # first segment: block 0 has no candidates
    (4, 1, 40, 64, 3840, 0),    # top_k > 32: the three kernels in turn
])
def test_groups_fused_layouts(Hq, Hkv, k, m, p0, sink):
    n_q = 256
    T = p0 + n_q
    x = inputs.small_random(300 + Hq + k, Hq, Hkv, 128, T, n_q, bf16=True)
    log(f"groups fused Hq={Hq} Hkv={Hkv} k={k} m={m} p0={p0} sink={sink}")
    a, b = _fused_and_separate(x, p0, k, m, sink=sink)
    _assert_same(a, b, f"Hq={Hq} Hkv={Hkv} k={k} m={m} p0={p0} sink={sink}")
