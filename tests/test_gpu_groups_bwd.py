"""GPU parity of hga_attend_bwd_groups (dQ; dK, dV of the active segment)
against the CPU oracle's gradients at the group level (C = 8 units, 64-query
blocks) on identical seeded inputs and the GPU's own group ids, through the C
ABI."""
import os

import numpy as np
import pytest
import torch

import oracle
from parity import check_close, from_dev, to_dev_bf16
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


def gpu_group_fwd_bwd(x, p0, k, m, gids_override=None):
    Hq, n_q, D = x["Q"].shape
    Hkv, T, _ = x["K"].shape
    nb = n_q // C
    cfg = hga.make_config(Hq, Hkv, k)
    Q, K, V, dO = (to_dev_bf16(x[n]) for n in ("Q", "K", "V", "dO"))
    S = torch.zeros((Hkv, T // C, D), device="cuda")
    SG = torch.zeros((Hkv, T // U, D), device="cuda")
    hga.hga_summarize(cfg, K, 0, T, S)
    hga.hga_summarize_groups(cfg, K, 0, T, SG)
    ids = torch.empty((Hkv, nb, k), dtype=torch.int32, device="cuda")
    hga.hga_route(cfg, Q, p0, S, (p0 + n_q) // C, ids)
    gids = torch.empty((Hkv, nb, m), dtype=torch.int32, device="cuda")
    hga.hga_route_groups(cfg, Q, p0, SG, ids, gids)
    if gids_override is not None:
        gids = torch.from_numpy(np.ascontiguousarray(gids_override, dtype=np.int32)).cuda()
    O = torch.empty((Hq, n_q, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((Hq, n_q), device="cuda")
    hga.hga_attend_fwd_groups(cfg, Q, K, V, p0, gids, O, lse)
    nan = float("nan")
    dQ = torch.full((Hq, n_q, D), nan, device="cuda")
    dK = torch.full((Hkv, n_q, D), nan, device="cuda")
    dV = torch.full((Hkv, n_q, D), nan, device="cuda")
    ws = torch.full((hga.hga_attend_bwd_workspace_bytes(cfg, n_q),), 255, dtype=torch.uint8,
                    device="cuda")
    hga.hga_attend_bwd_groups(cfg, Q, K, V, p0, gids, O, lse, dO, dQ, dK, dV, ws)
    torch.cuda.synchronize()
    return dict(ids=ids.cpu().numpy(), gids=gids.cpu().numpy(), dQ=from_dev(dQ),
                dK=from_dev(dK), dV=from_dev(dV),
                dev=dict(cfg=cfg, Q=Q, K=K, V=V, dO=dO, ids=ids, gids=gids, O=O, lse=lse, ws=ws))


def check_grads(x, p0, res, where, dq_mask=None):
    dQ, dK, dV = oracle.attend_bwd(x["Q"], x["K"], x["V"], x["dO"], res["gids"], p0, C=U,
                                   Bq=C, dq_mask=dq_mask)
    st = {}
    for name, ref in (("dQ", dQ), ("dK", dK), ("dV", dV)):
        assert np.all(np.isfinite(res[name])), f"{where} {name}: unwritten or non-finite"
        st[name] = check_close(f"{where} {name}", res[name], ref)
    log(f"{where}: {st}")


@pytest.mark.parametrize("m", [1, 13, 16, 31])
def test_tiny(m):
    w = inputs.TINY
    x = inputs.generate(w.replace(with_dO=True), bf16=True)
    res = gpu_group_fwd_bwd(x, w.p0, w.k, m)
    check_grads(x, w.p0, res, f"tiny m={m}")


def test_every_group_matches_chunk_backward():
    """m = 8k: the group backward must agree with hga_attend_bwd on the chunk
    ids (the same attended sets)."""
    w = inputs.TINY
    x = inputs.generate(w.replace(with_dO=True), bf16=True)
    res = gpu_group_fwd_bwd(x, w.p0, w.k, U * w.k)
    check_grads(x, w.p0, res, "tiny all groups")
    d = res["dev"]
    dQ = torch.empty_like(d["Q"], dtype=torch.float32)
    dK = torch.empty((w.Hkv, w.n_q, w.D), device="cuda")
    dV = torch.empty_like(dK)
    O = torch.empty_like(d["O"])
    lse = torch.empty_like(d["lse"])
    hga.hga_attend_fwd(d["cfg"], d["Q"], d["K"], d["V"], w.p0, d["ids"], O, lse)
    hga.hga_attend_bwd(d["cfg"], d["Q"], d["K"], d["V"], w.p0, d["ids"], O, lse, d["dO"], dQ, dK,
                       dV, d["ws"])
    torch.cuda.synchronize()
    for name, t in (("dQ", dQ), ("dK", dK), ("dV", dV)):
        check_close(f"groups vs chunks {name}", res[name], from_dev(t), atol=4e-3, rtol=1e-2)


def test_bwd16k_groups():
    w = inputs.BWD16K
    x = inputs.generate(w)
    log(f"bwd16k groups: {w}, m = {inputs.LAYER16K_GROUPS.m}")
    res = gpu_group_fwd_bwd(x, w.p0, w.k, inputs.LAYER16K_GROUPS.m)
    check_grads(x, w.p0, res, "bwd16k groups")


def test_bwd16k_groups_deterministic():
    w = inputs.BWD16K
    x = inputs.generate(w)
    a = gpu_group_fwd_bwd(x, w.p0, w.k, inputs.LAYER16K_GROUPS.m)
    d = a["dev"]
    dQ = torch.empty_like(d["Q"], dtype=torch.float32)
    dK = torch.empty((w.Hkv, w.n_q, w.D), device="cuda")
    dV = torch.empty_like(dK)
    hga.hga_attend_bwd_groups(d["cfg"], d["Q"], d["K"], d["V"], w.p0, d["gids"], d["O"],
                              d["lse"], d["dO"], dQ, dK, dV, d["ws"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(from_dev(dQ), a["dQ"])
    np.testing.assert_array_equal(from_dev(dK), a["dK"])
    np.testing.assert_array_equal(from_dev(dV), a["dV"])


@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (2, 1), (8, 2), (8, 1)])
@pytest.mark.parametrize("k,m", [(3, 5), (7, 27), (7, 56)])
def test_head_layouts_and_budgets(Hq, Hkv, k, m):
    T, n_q = 1024, 256
    x = inputs.small_random(400 + Hq * 10 + k, Hq, Hkv, 128, T, n_q, bf16=True, with_dO=True)
    res = gpu_group_fwd_bwd(x, T - n_q, k, m)
    check_grads(x, T - n_q, res, f"Hq={Hq} Hkv={Hkv} k={k} m={m}")


def test_first_segment_every_key_active():
    # p0 = 0: later blocks choose subsets of the groups of earlier active
    # chunks, so the key-major pass must apply per-block group masks
    T = n_q = 1024
    x = inputs.small_random(41, 4, 1, 128, T, n_q, bf16=True, with_dO=True)
    res = gpu_group_fwd_bwd(x, 0, 6, 20)
    check_grads(x, 0, res, "p0=0 k=6 m=20")


def test_messy_group_rows():
    """Repeats, any order, -1 and ids outside [0, P/8) in the group rows, and
    partial last tiles; active-segment groups chosen by later blocks."""
    T, n_q = 1024, 256
    x = inputs.small_random(42, 4, 1, 128, T, n_q, bf16=True, with_dO=True)
    p0 = T - n_q                                     # block b: P/8 = 96 + 8b
    rng = np.random.default_rng(9)
    m = 40
    g = np.full((1, n_q // C, m), -1, np.int32)
    g[0, 0] = rng.integers(0, 96, m)                 # history only, repeats
    g[0, 1, :10] = [96, 97, 96, 103, 5, 104, -2, 99, 99, 1 << 30]   # active chunk 12 groups
    g[0, 2, :7] = [111, 96, 100, 104, 105, 104, 3]   # groups of active chunks 12, 13
    g[0, 3] = (np.arange(m) * 3) % 120               # history and active, unsorted order
    res = gpu_group_fwd_bwd(x, p0, 4, 8, gids_override=g)
    check_grads(x, p0, res, "messy group rows")
