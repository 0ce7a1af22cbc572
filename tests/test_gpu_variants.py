"""GPU parity of the routing variants against the CPU oracle, through the C
ABI: per-query-head routing (route_heads = HGA_ROUTE_PER_Q_HEAD: one id row
per query head, scored against its kv head's summaries) through routing,
attention (separate and fused) and the backward; and strictly causal routing
(hga_route_causal: block b scores with the 64 queries before it, taken from
Q_prev for the first block)."""
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


def run(x, p0, k, s=0, per_head=True, fused=False, bwd=False, causal=False, Q_prev=None):
    Hq, n_q, D = x["Q"].shape
    Hkv, T, _ = x["K"].shape
    nb = n_q // C
    U = Hq if per_head else Hkv
    cfg = hga.make_config(Hq, Hkv, k, sink_chunks=s,
                          route_heads=hga.HGA_ROUTE_PER_Q_HEAD if per_head
                          else hga.HGA_ROUTE_PER_KV_HEAD)
    Q, K, V = to_dev_bf16(x["Q"]), to_dev_bf16(x["K"]), to_dev_bf16(x["V"])
    n_valid = (p0 + n_q) // C
    S = torch.empty((Hkv, max(n_valid, 1), D), device="cuda")
    hga.hga_summarize(cfg, K, 0, p0 + n_q, S)
    ids = torch.full((U, nb, k), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((U, nb, k), float("nan"), device="cuda")
    O = torch.full((Hq, n_q, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((Hq, n_q), float("nan"), device="cuda")
    if causal:
        qp = to_dev_bf16(Q_prev) if Q_prev is not None else None
        hga.hga_route_causal(cfg, Q, qp, p0, S, n_valid, ids, sc)
        hga.hga_attend_fwd(cfg, Q, K, V, p0, ids, O, lse)
    elif fused:
        hga.hga_route_attend_fwd(cfg, Q, K, V, p0, S, n_valid, ids, O, lse, sc)
    else:
        hga.hga_route(cfg, Q, p0, S, n_valid, ids, sc)
        hga.hga_attend_fwd(cfg, Q, K, V, p0, ids, O, lse)
    out = {}
    if bwd:
        dO = to_dev_bf16(x["dO"])
        dQ = torch.full((Hq, n_q, D), float("nan"), device="cuda")
        dK = torch.full((Hkv, n_q, D), float("nan"), device="cuda")
        dV = torch.full((Hkv, n_q, D), float("nan"), device="cuda")
        ws = torch.full((hga.hga_attend_bwd_workspace_bytes(cfg, n_q),), 255, dtype=torch.uint8,
                        device="cuda")
        hga.hga_attend_bwd(cfg, Q, K, V, p0, ids, O, lse, dO, dQ, dK, dV, ws)
        out.update(dQ=dQ, dK=dK, dV=dV)
    torch.cuda.synchronize()
    out.update(ids=ids.cpu().numpy(), scores=from_dev(sc), O=from_dev(O), lse=from_dev(lse))
    for n in ("dQ", "dK", "dV"):
        if n in out:
            out[n] = from_dev(out[n])
    return out


def check(x, p0, k, s, res, where, per_head=True, causal=False, Q_prev=None):
    Hkv = x["K"].shape[0]
    n_q = x["Q"].shape[1]
    S_ref = oracle.summarize(x["K"], C, 0, max((p0 + n_q) // C, 1))
    ids_ref, sig = oracle.route(x["Q"], S_ref, p0, k, Hkv, want_scores=True, sink=s * C,
                                per_q_head=per_head, prev_block=causal, Q_prev=Q_prev)
    ties = check_ids(res["ids"], ids_ref, sig, p0, where=where, sink_chunks=s)
    O_ref, lse_ref = oracle.attend_fwd(x["Q"], x["K"], x["V"], res["ids"], p0, sink=s * C,
                                       per_q_head=per_head)
    st = check_close(f"{where} O", res["O"], O_ref)
    check_close(f"{where} lse", res["lse"], lse_ref, atol=1e-3, rtol=0, rel_l2=None)
    if "dQ" in res:
        grads = oracle.attend_bwd(x["Q"], x["K"], x["V"], x["dO"], res["ids"], p0, sink=s * C,
                                  per_q_head=per_head)
        for name, ref in zip(("dQ", "dK", "dV"), grads):
            check_close(f"{where} {name}", res[name], ref)
    log(f"{where}: near ties {ties}; O {st}")


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("fused", [False, True])
def test_per_head_forward(G, fused):
    T, n_q, k, s = 1024, 256, 5, G % 3
    x = inputs.small_random(700 + G, 2 * G, 2, 128, T, n_q, bf16=True)
    res = run(x, T - n_q, k, s, fused=fused)
    check(x, T - n_q, k, s, res, f"per head G={G} fused={fused}")
    if G > 1:   # the heads of a kv head do route differently
        ids = res["ids"].reshape(2, G, *res["ids"].shape[1:])
        assert any(not np.array_equal(ids[0, 0], ids[0, j]) for j in range(1, G))


def test_per_head_fused_equals_separate():
    T, n_q, k = 2048, 512, 7
    x = inputs.small_random(710, 8, 2, 128, T, n_q, bf16=True)
    a = run(x, T - n_q, k, 1)
    b = run(x, T - n_q, k, 1, fused=True)
    for name in ("ids", "scores", "O", "lse"):
        np.testing.assert_array_equal(a[name], b[name], err_msg=name)


def test_per_head_with_one_head_per_kv_head_is_kv_head_routing():
    T, n_q, k = 1024, 256, 4
    x = inputs.small_random(711, 2, 2, 128, T, n_q, bf16=True, with_dO=True)
    a = run(x, T - n_q, k, bwd=True)
    b = run(x, T - n_q, k, per_head=False, bwd=True)
    for name in ("ids", "scores", "O", "lse", "dQ", "dK", "dV"):
        np.testing.assert_array_equal(a[name], b[name], err_msg=name)


@pytest.mark.parametrize("G,p0", [(4, 768), (8, 768), (4, 0), (2, 512)])
def test_per_head_backward(G, p0):
    T, k = 1024, 4
    n_q = T - p0
    x = inputs.small_random(720 + G + p0, 2 * G, 2, 128, T, n_q, bf16=True, with_dO=True)
    res = run(x, p0, k, 1, bwd=True)
    check(x, p0, k, 1, res, f"per head bwd G={G} p0={p0}")


def test_per_head_backward_beyond_the_sorted_queue():
    """More (unit, chunk) pairs than the dK/dV kernel sorts by size (1024):
    8 query-head units x 136 active blocks = 1088, so the items run in chunk
    order."""
    p0, n_q, k = 1024, 64 * 136, 3
    x = inputs.small_random(740, 8, 1, 128, p0 + n_q, n_q, bf16=True, with_dO=True)
    res = run(x, p0, k, bwd=True)
    check(x, p0, k, 0, res, "per head bwd, 1088 pairs")


def test_per_head_more_than_2048_candidates():
    T, n_q, k = 64 * 2100, 128, 9
    x = inputs.small_random(730, 4, 1, 128, T, n_q, bf16=True)
    res = run(x, T - n_q, k)
    check(x, T - n_q, k, 0, res, "per head 2098 candidates")


def test_per_head_layer16k():
    w = inputs.LAYER16K
    x = inputs.generate(w)
    res = run(x, w.p0, w.k, fused=True)
    check(x, w.p0, w.k, 0, res, "layer16k per head")


@pytest.mark.parametrize("per_head,s", [(False, 0), (True, 0), (False, 2), (True, 1)])
def test_causal_route(per_head, s):
    T, n_q, k = 1024, 256, 5
    x = inputs.small_random(740 + s + 10 * per_head, 8, 2, 128, T, n_q + C, bf16=True)
    Q_prev = x["Q"][:, :C].copy()
    x["Q"] = np.ascontiguousarray(x["Q"][:, C:])
    res = run(x, T - n_q, k, s, per_head=per_head, causal=True, Q_prev=Q_prev)
    check(x, T - n_q, k, s, res, f"causal per_head={per_head} s={s}", per_head=per_head,
          causal=True, Q_prev=Q_prev)


def test_causal_route_from_the_sequence_start():
    T, n_q, k = 512, 512, 3
    x = inputs.small_random(750, 4, 1, 128, T, n_q, bf16=True)
    res = run(x, 0, k, per_head=False, causal=True, Q_prev=None)
    check(x, 0, k, 0, res, "causal p0=0", per_head=False, causal=True)
    assert np.all(res["ids"][:, 0] == -1)


def test_causal_route_ignores_the_block_itself():
    # perturbing block 3's queries changes no ids of blocks 0..3
    T, n_q, k = 1024, 512, 4
    x = inputs.small_random(751, 4, 1, 128, T, n_q + C, bf16=True)
    Q_prev = x["Q"][:, :C].copy()
    x["Q"] = np.ascontiguousarray(x["Q"][:, C:])
    a = run(x, T - n_q, k, per_head=False, causal=True, Q_prev=Q_prev)
    y = dict(x)
    y["Q"] = x["Q"].copy()
    y["Q"][:, 3 * C:] = inputs.round_bf16(-4.0 * y["Q"][:, 3 * C:])
    b = run(y, T - n_q, k, per_head=False, causal=True, Q_prev=Q_prev)
    np.testing.assert_array_equal(a["ids"][:, :4], b["ids"][:, :4])
    assert not np.array_equal(a["ids"][:, 4:], b["ids"][:, 4:])


def test_causal_layer16k():
    w = inputs.LAYER16K
    x = inputs.generate(w)
    rng = np.random.default_rng(752)
    Q_prev = inputs.round_bf16(rng.standard_normal((w.Hq, C, w.D), dtype=np.float32))
    res = run(x, w.p0, w.k, per_head=False, causal=True, Q_prev=Q_prev)
    check(x, w.p0, w.k, 0, res, "layer16k causal", per_head=False, causal=True, Q_prev=Q_prev)
