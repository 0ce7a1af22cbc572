"""The Python binding refuses tensors whose shapes disagree with the config
and the call (the C ABI sees bare pointers and could not tell). CPU only:
shapes are checked before the device, so correctly shaped host tensors reach
the "must live on the GPU" refusal and a wrongly shaped one is named."""
import pytest
import torch

from sparse_long_context_summarize_amd import hga

Hq, Hkv, D, k, n_q, T = 8, 2, 128, 4, 128, 1024
nb = n_q // 64


def bf(*s):
    return torch.zeros(s, dtype=torch.bfloat16)


def f32(*s):
    return torch.zeros(s, dtype=torch.float32)


def i32(*s):
    return torch.zeros(s, dtype=torch.int32)


def _calls(cfg, per_q_head=False):
    U = Hq if per_q_head else Hkv
    Q, K, V = bf(Hq, n_q, D), bf(Hkv, T, D), bf(Hkv, T, D)
    S, SG = f32(Hkv, T // 64, D), f32(Hkv, T // 8, D)
    ids, sc = i32(U, nb, k), f32(U, nb, k)
    O, lse = bf(Hq, n_q, D), f32(Hq, n_q)
    dO, dQ, dK, dV = bf(Hq, n_q, D), f32(Hq, n_q, D), f32(Hkv, n_q, D), f32(Hkv, n_q, D)
    gids, ws = i32(Hkv, nb, 16), torch.zeros(16, dtype=torch.uint8)
    p0 = T - n_q
    yield "hga_summarize", (cfg, K, 0, 64, S), {"K": 1, "summaries": 4}
    yield "hga_route", (cfg, Q, p0, S, T // 64, ids, sc), {"Q": 1, "summaries": 3, "ids": 5,
                                                             "scores": 6}
    yield "hga_route_causal", (cfg, Q, bf(Hq, 64, D), p0, S, T // 64, ids, sc), \
        {"Q": 1, "Q_prev": 2, "ids": 6}
    yield "hga_attend_fwd", (cfg, Q, K, V, p0, ids, O, lse), {"Q": 1, "K": 2, "V": 3, "ids": 5,
                                                               "O": 6, "lse": 7}
    yield "hga_route_attend_fwd", (cfg, Q, K, V, p0, S, T // 64, ids, O, lse, sc), \
        {"ids": 7, "O": 8, "lse": 9, "scores": 10}
    yield "hga_attend_bwd", (cfg, Q, K, V, p0, ids, O, lse, dO, dQ, dK, dV, ws), \
        {"ids": 5, "O": 6, "lse": 7, "dO": 8, "dQ": 9, "dK": 10, "dV": 11}
    if per_q_head:
        return
    yield "hga_summarize_groups", (cfg, K, 0, 64, SG), {"group_summaries": 4}
    yield "hga_route_groups", (cfg, Q, p0, SG, ids, gids), {"chunk_ids": 4, "group_ids": 5}
    yield "hga_attend_fwd_groups", (cfg, Q, K, V, p0, gids, O, lse), {"group_ids": 5, "O": 6}
    yield "hga_route_attend_fwd_groups", (cfg, Q, K, V, p0, S, T // 64, SG, ids, gids, O, lse), \
        {"chunk_ids": 8, "group_ids": 9, "lse": 11}
    yield "hga_attend_bwd_groups", (cfg, Q, K, V, p0, gids, O, lse, dO, dQ, dK, dV, ws), \
        {"group_ids": 5, "dQ": 9, "dK": 10}
    dq = bf(Hq, 3, D)
    yield "hga_route_decode", (cfg, dq, 700, S, 10, i32(Hkv, 3, k), ws), {"ids": 5}
    yield "hga_attend_decode", (cfg, dq, K, V, 700, i32(Hkv, 3, k), bf(Hq, 3, D), f32(Hq, 3), ws), \
        {"ids": 5, "O": 6, "lse": 7}


def _bad(t):
    """The same tensor with its first dimension one larger."""
    s = list(t.shape)
    s[0] += 1
    return torch.zeros(s, dtype=t.dtype)


@pytest.mark.parametrize("per_q_head", [False, True])
def test_shapes_checked_before_launch(per_q_head):
    cfg = hga.make_config(Hq, Hkv, k, route_heads=hga.HGA_ROUTE_PER_Q_HEAD if per_q_head
                          else hga.HGA_ROUTE_PER_KV_HEAD)
    seen = 0
    for name, args, bad in _calls(cfg, per_q_head):
        fn = getattr(hga, name)
        with pytest.raises(ValueError, match="GPU"):
            fn(*args)                                  # right shapes: device refusal next
        for tname, pos in bad.items():
            a = list(args)
            a[pos] = _bad(a[pos])
            with pytest.raises(ValueError, match=f"{tname}|K and V"):
                fn(*a)
            seen += 1
    assert seen >= 20


def test_id_rows_follow_the_routing_granularity():
    cfg = hga.make_config(Hq, Hkv, k, route_heads=hga.HGA_ROUTE_PER_Q_HEAD)
    Q, S = bf(Hq, n_q, D), f32(Hkv, T // 64, D)
    with pytest.raises(ValueError, match="ids has shape"):       # per kv head rows
        hga.hga_route(cfg, Q, T - n_q, S, T // 64, i32(Hkv, nb, k))
    cfg = hga.make_config(Hq, Hkv, k)
    with pytest.raises(ValueError, match="ids has shape"):       # per query head rows
        hga.hga_route(cfg, Q, T - n_q, S, T // 64, i32(Hq, nb, k))
    with pytest.raises(ValueError, match="Q has shape"):         # head count
        hga.hga_route(cfg, bf(Hq + 1, n_q, D), T - n_q, S, T // 64, i32(Hkv, nb, k))
