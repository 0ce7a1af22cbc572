"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and each argument check returns its status code before any
HIP call (the pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

from sparse_long_context_summarize_amd import hga

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "hga.h")
FAKE = ctypes.c_void_p(0x1000)    # a non-NULL pointer; argument checks fail first


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hga_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function():
    L = hga.lib()
    declared = _declared_functions()
    assert set(declared) == set(hga.EXPORTED), declared
    for name in declared:
        assert hasattr(L, name), name


def test_version_and_status_strings():
    assert hga.hga_version() == 10000
    assert hga.hga_status_string(hga.HGA_OK) == "HGA_OK"
    assert hga.hga_status_string(hga.HGA_ERR_CAPACITY) == "HGA_ERR_CAPACITY"
    assert hga.hga_status_string(99) == "HGA_ERR_UNKNOWN"


def _cfg(**kw):
    base = dict(n_q_heads=32, n_kv_heads=8, top_k=16)
    base.update(kw)
    return hga.make_config(base.pop("n_q_heads"), base.pop("n_kv_heads"), base.pop("top_k"),
                           **base)


def _fwd(cfg, p0=14336, n_q=2048, T=16384, ids=FAKE, O=FAKE):
    return hga.lib().hga_attend_fwd(ctypes.byref(cfg), FAKE, FAKE, FAKE, T, p0, n_q, ids, O,
                                    FAKE, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(n_q_heads=30, n_kv_heads=8), hga.HGA_ERR_INVALID_ARG, "multiple"),
    (dict(n_q_heads=48, n_kv_heads=8), hga.HGA_ERR_UNSUPPORTED, "1, 2, 4 or 8"),
    (dict(n_kv_heads=0), hga.HGA_ERR_INVALID_ARG, "positive"),
    (dict(head_dim=64), hga.HGA_ERR_UNSUPPORTED, "head_dim"),
    (dict(chunk=32, q_block=32), hga.HGA_ERR_UNSUPPORTED, "chunk"),
    (dict(q_block=128), hga.HGA_ERR_UNSUPPORTED, "q_block"),
    (dict(top_k=257), hga.HGA_ERR_INVALID_ARG, "top_k"),
    (dict(top_k=-1), hga.HGA_ERR_INVALID_ARG, "top_k"),
    (dict(dtype=1), hga.HGA_ERR_UNSUPPORTED, "dtype"),
    (dict(softmax_scale=float("nan")), hga.HGA_ERR_INVALID_ARG, "finite"),
    (dict(sink_chunks=-1), hga.HGA_ERR_INVALID_ARG, "sink_chunks"),
    (dict(sink_chunks=65), hga.HGA_ERR_UNSUPPORTED, "sink_chunks"),
])
def test_config_checks(kw, status, needle):
    cfg = _cfg(**kw)
    assert _fwd(cfg) == status
    assert needle in hga.hga_last_error()


def test_null_config():
    assert hga.lib().hga_attend_fwd(None, FAKE, FAKE, FAKE, 16384, 0, 64, FAKE, FAKE, FAKE,
                                    None) == hga.HGA_ERR_INVALID_ARG


@pytest.mark.parametrize("p0,n_q,T,needle", [
    (14335, 2048, 16384, "p0"),
    (14336, 2047, 16384, "n_q"),
    (14336, 2048, 16383, "T_cap"),
    (-64, 64, 16384, ">= 0"),
])
def test_segment_checks(p0, n_q, T, needle):
    assert _fwd(_cfg(), p0=p0, n_q=n_q, T=T) == hga.HGA_ERR_INVALID_ARG
    assert needle in hga.hga_last_error()


def test_null_pointers():
    assert _fwd(_cfg(), O=None) == hga.HGA_ERR_INVALID_ARG
    assert _fwd(_cfg(), ids=None) == hga.HGA_ERR_INVALID_ARG
    # k = 0 needs no ids; n_q = 0 is a no-op that launches nothing
    assert _fwd(_cfg(top_k=0), n_q=0, ids=None) == hga.HGA_OK


def test_summarize_checks():
    L = hga.lib()
    cfg = _cfg()
    s = L.hga_summarize
    assert s(ctypes.byref(cfg), FAKE, 16384, 32, 64, FAKE, 256, None) == hga.HGA_ERR_INVALID_ARG
    assert s(ctypes.byref(cfg), FAKE, 16384, 0, 100, FAKE, 256, None) == hga.HGA_ERR_INVALID_ARG
    assert s(ctypes.byref(cfg), FAKE, 16384, 16320, 128, FAKE, 512, None) == hga.HGA_ERR_INVALID_ARG
    assert s(ctypes.byref(cfg), FAKE, 16384, 0, 16384, FAKE, 255, None) == hga.HGA_ERR_CAPACITY
    assert "255" in hga.hga_last_error()
    assert s(ctypes.byref(cfg), None, 16384, 0, 64, FAKE, 256, None) == hga.HGA_ERR_INVALID_ARG
    assert s(ctypes.byref(cfg), FAKE, 16384, 64, 0, FAKE, 256, None) == hga.HGA_OK


def test_route_checks():
    L = hga.lib()
    cfg = _cfg()
    r = L.hga_route
    # the last block of 14336 + 2048 needs 255 summaries
    assert r(ctypes.byref(cfg), FAKE, 14336, 2048, FAKE, 256, 254, FAKE, None,
             None) == hga.HGA_ERR_CAPACITY
    assert r(ctypes.byref(cfg), FAKE, 14336, 2048, FAKE, 256, 257, FAKE, None,
             None) == hga.HGA_ERR_CAPACITY
    assert r(ctypes.byref(cfg), FAKE, 14300, 2048, FAKE, 256, 255, FAKE, None,
             None) == hga.HGA_ERR_INVALID_ARG
    assert r(ctypes.byref(cfg), FAKE, 14336, 2048, FAKE, 256, 255, None, None,
             None) == hga.HGA_ERR_INVALID_ARG
    big = 64 * 30000
    assert r(ctypes.byref(cfg), FAKE, big, 64, FAKE, 30000, 30000, FAKE, None,
             None) == hga.HGA_ERR_UNSUPPORTED
    assert r(ctypes.byref(_cfg(top_k=0)), FAKE, 14336, 2048, FAKE, 256, 255, None, None,
             None) == hga.HGA_OK


def test_bwd_second_pass_diag_checks():
    L = hga.lib()
    cfg = _cfg()
    need = hga.hga_attend_bwd_workspace_bytes(cfg, 2048)
    n2, nw = ctypes.c_int64(-1), ctypes.c_int64(-1)
    d = L.hga_diag_bwd_second_pass
    assert d(ctypes.byref(cfg), 2047, FAKE, need, ctypes.byref(n2), ctypes.byref(nw),
             None) == hga.HGA_ERR_INVALID_ARG
    assert d(ctypes.byref(cfg), 2048, FAKE, need - 1, ctypes.byref(n2), ctypes.byref(nw),
             None) == hga.HGA_ERR_CAPACITY
    assert d(ctypes.byref(cfg), 2048, None, need, ctypes.byref(n2), ctypes.byref(nw),
             None) == hga.HGA_ERR_INVALID_ARG
    assert d(ctypes.byref(cfg), 2048, FAKE, need, None, ctypes.byref(nw),
             None) == hga.HGA_ERR_INVALID_ARG
    assert d(ctypes.byref(cfg), 0, None, 0, ctypes.byref(n2), ctypes.byref(nw), None) == hga.HGA_OK
    assert (n2.value, nw.value) == (0, 0)


def test_bwd_checks():
    L = hga.lib()
    cfg = _cfg()
    need = hga.hga_attend_bwd_workspace_bytes(cfg, 2048)
    assert need > 0
    assert hga.hga_attend_bwd_workspace_bytes(cfg, 2047) == 0
    assert hga.hga_attend_bwd_workspace_bytes(_cfg(head_dim=64), 2048) == 0
    b = L.hga_attend_bwd
    args = [ctypes.byref(cfg), FAKE, FAKE, FAKE, 16384, 14336, 2048, FAKE, FAKE, FAKE, FAKE,
            FAKE, FAKE, FAKE]
    assert b(*args, FAKE, need - 1, None) == hga.HGA_ERR_CAPACITY
    assert b(*args, None, need, None) == hga.HGA_ERR_INVALID_ARG
    bad = list(args)
    bad[13] = None                      # dV
    assert b(*bad, FAKE, need, None) == hga.HGA_ERR_INVALID_ARG


def test_binding_rejects_host_tensors():
    import torch
    cfg = _cfg()
    K = torch.zeros(8, 64, 128, dtype=torch.bfloat16)
    S = torch.zeros(8, 1, 128)
    with pytest.raises(ValueError, match="GPU"):
        hga.hga_summarize(cfg, K, 0, 64, S)


def test_group_entry_point_checks():
    L = hga.lib()
    cfg = _cfg()
    c = ctypes.byref(cfg)
    s = L.hga_summarize_groups
    assert s(c, FAKE, 16384, 32, 64, FAKE, 2048, None) == hga.HGA_ERR_INVALID_ARG
    assert s(c, FAKE, 16384, 0, 16384, FAKE, 2047, None) == hga.HGA_ERR_CAPACITY
    assert "2048" in hga.hga_last_error()
    assert s(c, None, 16384, 0, 64, FAKE, 2048, None) == hga.HGA_ERR_INVALID_ARG
    assert s(c, FAKE, 16384, 64, 0, FAKE, 2048, None) == hga.HGA_OK
    r = L.hga_route_groups
    assert r(c, FAKE, 14336, 2048, FAKE, 2040, FAKE, 2049, FAKE, None,
             None) == hga.HGA_ERR_INVALID_ARG
    assert r(c, FAKE, 14336, 2048, FAKE, 2040, FAKE, -1, FAKE, None,
             None) == hga.HGA_ERR_INVALID_ARG
    # the last block may route to chunk 254, i.e. groups up to 2039
    assert r(c, FAKE, 14336, 2048, FAKE, 2039, FAKE, 64, FAKE, None,
             None) == hga.HGA_ERR_CAPACITY
    assert r(c, FAKE, 14336, 2048, FAKE, 2040, None, 64, FAKE, None,
             None) == hga.HGA_ERR_INVALID_ARG
    assert r(c, FAKE, 14336, 2047, FAKE, 2040, FAKE, 64, FAKE, None,
             None) == hga.HGA_ERR_INVALID_ARG
    assert r(c, FAKE, 14336, 2048, FAKE, 2040, FAKE, 0, None, None, None) == hga.HGA_OK
    a = L.hga_attend_fwd_groups
    assert a(c, FAKE, FAKE, FAKE, 16384, 14336, 2048, FAKE, 2049, FAKE, FAKE,
             None) == hga.HGA_ERR_INVALID_ARG
    assert a(c, FAKE, FAKE, FAKE, 16384, 14336, 2048, None, 64, FAKE, FAKE,
             None) == hga.HGA_ERR_INVALID_ARG
    assert a(c, FAKE, FAKE, FAKE, 16383, 14336, 2048, FAKE, 64, FAKE, FAKE,
             None) == hga.HGA_ERR_INVALID_ARG
    assert a(c, FAKE, FAKE, FAKE, 16384, 14336, 0, None, 64, FAKE, FAKE, None) == hga.HGA_OK


def test_route_attend_checks():
    L = hga.lib()
    cfg = _cfg()
    c = ctypes.byref(cfg)
    f = L.hga_route_attend_fwd
    args = dict(T=16384, p0=14336, n_q=2048, cap=256, valid=256, ids=FAKE)

    def call(**kw):
        a = dict(args, **kw)
        return f(c, FAKE, FAKE, FAKE, a["T"], a["p0"], a["n_q"], FAKE, a["cap"], a["valid"],
                 a["ids"], None, FAKE, FAKE, None)

    # the last block needs 255 valid summaries
    assert call(valid=254) == hga.HGA_ERR_CAPACITY
    assert call(valid=257) == hga.HGA_ERR_CAPACITY          # valid > capacity
    assert call(T=16383) == hga.HGA_ERR_INVALID_ARG
    assert call(ids=None) == hga.HGA_ERR_INVALID_ARG
    assert call(n_q=0) == hga.HGA_OK
    cfg0 = _cfg(top_k=0)
    assert f(ctypes.byref(cfg0), FAKE, FAKE, FAKE, 16384, 14336, 0, None, 0, 0, None, None,
             FAKE, FAKE, None) == hga.HGA_OK


def test_decode_checks():
    L = hga.lib()
    cfg = _cfg(top_k=32)
    # router keys: one per candidate (chunks before the last token's open
    # chunk) per token and kv head; attention partials: 130 floats per split
    # (one tile of the token's list a split) per token and query head; one
    # size serves both
    p0, n_q = 131071, 1
    keys = n_q * 8 * (p0 // 64) * 4
    parts = n_q * 32 * (32 + 1) * 130 * 4
    assert hga.hga_decode_workspace_bytes(cfg, p0, n_q) == max(keys, parts)
    assert hga.hga_decode_workspace_bytes(cfg, 100, 1) == parts
    assert hga.hga_decode_workspace_bytes(_cfg(top_k=32, sink_chunks=4), 64 * 10, 1) == \
        1 * 32 * (4 + 32 + 1) * 130 * 4
    assert hga.hga_decode_workspace_bytes(cfg, -1, 1) == 0
    assert hga.hga_decode_workspace_bytes(_cfg(head_dim=64), p0, 1) == 0
    need = hga.hga_decode_workspace_bytes(cfg, p0, n_q)
    n_closed = p0 // 64

    def route(ws, ws_bytes, n_valid=n_closed, n_cap=n_closed):
        return L.hga_route_decode(ctypes.byref(cfg), FAKE, p0, n_q, FAKE, n_cap, n_valid,
                                  FAKE, None, ws, ws_bytes, None)

    assert route(FAKE, need - 1) == hga.HGA_ERR_CAPACITY
    assert "workspace" in hga.hga_last_error()
    assert route(None, need) == hga.HGA_ERR_INVALID_ARG
    assert route(FAKE, need, n_valid=n_closed - 1) == hga.HGA_ERR_CAPACITY
    assert route(FAKE, need, n_valid=n_closed + 1) == hga.HGA_ERR_CAPACITY   # above the cap

    def attend(ws_bytes, T=p0 + n_q):
        return L.hga_attend_decode(ctypes.byref(cfg), FAKE, FAKE, FAKE, T, p0, n_q, FAKE,
                                   FAKE, FAKE, FAKE, ws_bytes, None)

    assert attend(need - 1) == hga.HGA_ERR_CAPACITY
    assert attend(need, T=p0) == hga.HGA_ERR_INVALID_ARG


def test_route_attend_decode_checks():
    """hga_route_attend_decode: its workspace (the scoring blocks' survivor
    keys and ids, the split partials, each 256-B aligned) and its refusals,
    all before any launch."""
    L = hga.lib()
    cfg = _cfg(top_k=32)
    p0, n_q = 131071, 1
    n_blk = -(-(p0 // 64) // 256)                 # 2047 candidates in blocks of 256
    surv = n_q * 8 * n_blk * 32 * 4
    parts = n_q * 32 * (32 + 1) * 130 * 4
    need = surv + surv + parts
    assert hga.hga_route_attend_decode_workspace_bytes(cfg, p0, n_q) == need
    assert hga.hga_route_attend_decode_workspace_bytes(cfg, -1, 1) == 0
    n_closed = p0 // 64

    def call(cfg=cfg, p0=p0, n_q=n_q, T=p0 + n_q, n_valid=n_closed, ids=FAKE, ws=FAKE,
             ws_bytes=need):
        return L.hga_route_attend_decode(ctypes.byref(cfg), FAKE, FAKE, FAKE, T, p0, n_q,
                                         FAKE, n_closed + 8, n_valid, ids, None, FAKE, FAKE,
                                         ws, ws_bytes, None)

    assert call(ws_bytes=need - 1) == hga.HGA_ERR_CAPACITY
    assert "workspace" in hga.hga_last_error()
    assert call(ws=None) == hga.HGA_ERR_INVALID_ARG
    assert call(T=p0) == hga.HGA_ERR_INVALID_ARG
    assert call(n_valid=n_closed - 1) == hga.HGA_ERR_CAPACITY
    assert call(n_valid=n_closed + 9) == hga.HGA_ERR_CAPACITY            # above the cap
    assert call(ids=None) == hga.HGA_ERR_INVALID_ARG
    assert call(n_q=65536, T=p0 + 65536) == hga.HGA_ERR_UNSUPPORTED
    assert call(n_q=0) == hga.HGA_OK
    # top_k 256 over 13000 candidates: 51 blocks x 256 survivors > 12288
    big = _cfg(top_k=256)
    p_big = 64 * 13000 + 3
    n_big = hga.hga_route_attend_decode_workspace_bytes(big, p_big, 1)
    assert L.hga_route_attend_decode(ctypes.byref(big), FAKE, FAKE, FAKE, p_big + 1, p_big, 1,
                                     FAKE, 13000, 13000, FAKE, None, FAKE, FAKE, FAKE, n_big,
                                     None) == hga.HGA_ERR_UNSUPPORTED
    assert "hga_route_decode" in hga.hga_last_error()
    # no routing: ids and summaries may be NULL
    k0 = _cfg(top_k=0)
    n0 = hga.hga_route_attend_decode_workspace_bytes(k0, p0, 1)
    assert L.hga_route_attend_decode(ctypes.byref(k0), FAKE, FAKE, FAKE, p0 + 1, p0, 0, None,
                                     0, 0, None, None, FAKE, FAKE, FAKE, n0,
                                     None) == hga.HGA_OK


def test_grid_limits():
    """Sizes past what one launch's grid holds are refused before any launch:
    more than 65535 query blocks, more than 65535 decode tokens, more than
    65535 kv heads."""
    L = hga.lib()
    cfg = _cfg()
    n_big = 65536 * 64
    assert _fwd(cfg, p0=0, n_q=n_big, T=n_big) == hga.HGA_ERR_UNSUPPORTED
    assert "65535 query blocks" in hga.hga_last_error()
    assert _fwd(_cfg(n_q_heads=65536, n_kv_heads=65536)) == hga.HGA_ERR_UNSUPPORTED
    assert "n_kv_heads" in hga.hga_last_error()
    p0, n_q = 64 * 100, 65536
    assert L.hga_route_decode(ctypes.byref(cfg), FAKE, p0, n_q, FAKE, 4096, 4096, FAKE, None,
                              FAKE, 1 << 40, None) == hga.HGA_ERR_UNSUPPORTED
    assert "tokens per call" in hga.hga_last_error()
    assert L.hga_attend_decode(ctypes.byref(cfg), FAKE, FAKE, FAKE, p0 + n_q, p0, n_q, FAKE,
                               FAKE, FAKE, FAKE, 1 << 40, None) == hga.HGA_ERR_UNSUPPORTED
    assert "tokens per call" in hga.hga_last_error()


def test_route_attend_fwd_groups_checks():
    """hga_route_attend_fwd_groups refuses bad arguments before any launch."""
    L = hga.lib()

    def call(cfg, m=64, n_gcap=16384 // 8, chunk_ids=FAKE, group_ids=FAKE, n_valid=256):
        return L.hga_route_attend_fwd_groups(ctypes.byref(cfg), FAKE, FAKE, FAKE, 16384, 14336,
                                             2048, FAKE, 256, n_valid, FAKE, n_gcap, m,
                                             chunk_ids, group_ids, None, FAKE, FAKE, None)

    cfg = _cfg()
    assert call(_cfg(route_heads=hga.HGA_ROUTE_PER_Q_HEAD)) == hga.HGA_ERR_UNSUPPORTED
    assert call(cfg, m=2049) == hga.HGA_ERR_INVALID_ARG
    assert "group_top_k" in hga.hga_last_error()
    assert call(cfg, n_gcap=100) == hga.HGA_ERR_CAPACITY          # groups of 255 chunks needed
    assert call(cfg, n_valid=200) == hga.HGA_ERR_CAPACITY         # summaries of 255 chunks needed
    assert call(cfg, chunk_ids=None) == hga.HGA_ERR_INVALID_ARG
    assert call(cfg, group_ids=None) == hga.HGA_ERR_INVALID_ARG


def test_routing_variant_checks():
    L = hga.lib()
    bad = _cfg(route_heads=2)
    assert _fwd(bad) == hga.HGA_ERR_INVALID_ARG
    assert "route_heads" in hga.hga_last_error()
    per_head = _cfg(route_heads=hga.HGA_ROUTE_PER_Q_HEAD)
    # the group level, decode and the diagnostic know one id row per kv head
    assert L.hga_route_groups(ctypes.byref(per_head), FAKE, 14336, 2048, FAKE, 14336 // 8, FAKE,
                              8, FAKE, None, None) == hga.HGA_ERR_UNSUPPORTED
    assert L.hga_attend_fwd_groups(ctypes.byref(per_head), FAKE, FAKE, FAKE, 16384, 14336,
                                   2048, FAKE, 8, FAKE, FAKE, None) == hga.HGA_ERR_UNSUPPORTED
    assert L.hga_route_decode(ctypes.byref(per_head), FAKE, 100, 1, FAKE, 1, 1, FAKE, None,
                              FAKE, 1 << 20, None) == hga.HGA_ERR_UNSUPPORTED
    # the backward workspace grows by the per-head dK and dV and the per-head
    # counters, block lists and partial sums
    n_q = 2048
    a = hga.hga_attend_bwd_workspace_bytes(_cfg(), n_q)
    b = hga.hga_attend_bwd_workspace_bytes(per_head, n_q)
    up = lambda v: (v + 255) // 256 * 256
    delta = up(32 * n_q * 4)
    nb = n_q // 64

    def plan(U):               # per (unit, chunk): list length, block ids, group masks,
        # and the dq workgroups' second-pass flags (two workgroups per unit at G = 8)
        return up(U * nb * 4) + up(U * nb * nb * 2) + up(U * nb * nb) + up(U * 2 * nb)

    slots = 7                  # workgroups past the first that may share one active chunk
    assert a == delta + up((8 * nb + 1) * 4) + plan(8) + slots * 2 * 8 * n_q * 128 * 4
    assert b == delta + up((32 * nb + 1) * 4) + plan(32) + slots * 2 * 32 * n_q * 128 * 4 \
        + 2 * 32 * n_q * 128 * 4
    # strictly causal routing needs the queries before p0 once p0 > 0
    args = lambda p0, qp: (ctypes.byref(_cfg()), FAKE, qp, p0, 2048, FAKE, 256, 256, FAKE,
                           None, None)
    assert L.hga_route_causal(*args(14336, None)) == hga.HGA_ERR_INVALID_ARG
    assert "Q_prev" in hga.hga_last_error()
