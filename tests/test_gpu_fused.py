"""hga_route_attend_fwd (routing and attention in one launch) against the two
separate calls, hga_route then hga_attend_fwd, on the same inputs: ids,
scores, O and lse must be bit-identical (the fused kernel runs the router's
own device code). The separate calls are checked against the oracle in
test_gpu_fwd.py; the tiny workload is also checked against the oracle here."""
import os

import numpy as np
import pytest
import torch

import oracle
from parity import check_close, check_ids, to_dev_bf16, from_dev
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


def _draw(seed, Hq, Hkv, T, n_q):
    """bf16 inputs drawn on the GPU (seeded), keys with per-chunk offsets."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    Q = torch.randn((Hq, n_q, 128), generator=g, device="cuda").to(torch.bfloat16)
    K = torch.randn((Hkv, T, 128), generator=g, device="cuda")
    K += 0.5 * torch.randn((Hkv, T // C, 1, 1), generator=g, device="cuda").repeat_interleave(
        C, dim=1).view(Hkv, T, 1)
    V = torch.randn((Hkv, T, 128), generator=g, device="cuda").to(torch.bfloat16)
    return Q, K.to(torch.bfloat16), V


def _both(Q, K, V, p0, k):
    Hq, n_q, _ = Q.shape
    Hkv, T, _ = K.shape
    cfg = hga.make_config(Hq, Hkv, k)
    n_valid = (p0 + n_q) // C
    S = torch.empty((Hkv, n_valid, 128), device="cuda")
    hga.hga_summarize(cfg, K, 0, p0 + n_q, S)
    nb = n_q // C
    out = []
    for fused in (False, True):
        ids = torch.full((Hkv, nb, max(k, 1)), -7, dtype=torch.int32, device="cuda")[..., :k]
        ids = ids.contiguous()
        sc = torch.full((Hkv, nb, k), float("nan"), device="cuda")
        O = torch.full((Hq, n_q, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((Hq, n_q), float("nan"), device="cuda")
        if fused:
            hga.hga_route_attend_fwd(cfg, Q, K, V, p0, S, n_valid, ids, O, lse, sc)
        else:
            hga.hga_route(cfg, Q, p0, S, n_valid, ids, sc)
            hga.hga_attend_fwd(cfg, Q, K, V, p0, ids, O, lse)
        torch.cuda.synchronize()
        out.append(dict(ids=ids, scores=sc, O=O, lse=lse))
    return out


def _identical(a, b, where):
    for name in ("ids", "scores", "O", "lse"):
        x, y = a[name], b[name]
        assert x.shape == y.shape, (where, name)
        same = torch.equal(x, y) if name in ("ids",) else torch.equal(
            x.view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32),
            y.view(torch.int16 if y.dtype == torch.bfloat16 else torch.int32))
        assert same, f"{where}: {name} differs between the fused and the separate calls"


@pytest.mark.parametrize("Hq,Hkv,k,T,n_q", [
    (32, 8, 16, 16384, 2048),       # the 16K layer shape
    (8, 2, 7, 1024, 256),
    (1, 1, 1, 1024, 256),
    (2, 1, 5, 2048, 512),
    (16, 8, 3, 1024, 256),          # G = 2
    (8, 1, 9, 2048, 256),           # G = 8: two workgroups per unit
    (4, 1, 256, 64 * 300, 128),     # k = 256, register selection over 298-299 candidates
    (4, 2, 32, 64 * 1100, 128),     # 16 keys per lane
    (4, 1, 40, 64 * 2200, 128),     # over 2048 candidates: the selection in LDS
    (4, 1, 0, 1024, 256),           # k = 0: the local block only
])
def test_matches_separate_calls(Hq, Hkv, k, T, n_q):
    Q, K, V = _draw(Hq * 1000 + k, Hq, Hkv, T, n_q)
    log(f"fused Hq={Hq} Hkv={Hkv} k={k} T={T} n_q={n_q}")
    a, b = _both(Q, K, V, T - n_q, k)
    _identical(a, b, f"Hq={Hq} Hkv={Hkv} k={k} T={T}")


def test_first_segment():
    Q, K, V = _draw(5, 4, 2, 512, 512)
    a, b = _both(Q, K, V, 0, 6)
    _identical(a, b, "p0 = 0")
    assert torch.all(a["ids"][:, 0] == -1)


def test_more_candidates_than_the_fused_kernel_holds():
    # 17600 candidate chunks: the entry point runs the two kernels in turn
    T, n_q = 64 * 17602, 128
    Q, K, V = _draw(6, 4, 1, T, n_q)
    a, b = _both(Q, K, V, T - n_q, 8)
    _identical(a, b, "17600 candidates")


def test_tiny_against_the_oracle():
    w = inputs.TINY
    x = inputs.generate(w, bf16=True)
    Q, K, V = to_dev_bf16(x["Q"]), to_dev_bf16(x["K"]), to_dev_bf16(x["V"])
    _, b = _both(Q, K, V, w.p0, w.k)
    S_ref = oracle.summarize(x["K"], C, 0, w.T // C)
    ids_ref, sigma = oracle.route(x["Q"], S_ref, w.p0, w.k, w.Hkv, want_scores=True)
    ids = b["ids"].cpu().numpy()
    check_ids(ids, ids_ref, sigma, w.p0, where="fused tiny")
    O_ref, lse_ref = oracle.attend_fwd(x["Q"], x["K"], x["V"], ids, w.p0)
    check_close("fused tiny O", from_dev(b["O"]), O_ref)
    check_close("fused tiny lse", from_dev(b["lse"]), lse_ref, atol=1e-3, rtol=0, rel_l2=None)


def test_gather_diagnostic_reads_the_attended_rows():
    """hga_diag_gather folds exactly the rows the attention gathers: each
    thread's word is the XOR of its slices of the block's distinct valid
    routed chunks and local block (recomputed here from the bf16 bits)."""
    Hq, Hkv, T, n_q, k = 4, 2, 1024, 256, 5
    x = inputs.small_random(51, Hq, Hkv, 128, T, n_q, bf16=True)
    p0 = T - n_q
    ids = np.array([[[3, 1, 3, -1, 40], [0, 12, 13, 2, 2], [-1] * 5, [14, 15, 1, 0, 9]],
                    [[11, 10, 9, 8, 7], [1, 1, 1, 1, 1], [5, 6, 7, 8, 9], [2, 3, 4, 5, 6]]],
                   np.int32)
    cfg = hga.make_config(Hq, Hkv, k)
    K, V = to_dev_bf16(x["K"]), to_dev_bf16(x["V"])
    idd = torch.from_numpy(ids).cuda()
    sink = torch.empty(hga.hga_diag_gather_sink_words(cfg, n_q), dtype=torch.int32, device="cuda")
    hga.hga_diag_gather(cfg, K, V, p0, n_q, idd, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    kb = inputs.bf16_bits(x["K"]).view(np.uint16).astype(np.uint32)
    vb = inputs.bf16_bits(x["V"]).view(np.uint16).astype(np.uint32)
    # 32-bit words as the kernel reads them: pairs of bf16 (low half first)
    kw = kb[..., 0::2] | (kb[..., 1::2] << 16)           # [Hkv][T][64]
    vw = vb[..., 0::2] | (vb[..., 1::2] << 16)
    nb = n_q // C
    for g in range(Hkv):
        for b in range(nb):
            P = p0 + b * C
            tiles = sorted({int(c) for c in ids[g, b] if 0 <= c < P // C}) + [P // C]
            for tid in range(256):
                acc = 0
                for c in tiles:
                    for j in range(4):
                        r = c * C + (tid >> 4) + 16 * j
                        sl = slice(4 * (tid & 15), 4 * (tid & 15) + 4)
                        for wds in (kw[g, r, sl], vw[g, r, sl]):
                            for wd in wds:
                                acc ^= int(wd)
                assert got[(b * Hkv + g) * 256 + tid] == acc, (g, b, tid)
