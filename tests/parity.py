"""Parity rules shared by the GPU tests.

Chunk ids (the routing decision): the GPU's ids for a (kv head, block) pass if
they equal the oracle's, or if both lists have the same number of valid ids,
the GPU list is ascending with -1 padding, and every chunk in the symmetric
difference scores (oracle, fp64) within 1e-4 * M of the oracle's k-th best
score, M being the largest |score| among the block's candidates. The GPU
decides in fp32, the oracle in fp64; the 1e-4 relative gap is the stated
tolerance for near-ties.

Floating-point outputs: elementwise |x - ref| <= 1e-2 + 2e-2 |ref| (the stated
bf16 bar), plus a tighter relative L2 bound per tensor that catches structural
mistakes the elementwise bar is too loose to see (a dropped term in a
gradient moves it by a few percent of its norm). The L2 bound is 1e-2 = about
5 bf16 unit roundoffs (2^-9): the GPU rounds its operands, the probabilities
and the output to bf16 once each.
"""
from __future__ import annotations

import numpy as np
import torch

ATOL = 1e-2
RTOL = 2e-2
REL_L2 = 1e-2
GAP = 1e-4


def to_dev_bf16(a: np.ndarray) -> torch.Tensor:
    """Upload float32 values that are bf16-representable (exact conversion)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).cuda()


def from_dev(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_ids(gpu_ids: np.ndarray, ref_ids: np.ndarray, sigma: np.ndarray, p0: int,
              C: int = 64, Bq: int = 64, where: str = "", sink_chunks: int = 0) -> int:
    """Returns the number of (head, block) rows whose sets differ within the gap.
    With a sink window the candidates are the chunks sink_chunks <= c < P/C."""
    assert gpu_ids.shape == ref_ids.shape, (gpu_ids.shape, ref_ids.shape)
    Hkv, nb, k = gpu_ids.shape
    near_ties = 0
    lo = sink_chunks
    for g in range(Hkv):
        for b in range(nb):
            a, r = gpu_ids[g, b], ref_ids[g, b]
            nE = (p0 + b * Bq) // C
            na, nr = int((a >= 0).sum()), int((r >= 0).sum())
            ctx = f"{where} head {g} block {b}: gpu {a.tolist()} oracle {r.tolist()}"
            assert na == nr == min(k, max(0, nE - lo)), ctx
            assert np.all(a[na:] == -1), ctx
            assert np.all(np.diff(a[:na]) > 0), ctx
            assert na == 0 or (a[0] >= lo and a[na - 1] < nE), ctx
            if np.array_equal(a, r):
                continue
            # candidate scores; sigma is indexed by absolute chunk id
            cand = sigma[g, b, lo:nE]
            M = np.max(np.abs(cand))
            kth = np.sort(cand)[::-1][nr - 1]
            for c in set(a[:na].tolist()) ^ set(r[:nr].tolist()):
                assert abs(sigma[g, b, c] - kth) <= GAP * M, (ctx, c, sigma[g, b, c], kth, M)
            near_ties += 1
    return near_ties


def check_close(name: str, got: np.ndarray, ref: np.ndarray, *, atol: float = ATOL,
                rtol: float = RTOL, rel_l2: float | None = REL_L2) -> dict:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    sel = ~np.isnan(ref)
    assert sel.any(), name
    g, r = got[sel], ref[sel]
    assert np.all(np.isfinite(g)), f"{name}: non-finite GPU values"
    err = np.abs(g - r)
    lim = atol + rtol * np.abs(r)
    worst = int(np.argmax(err - lim))
    assert np.all(err <= lim), (f"{name}: {int((err > lim).sum())} of {err.size} outside "
                                f"{atol} + {rtol}|ref|; worst got {g[worst]} ref {r[worst]}")
    rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
    if rel_l2 is not None:
        assert rel <= rel_l2, f"{name}: relative L2 error {rel:.3e} > {rel_l2}"
    return {"max_abs": float(err.max()), "rel_l2": rel}


def summary_bound(K: np.ndarray, c_begin: int, c_end: int, C: int = 64) -> np.ndarray:
    """Worst-case error of an fp32 sum of C terms, divided by C:
    (C-1) * 2^-24 * mean_t |K| per (head, chunk, d), plus one rounding of the
    result."""
    out = np.empty((K.shape[0], c_end - c_begin, K.shape[2]))
    for g in range(K.shape[0]):
        a = np.abs(K[g, c_begin * C:c_end * C]).reshape(c_end - c_begin, C, K.shape[2])
        out[g] = a.mean(axis=1, dtype=np.float64)
    return (C - 1) * 2.0 ** -24 * out * 1.0001 + 2.0 ** -24 * out


def group_candidates(chunk_row: np.ndarray, P: int, C: int = 64, U: int = 8,
                     sink_chunks: int = 0) -> np.ndarray:
    """Candidate groups of one block: the U-token groups of the distinct chunk
    ids c of its routed row with sink_chunks <= c < P/C, ascending."""
    ch = sorted({int(c) for c in chunk_row if sink_chunks <= c < P // C})
    return np.array([c * (C // U) + j for c in ch for j in range(C // U)], dtype=np.int64)


def check_group_ids(gpu_gids: np.ndarray, ref_gids: np.ndarray, sigma: np.ndarray,
                    chunk_ids: np.ndarray, p0: int, C: int = 64, Bq: int = 64, U: int = 8,
                    where: str = "", sink_chunks: int = 0) -> int:
    """The id rule of check_ids at the group level: the candidates of a block
    are the groups of its routed chunks (group_candidates), M is the largest
    |score| among them. Returns the number of rows that differ within the gap."""
    assert gpu_gids.shape == ref_gids.shape, (gpu_gids.shape, ref_gids.shape)
    Hkv, nb, m = gpu_gids.shape
    near_ties = 0
    for g in range(Hkv):
        for b in range(nb):
            a, r = gpu_gids[g, b], ref_gids[g, b]
            cand = group_candidates(chunk_ids[g, b], p0 + b * Bq, C, U, sink_chunks)
            na, nr = int((a >= 0).sum()), int((r >= 0).sum())
            ctx = f"{where} head {g} block {b}: gpu {a.tolist()} oracle {r.tolist()}"
            assert na == nr == min(m, cand.size), ctx
            assert np.all(a[na:] == -1), ctx
            assert np.all(np.diff(a[:na]) > 0), ctx
            assert np.all(np.isin(a[:na], cand)), ctx
            if np.array_equal(a, r):
                continue
            sig = sigma[g, b, cand]
            M = np.max(np.abs(sig))
            kth = np.sort(sig)[::-1][nr - 1]
            for u in set(a[:na].tolist()) ^ set(r[:nr].tolist()):
                assert abs(sigma[g, b, u] - kth) <= GAP * M, (ctx, u, sigma[g, b, u], kth, M)
            near_ties += 1
    return near_ties
