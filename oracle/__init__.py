"""CPU oracle for the HGA hot path (ctypes binding of ``hga_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg import this package; the product library never does.

Every function returns float64 numpy arrays. Inputs are float32 arrays laid out
as in the GPU library: Q/dO [Hq][n_q][D], K/V [Hkv][T][D], summaries
[Hkv][n_cap][D], ids [Hkv][n_blocks][k].
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hga_oracle.c")
_LIB = os.path.join(_HERE, "libhga_oracle.so")
_lib = None

_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64


def build() -> str:
    """Compile the oracle with gcc (portable flags: the library may run on
    another host CPU). Always rebuilds."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_get_threads.restype = ctypes.c_int
    lib.oracle_summarize.argtypes = [_f32p, _i64, _i64, _i64, _i64, _i64, _i64, _f64p, _i64]
    lib.oracle_route.argtypes = [_f32p, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                 _f64p, _i64, _i64, _i32p, ctypes.c_void_p, _i64,
                                 _i64, ctypes.c_void_p, _i64]
    lib.oracle_route_groups.argtypes = [_f32p, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                        _i64, _f64p, _i64, _i32p, _i64, _i64, _i32p,
                                        ctypes.c_void_p, _i64]
    lib.oracle_attend_fwd.argtypes = [_f32p, _f32p, _f32p, _i64, _i64, _i64, _i64,
                                      _i64, _i64, _i64, _i64, _i32p, _i64,
                                      ctypes.c_double, ctypes.c_void_p, _f64p, _f64p, _i64,
                                      _i64]
    lib.oracle_attend_bwd.argtypes = [_f32p, _f32p, _f32p, _f32p, _i64, _i64, _i64,
                                      _i64, _i64, _i64, _i64, _i64, _i32p, _i64,
                                      ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p,
                                      _f64p, _f64p, _f64p, _i64, _i64]
    lib.oracle_attend_decode.argtypes = [_f32p, _f32p, _f32p, _i64, _i64, _i64, _i64,
                                         _i64, _i64, _i64, _i32p, _i64, ctypes.c_double,
                                         _i64, _f64p, _f64p]
    _lib = lib
    return lib


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _mask_ptr(mask):
    if mask is None:
        return None, None
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    return m, m.ctypes.data_as(ctypes.c_void_p)


def summarize(K, C: int, c_begin: int, c_end: int, out=None, n_cap: int | None = None):
    """Chunk means of K [Hkv][T][D] for chunks c_begin..c_end-1.

    Writes rows into ``out`` ([Hkv][n_cap][D] float64, created if None) and
    returns it. Rows outside the range are left as they were (NaN if new)."""
    K = _f32(K)
    Hkv, T, D = K.shape
    if n_cap is None:
        n_cap = out.shape[1] if out is not None else T // C
    if out is None:
        out = np.full((Hkv, n_cap, D), np.nan)
    assert out.shape == (Hkv, n_cap, D) and out.dtype == np.float64 and out.flags.c_contiguous
    assert 0 <= c_begin <= c_end <= n_cap and c_end * C <= T
    _load().oracle_summarize(K, Hkv, T, D, C, c_begin, c_end, out, n_cap)
    return out


def route(Q, S, p0: int, k: int, Hkv: int, C: int = 64, Bq: int = 64, want_scores=False,
          sink: int = 0, per_q_head: bool = False, prev_block: bool = False, Q_prev=None):
    """Per (kv head, block) top-k chunk ids, ascending, -1 padded. Candidates
    are the closed chunks before the block that lie past the first ``sink``
    tokens (the sink window, attended by every block; a multiple of C).

    per_q_head: one routing unit per query head (ids [Hq][n_blocks][k]).
    prev_block: strictly causal routing -- block b scores with the queries of
    the block before it; Q_prev [Hq][Bq][D] holds the Bq queries before p0
    (None only when p0 == 0).

    Returns ids [units][n_blocks][k] int32 (and sigma [units][n_blocks][n_cap]
    float64, NaN for ineligible chunks, if want_scores)."""
    Q = _f32(Q)
    Hq, n_q, D = Q.shape
    S = np.ascontiguousarray(S, dtype=np.float64)
    assert S.shape[0] == Hkv and S.shape[2] == D
    n_cap = S.shape[1]
    n_blocks = n_q // Bq
    units = Hq if per_q_head else Hkv
    ids = np.empty((units, n_blocks, k), dtype=np.int32)
    sig = np.empty((units, n_blocks, n_cap)) if want_scores else None
    assert sink % C == 0 and sink >= 0
    qp = None
    if prev_block and Q_prev is not None:
        qp = _f32(Q_prev)
        assert qp.shape == (Hq, Bq, D)
    assert not prev_block or qp is not None or p0 == 0
    _load().oracle_route(Q, Hq, Hkv, n_q, D, p0, C, Bq, S, n_cap, k, ids,
                         sig.ctypes.data_as(ctypes.c_void_p) if want_scores else None, sink,
                         int(per_q_head),
                         qp.ctypes.data_as(ctypes.c_void_p) if qp is not None else None,
                         int(prev_block))
    return (ids, sig) if want_scores else ids


def route_groups(Q, SG, p0: int, chunk_ids, m: int, Hkv: int, C: int = 64, Bq: int = 64,
                 U: int = 8, want_scores=False, sink: int = 0):
    """Per (kv head, block) top-m groups of U tokens among the groups of the
    block's routed chunks (chunk_ids [Hkv][n_blocks][k]) past the first
    ``sink`` tokens, ascending, -1 padded.

    SG holds group summaries [Hkv][n_gcap][D] (summarize with C = U). Returns
    gids [Hkv][n_blocks][m] int32 (and sigma [Hkv][n_blocks][n_gcap] float64,
    NaN for groups that are not candidates, if want_scores)."""
    Q = _f32(Q)
    Hq, n_q, D = Q.shape
    SG = np.ascontiguousarray(SG, dtype=np.float64)
    assert SG.shape[0] == Hkv and SG.shape[2] == D and C % U == 0
    n_gcap = SG.shape[1]
    chunk_ids = np.ascontiguousarray(chunk_ids, dtype=np.int32)
    n_blocks = n_q // Bq
    assert chunk_ids.shape[:2] == (Hkv, n_blocks)
    gids = np.empty((Hkv, n_blocks, m), dtype=np.int32)
    sig = np.empty((Hkv, n_blocks, n_gcap)) if want_scores else None
    assert sink % C == 0 and sink >= 0
    _load().oracle_route_groups(Q, Hq, Hkv, n_q, D, p0, C, Bq, U, SG, n_gcap, chunk_ids,
                                chunk_ids.shape[2], m, gids,
                                sig.ctypes.data_as(ctypes.c_void_p) if want_scores else None,
                                sink)
    return (gids, sig) if want_scores else gids


def attend_fwd(Q, K, V, ids, p0: int, C: int = 64, Bq: int = 64, scale: float | None = None,
               unit_mask=None, sink: int = 0, per_q_head: bool = False):
    """Exact attention over the first ``sink`` tokens (the sink window; a
    multiple of C), the routed units and the causal local block. ids count
    units of C tokens: chunks (C = 64) or groups (C = 8, with Bq = 64); one
    row per (kv head, block), or per (query head, block) with per_q_head.

    Returns (O [Hq][n_q][D], lse [Hq][n_q]) float64; rows of units excluded by
    ``unit_mask`` ([Hq][n_blocks]) are NaN."""
    Q, K, V = _f32(Q), _f32(K), _f32(V)
    Hq, n_q, D = Q.shape
    Hkv, T, _ = K.shape
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    k = ids.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    O = np.full((Hq, n_q, D), np.nan)
    lse = np.full((Hq, n_q), np.nan)
    m, mp = _mask_ptr(unit_mask)
    assert sink % C == 0 and sink >= 0
    assert ids.shape[:2] == ((Hq if per_q_head else Hkv), n_q // Bq)
    _load().oracle_attend_fwd(Q, K, V, Hq, Hkv, D, T, p0, n_q, C, Bq, ids, k,
                              float(scale), mp, O, lse, sink, int(per_q_head))
    return O, lse


def attend_bwd(Q, K, V, dO, ids, p0: int, C: int = 64, Bq: int = 64,
               scale: float | None = None, dq_mask=None, dkv_mask=None, sink: int = 0,
               per_q_head: bool = False):
    """Gradients of sum(O * dO): dQ [Hq][n_q][D], and dK, dV [Hkv][n_q][D] for
    the active keys p0 .. p0+n_q-1 only (history detached); the attended set
    as in attend_fwd, sink window and id-row granularity included."""
    Q, K, V, dO = _f32(Q), _f32(K), _f32(V), _f32(dO)
    Hq, n_q, D = Q.shape
    Hkv, T, _ = K.shape
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    k = ids.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dQ = np.full((Hq, n_q, D), np.nan)
    dK = np.full((Hkv, n_q, D), np.nan)
    dV = np.full((Hkv, n_q, D), np.nan)
    m1, p1 = _mask_ptr(dq_mask)
    m2, p2 = _mask_ptr(dkv_mask)
    assert sink % C == 0 and sink >= 0
    assert ids.shape[:2] == ((Hq if per_q_head else Hkv), n_q // Bq)
    _load().oracle_attend_bwd(Q, K, V, dO, Hq, Hkv, D, T, p0, n_q, C, Bq, ids, k,
                              float(scale), p1, p2, dQ, dK, dV, sink, int(per_q_head))
    return dQ, dK, dV


def route_decode(Q, S, p0: int, k: int, Hkv: int, C: int = 64, want_scores=False,
                 sink: int = 0):
    """Routing of a decode step, one token at a time: token i (position
    p0 + i) routes on the mean of its own G query heads over the closed chunks
    before its open chunk -- the block router with blocks of one query.
    Returns ids [Hkv][n_q][k] (and sigma [Hkv][n_q][n_cap])."""
    return route(Q, S, p0, k, Hkv, C, 1, want_scores=want_scores, sink=sink)


def attend_decode(Q, K, V, ids, p0: int, C: int = 64, scale: float | None = None,
                  sink: int = 0):
    """Exact attention of a decode step: token i at p = p0 + i attends the
    sink window, its routed chunks before its open chunk, and its open chunk
    up to p. ids [Hkv][n_q][k]. Returns (O [Hq][n_q][D], lse [Hq][n_q])."""
    Q, K, V = _f32(Q), _f32(K), _f32(V)
    Hq, n_q, D = Q.shape
    Hkv, T, _ = K.shape
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    assert ids.shape[:2] == (Hkv, n_q) and sink % C == 0 and sink >= 0
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    O = np.full((Hq, n_q, D), np.nan)
    lse = np.full((Hq, n_q), np.nan)
    _load().oracle_attend_decode(Q, K, V, Hq, Hkv, D, T, p0, n_q, C, ids, ids.shape[2],
                                 float(scale), sink, O, lse)
    return O, lse
