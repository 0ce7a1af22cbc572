"""Thin ctypes binding of libhga (include/hga.h), one Python function per C
entry point and with the same name. Argument marshalling only: torch tensors
provide device memory and the current HIP stream; every step of the hot path
runs in the library's HIP kernels. There is no fallback: without a built
``libhga.so`` every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhga.so")

HGA_OK = 0
HGA_ERR_INVALID_ARG = 1
HGA_ERR_UNSUPPORTED = 2
HGA_ERR_CAPACITY = 3
HGA_ERR_HIP = 4
HGA_BF16 = 0

EXPORTED = ("hga_summarize", "hga_route", "hga_route_causal", "hga_attend_fwd",
            "hga_route_attend_fwd",
            "hga_attend_bwd_workspace_bytes", "hga_attend_bwd", "hga_attend_bwd_noalloc",
            "hga_summarize_groups", "hga_route_groups", "hga_attend_fwd_groups",
            "hga_route_attend_fwd_groups",
            "hga_attend_bwd_groups", "hga_route_decode", "hga_decode_workspace_bytes",
            "hga_attend_decode", "hga_route_attend_decode_workspace_bytes",
            "hga_route_attend_decode", "hga_diag_gather_sink_words", "hga_diag_gather",
            "hga_diag_bwd_second_pass", "hga_status_string", "hga_last_error", "hga_version")
HGA_GROUP = 8
HGA_MAX_SINK_CHUNKS = 64
HGA_ROUTE_PER_KV_HEAD = 0
HGA_ROUTE_PER_Q_HEAD = 1
HGA_BWD_NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024


class hga_config(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("q_block", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("sink_chunks", ctypes.c_int32), ("route_heads", ctypes.c_int32)]


def make_config(n_q_heads: int, n_kv_heads: int, top_k: int, *, head_dim: int = 128,
                chunk: int = 64, q_block: int = 64, softmax_scale: float = 0.0,
                dtype: int = HGA_BF16, sink_chunks: int = 0,
                route_heads: int = HGA_ROUTE_PER_KV_HEAD) -> hga_config:
    return hga_config(n_q_heads, n_kv_heads, head_dim, chunk, q_block, top_k,
                      softmax_scale, dtype, sink_chunks, route_heads)


class HGAError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"{fn}: {_status_name(status)}: {detail}")


_lib = None
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_cfgp = ctypes.POINTER(hga_config)


def lib() -> ctypes.CDLL:
    """The loaded libhga (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libhga.so not found at {LIB_PATH}; build it with "
            "`python -m sparse_long_context_summarize_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    L.hga_summarize.argtypes = [_cfgp, _vp, _i64, _i64, _i64, _vp, _i64, _vp]
    L.hga_route.argtypes = [_cfgp, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _vp]
    L.hga_route_causal.argtypes = [_cfgp, _vp, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp,
                                   _vp]
    L.hga_attend_fwd.argtypes = [_cfgp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp]
    L.hga_attend_bwd_workspace_bytes.argtypes = [_cfgp, _i64]
    L.hga_attend_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.hga_attend_bwd.argtypes = [_cfgp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp,
                                 _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.hga_attend_bwd_noalloc.argtypes = [_cfgp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp,
                                         _vp, _vp, _vp, _vp, _vp]
    L.hga_route_attend_fwd.argtypes = [_cfgp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i64, _i64,
                                       _vp, _vp, _vp, _vp, _vp]
    L.hga_summarize_groups.argtypes = [_cfgp, _vp, _i64, _i64, _i64, _vp, _i64, _vp]
    L.hga_route_groups.argtypes = [_cfgp, _vp, _i64, _i64, _vp, _i64, _vp, ctypes.c_int32,
                                   _vp, _vp, _vp]
    L.hga_attend_fwd_groups.argtypes = [_cfgp, _vp, _vp, _vp, _i64, _i64, _i64, _vp,
                                        ctypes.c_int32, _vp, _vp, _vp]
    L.hga_route_attend_fwd_groups.argtypes = [_cfgp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i64,
                                              _i64, _vp, _i64, ctypes.c_int32, _vp, _vp, _vp,
                                              _vp, _vp, _vp]
    L.hga_route_decode.argtypes = [_cfgp, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _vp,
                                   ctypes.c_size_t, _vp]
    L.hga_decode_workspace_bytes.argtypes = [_cfgp, _i64, _i64]
    L.hga_decode_workspace_bytes.restype = ctypes.c_size_t
    L.hga_attend_decode.argtypes = [_cfgp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp,
                                    ctypes.c_size_t, _vp]
    L.hga_route_attend_decode_workspace_bytes.argtypes = [_cfgp, _i64, _i64]
    L.hga_route_attend_decode_workspace_bytes.restype = ctypes.c_size_t
    L.hga_route_attend_decode.argtypes = [_cfgp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i64,
                                          _i64, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.hga_diag_gather_sink_words.argtypes = [_cfgp, _i64]
    L.hga_diag_gather_sink_words.restype = ctypes.c_size_t
    L.hga_diag_gather.argtypes = [_cfgp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, ctypes.c_size_t,
                                  _vp]
    L.hga_diag_bwd_second_pass.argtypes = [_cfgp, _i64, _vp, ctypes.c_size_t,
                                           ctypes.POINTER(ctypes.c_int64),
                                           ctypes.POINTER(ctypes.c_int64), _vp]
    L.hga_diag_bwd_second_pass.restype = ctypes.c_int
    L.hga_attend_bwd_groups.argtypes = [_cfgp, _vp, _vp, _vp, _i64, _i64, _i64, _vp,
                                        ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        ctypes.c_size_t, _vp]
    for fn in ("hga_summarize", "hga_route", "hga_route_causal", "hga_attend_fwd",
               "hga_attend_bwd", "hga_attend_bwd_noalloc",
               "hga_route_attend_fwd",
               "hga_summarize_groups", "hga_route_groups", "hga_attend_fwd_groups",
               "hga_route_attend_fwd_groups",
               "hga_attend_bwd_groups", "hga_diag_gather", "hga_route_decode",
               "hga_attend_decode", "hga_route_attend_decode"):
        getattr(L, fn).restype = ctypes.c_int
    L.hga_status_string.argtypes = [ctypes.c_int]
    L.hga_status_string.restype = ctypes.c_char_p
    L.hga_last_error.restype = ctypes.c_char_p
    L.hga_version.restype = ctypes.c_int32
    _lib = L
    return L


def _status_name(status: int) -> str:
    return lib().hga_status_string(status).decode()


def hga_status_string(status: int) -> str:
    return _status_name(status)


def hga_last_error() -> str:
    return lib().hga_last_error().decode()


def hga_version() -> int:
    return int(lib().hga_version())


def _check(fn: str, status: int) -> None:
    if status != HGA_OK:
        raise HGAError(fn, status, hga_last_error())


def _dev(t: torch.Tensor | None, name: str, dtype: torch.dtype):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _units(cfg: hga_config) -> int:
    """Id rows per query block: one per kv head, or per query head."""
    return cfg.n_q_heads if cfg.route_heads == HGA_ROUTE_PER_Q_HEAD else cfg.n_kv_heads


def _blocks(cfg: hga_config, n_q: int) -> int:
    return n_q // cfg.q_block if cfg.q_block > 0 else 0


def _shape(t, name: str, want) -> None:
    """Refuse a tensor whose shape differs from the one the call implies (a
    wrong shape would otherwise become an out-of-bounds device access: the C
    ABI sees pointers only). Entries of `want` that are None are free."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    got = tuple(t.shape)
    if len(got) != len(want) or any(w is not None and g != w for g, w in zip(got, want)):
        shown = tuple("*" if w is None else w for w in want)
        raise ValueError(f"{name} has shape {got}; this call needs {shown}")


def _q_shapes(cfg: hga_config, Q, name: str = "Q") -> int:
    _shape(Q, name, (cfg.n_q_heads, None, cfg.head_dim))
    return Q.shape[1]


def _kv_shapes(cfg: hga_config, K, V=None) -> None:
    _shape(K, "K", (cfg.n_kv_heads, None, cfg.head_dim))
    if V is not None and tuple(K.shape) != tuple(V.shape):
        raise ValueError("K and V shapes differ")


def _summary_shapes(cfg: hga_config, S, name: str = "summaries") -> None:
    _shape(S, name, (cfg.n_kv_heads, None, cfg.head_dim))


def _out_shapes(cfg: hga_config, n_q: int, O, lse, O_name: str = "O") -> None:
    _shape(O, O_name, (cfg.n_q_heads, n_q, cfg.head_dim))
    _shape(lse, "lse", (cfg.n_q_heads, n_q))


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _m_summarize(cfg: hga_config, K, tok_begin: int, n_tok: int, summaries, stream=None):
    _kv_shapes(cfg, K)
    _summary_shapes(cfg, summaries)
    return (ctypes.byref(cfg), _dev(K, "K", torch.bfloat16), K.shape[1], tok_begin, n_tok,
            _dev(summaries, "summaries", torch.float32), summaries.shape[1], _stream(stream))


def _m_route(cfg: hga_config, Q, p0: int, summaries, n_chunks_valid: int, ids, scores=None,
             stream=None):
    n_q = _q_shapes(cfg, Q)
    _summary_shapes(cfg, summaries)
    _shape(ids, "ids", (_units(cfg), _blocks(cfg, n_q), cfg.top_k))
    _shape(scores, "scores", (_units(cfg), _blocks(cfg, n_q), cfg.top_k))
    return (ctypes.byref(cfg), _dev(Q, "Q", torch.bfloat16), p0, Q.shape[1],
            _dev(summaries, "summaries", torch.float32), summaries.shape[1], n_chunks_valid,
            _dev(ids, "ids", torch.int32), _dev(scores, "scores", torch.float32),
            _stream(stream))


def _m_route_causal(cfg: hga_config, Q, Q_prev, p0: int, summaries, n_chunks_valid: int, ids,
                    scores=None, stream=None):
    n_q = _q_shapes(cfg, Q)
    _shape(Q_prev, "Q_prev", (cfg.n_q_heads, cfg.q_block, cfg.head_dim))
    _summary_shapes(cfg, summaries)
    _shape(ids, "ids", (_units(cfg), _blocks(cfg, n_q), cfg.top_k))
    _shape(scores, "scores", (_units(cfg), _blocks(cfg, n_q), cfg.top_k))
    return (ctypes.byref(cfg), _dev(Q, "Q", torch.bfloat16),
            _dev(Q_prev, "Q_prev", torch.bfloat16), p0, Q.shape[1],
            _dev(summaries, "summaries", torch.float32), summaries.shape[1], n_chunks_valid,
            _dev(ids, "ids", torch.int32), _dev(scores, "scores", torch.float32),
            _stream(stream))


def _m_attend_fwd(cfg: hga_config, Q, K, V, p0: int, ids, O, lse, stream=None):
    n_q = _q_shapes(cfg, Q)
    _kv_shapes(cfg, K, V)
    _shape(ids, "ids", (_units(cfg), _blocks(cfg, n_q), cfg.top_k))
    _out_shapes(cfg, n_q, O, lse)
    args = (_dev(Q, "Q", torch.bfloat16), _dev(K, "K", torch.bfloat16),
            _dev(V, "V", torch.bfloat16))
    if K.shape != V.shape:
        raise ValueError("K and V shapes differ")
    return (ctypes.byref(cfg), *args, K.shape[1], p0, Q.shape[1], _dev(ids, "ids", torch.int32),
            _dev(O, "O", torch.bfloat16), _dev(lse, "lse", torch.float32), _stream(stream))


def _m_attend_bwd(cfg: hga_config, Q, K, V, p0: int, ids, O, lse, dO, dQ, dK, dV, workspace,
                  stream=None):
    n_q = _q_shapes(cfg, Q)
    _kv_shapes(cfg, K, V)
    _shape(ids, "ids", (_units(cfg), _blocks(cfg, n_q), cfg.top_k))
    _out_shapes(cfg, n_q, O, lse)
    _shape(dO, "dO", (cfg.n_q_heads, n_q, cfg.head_dim))
    _shape(dQ, "dQ", (cfg.n_q_heads, n_q, cfg.head_dim))
    _shape(dK, "dK", (cfg.n_kv_heads, n_q, cfg.head_dim))
    _shape(dV, "dV", (cfg.n_kv_heads, n_q, cfg.head_dim))
    if K.shape != V.shape:
        raise ValueError("K and V shapes differ")
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" \
            or not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous GPU memory")
    ws_bytes = workspace.numel() * workspace.element_size()
    return (ctypes.byref(cfg), _dev(Q, "Q", torch.bfloat16), _dev(K, "K", torch.bfloat16),
            _dev(V, "V", torch.bfloat16), K.shape[1], p0, Q.shape[1],
            _dev(ids, "ids", torch.int32), _dev(O, "O", torch.bfloat16),
            _dev(lse, "lse", torch.float32), _dev(dO, "dO", torch.bfloat16),
            _dev(dQ, "dQ", torch.float32), _dev(dK, "dK", torch.float32),
            _dev(dV, "dV", torch.float32), workspace.data_ptr(), ws_bytes, _stream(stream))


def _m_attend_bwd_noalloc(cfg: hga_config, Q, K, V, p0: int, ids, O, lse, dO, dQ, dK, dV,
                          stream=None):
    n_q = _q_shapes(cfg, Q)
    _kv_shapes(cfg, K, V)
    _shape(ids, "ids", (_units(cfg), _blocks(cfg, n_q), cfg.top_k))
    _out_shapes(cfg, n_q, O, lse)
    _shape(dO, "dO", (cfg.n_q_heads, n_q, cfg.head_dim))
    _shape(dQ, "dQ", (cfg.n_q_heads, n_q, cfg.head_dim))
    _shape(dK, "dK", (cfg.n_kv_heads, n_q, cfg.head_dim))
    _shape(dV, "dV", (cfg.n_kv_heads, n_q, cfg.head_dim))
    return (ctypes.byref(cfg), _dev(Q, "Q", torch.bfloat16), _dev(K, "K", torch.bfloat16),
            _dev(V, "V", torch.bfloat16), K.shape[1], p0, Q.shape[1],
            _dev(ids, "ids", torch.int32), _dev(O, "O", torch.bfloat16),
            _dev(lse, "lse", torch.float32), _dev(dO, "dO", torch.bfloat16),
            _dev(dQ, "dQ", torch.float32), _dev(dK, "dK", torch.float32),
            _dev(dV, "dV", torch.float32), _stream(stream))


def _m_route_attend_fwd(cfg: hga_config, Q, K, V, p0: int, summaries, n_chunks_valid: int, ids,
                        O, lse, scores=None, stream=None):
    n_q = _q_shapes(cfg, Q)
    _kv_shapes(cfg, K, V)
    _summary_shapes(cfg, summaries)
    _shape(ids, "ids", (_units(cfg), _blocks(cfg, n_q), cfg.top_k))
    _shape(scores, "scores", (_units(cfg), _blocks(cfg, n_q), cfg.top_k))
    _out_shapes(cfg, n_q, O, lse)
    args = (_dev(Q, "Q", torch.bfloat16), _dev(K, "K", torch.bfloat16),
            _dev(V, "V", torch.bfloat16))
    if K.shape != V.shape:
        raise ValueError("K and V shapes differ")
    return (ctypes.byref(cfg), *args, K.shape[1], p0, Q.shape[1],
            _dev(summaries, "summaries", torch.float32),
            summaries.shape[1] if summaries is not None else 0, n_chunks_valid,
            _dev(ids, "ids", torch.int32), _dev(scores, "scores", torch.float32),
            _dev(O, "O", torch.bfloat16), _dev(lse, "lse", torch.float32), _stream(stream))


def _m_summarize_groups(cfg: hga_config, K, tok_begin: int, n_tok: int, group_summaries,
                        stream=None):
    _kv_shapes(cfg, K)
    _summary_shapes(cfg, group_summaries, "group_summaries")
    return (ctypes.byref(cfg), _dev(K, "K", torch.bfloat16), K.shape[1], tok_begin, n_tok,
            _dev(group_summaries, "group_summaries", torch.float32), group_summaries.shape[1],
            _stream(stream))


def _m_route_groups(cfg: hga_config, Q, p0: int, group_summaries, chunk_ids, group_ids,
                    scores=None, stream=None):
    n_q = _q_shapes(cfg, Q)
    _summary_shapes(cfg, group_summaries, "group_summaries")
    _shape(chunk_ids, "chunk_ids", (cfg.n_kv_heads, _blocks(cfg, n_q), cfg.top_k))
    _shape(group_ids, "group_ids", (cfg.n_kv_heads, _blocks(cfg, n_q), None))
    _shape(scores, "scores", (cfg.n_kv_heads, _blocks(cfg, n_q), group_ids.shape[2]))
    return (ctypes.byref(cfg), _dev(Q, "Q", torch.bfloat16), p0, Q.shape[1],
            _dev(group_summaries, "group_summaries", torch.float32), group_summaries.shape[1],
            _dev(chunk_ids, "chunk_ids", torch.int32), group_ids.shape[2],
            _dev(group_ids, "group_ids", torch.int32), _dev(scores, "scores", torch.float32),
            _stream(stream))


def _m_route_attend_fwd_groups(cfg: hga_config, Q, K, V, p0: int, summaries, n_chunks_valid: int,
                               group_summaries, chunk_ids, group_ids, O, lse, scores=None,
                               stream=None):
    n_q = _q_shapes(cfg, Q)
    _kv_shapes(cfg, K, V)
    _summary_shapes(cfg, summaries)
    _summary_shapes(cfg, group_summaries, "group_summaries")
    _shape(chunk_ids, "chunk_ids", (cfg.n_kv_heads, _blocks(cfg, n_q), cfg.top_k))
    _shape(group_ids, "group_ids", (cfg.n_kv_heads, _blocks(cfg, n_q), None))
    _shape(scores, "scores", (cfg.n_kv_heads, _blocks(cfg, n_q), group_ids.shape[2]))
    _out_shapes(cfg, n_q, O, lse)
    args = (_dev(Q, "Q", torch.bfloat16), _dev(K, "K", torch.bfloat16),
            _dev(V, "V", torch.bfloat16))
    return (ctypes.byref(cfg), *args, K.shape[1], p0, Q.shape[1],
            _dev(summaries, "summaries", torch.float32), summaries.shape[1], n_chunks_valid,
            _dev(group_summaries, "group_summaries", torch.float32), group_summaries.shape[1],
            group_ids.shape[2], _dev(chunk_ids, "chunk_ids", torch.int32),
            _dev(group_ids, "group_ids", torch.int32), _dev(scores, "scores", torch.float32),
            _dev(O, "O", torch.bfloat16), _dev(lse, "lse", torch.float32), _stream(stream))


def _m_attend_fwd_groups(cfg: hga_config, Q, K, V, p0: int, group_ids, O, lse, stream=None):
    n_q = _q_shapes(cfg, Q)
    _kv_shapes(cfg, K, V)
    _shape(group_ids, "group_ids", (cfg.n_kv_heads, _blocks(cfg, n_q), None))
    _out_shapes(cfg, n_q, O, lse)
    args = (_dev(Q, "Q", torch.bfloat16), _dev(K, "K", torch.bfloat16),
            _dev(V, "V", torch.bfloat16))
    return (ctypes.byref(cfg), *args, K.shape[1], p0, Q.shape[1],
            _dev(group_ids, "group_ids", torch.int32), group_ids.shape[2],
            _dev(O, "O", torch.bfloat16), _dev(lse, "lse", torch.float32), _stream(stream))


def _m_attend_bwd_groups(cfg: hga_config, Q, K, V, p0: int, group_ids, O, lse, dO, dQ, dK, dV,
                        workspace, stream=None):
    n_q = _q_shapes(cfg, Q)
    _kv_shapes(cfg, K, V)
    _shape(group_ids, "group_ids", (cfg.n_kv_heads, _blocks(cfg, n_q), None))
    _out_shapes(cfg, n_q, O, lse)
    _shape(dO, "dO", (cfg.n_q_heads, n_q, cfg.head_dim))
    _shape(dQ, "dQ", (cfg.n_q_heads, n_q, cfg.head_dim))
    _shape(dK, "dK", (cfg.n_kv_heads, n_q, cfg.head_dim))
    _shape(dV, "dV", (cfg.n_kv_heads, n_q, cfg.head_dim))
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" \
            or not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous GPU memory")
    ws_bytes = workspace.numel() * workspace.element_size()
    return (ctypes.byref(cfg), _dev(Q, "Q", torch.bfloat16), _dev(K, "K", torch.bfloat16),
            _dev(V, "V", torch.bfloat16), K.shape[1], p0, Q.shape[1],
            _dev(group_ids, "group_ids", torch.int32), group_ids.shape[2],
            _dev(O, "O", torch.bfloat16), _dev(lse, "lse", torch.float32),
            _dev(dO, "dO", torch.bfloat16), _dev(dQ, "dQ", torch.float32),
            _dev(dK, "dK", torch.float32), _dev(dV, "dV", torch.float32), workspace.data_ptr(),
            ws_bytes, _stream(stream))


def _workspace(workspace):
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" \
            or not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous GPU memory")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _m_route_decode(cfg: hga_config, Q, p0: int, summaries, n_chunks_valid: int, ids,
                    workspace, scores=None, stream=None):
    n_q = _q_shapes(cfg, Q)
    _summary_shapes(cfg, summaries)
    _shape(ids, "ids", (cfg.n_kv_heads, n_q, cfg.top_k))
    _shape(scores, "scores", (cfg.n_kv_heads, n_q, cfg.top_k))
    return (ctypes.byref(cfg), _dev(Q, "Q", torch.bfloat16), p0, Q.shape[1],
            _dev(summaries, "summaries", torch.float32), summaries.shape[1], n_chunks_valid,
            _dev(ids, "ids", torch.int32), _dev(scores, "scores", torch.float32),
            *_workspace(workspace), _stream(stream))


def _m_attend_decode(cfg: hga_config, Q, K, V, p0: int, ids, O, lse, workspace, stream=None):
    n_q = _q_shapes(cfg, Q)
    _kv_shapes(cfg, K, V)
    _shape(ids, "ids", (cfg.n_kv_heads, n_q, cfg.top_k))
    _out_shapes(cfg, n_q, O, lse)
    _workspace(workspace)
    return (ctypes.byref(cfg), _dev(Q, "Q", torch.bfloat16), _dev(K, "K", torch.bfloat16),
            _dev(V, "V", torch.bfloat16), K.shape[1], p0, Q.shape[1],
            _dev(ids, "ids", torch.int32), _dev(O, "O", torch.bfloat16),
            _dev(lse, "lse", torch.float32), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream(stream))


def _m_route_attend_decode(cfg: hga_config, Q, K, V, p0: int, summaries, n_chunks_valid: int,
                           ids, O, lse, workspace, scores=None, stream=None):
    n_q = _q_shapes(cfg, Q)
    _kv_shapes(cfg, K, V)
    _summary_shapes(cfg, summaries)
    _shape(ids, "ids", (cfg.n_kv_heads, n_q, cfg.top_k))
    _shape(scores, "scores", (cfg.n_kv_heads, n_q, cfg.top_k))
    _out_shapes(cfg, n_q, O, lse)
    return (ctypes.byref(cfg), _dev(Q, "Q", torch.bfloat16), _dev(K, "K", torch.bfloat16),
            _dev(V, "V", torch.bfloat16), K.shape[1], p0, Q.shape[1],
            _dev(summaries, "summaries", torch.float32),
            summaries.shape[1] if summaries is not None else 0, n_chunks_valid,
            _dev(ids, "ids", torch.int32), _dev(scores, "scores", torch.float32),
            _dev(O, "O", torch.bfloat16), _dev(lse, "lse", torch.float32),
            *_workspace(workspace), _stream(stream))


def _m_diag_gather(cfg: hga_config, K, V, p0: int, n_q: int, ids, sink, stream=None):
    _kv_shapes(cfg, K, V)
    _shape(ids, "ids", (cfg.n_kv_heads, _blocks(cfg, n_q), cfg.top_k))
    return (ctypes.byref(cfg), _dev(K, "K", torch.bfloat16), _dev(V, "V", torch.bfloat16),
            K.shape[1], p0, n_q, _dev(ids, "ids", torch.int32), _dev(sink, "sink", torch.int32),
            sink.numel(), _stream(stream))


_MARSHAL = {"hga_summarize": _m_summarize, "hga_route": _m_route,
            "hga_route_causal": _m_route_causal,
            "hga_attend_fwd": _m_attend_fwd, "hga_attend_bwd": _m_attend_bwd,
            "hga_attend_bwd_noalloc": _m_attend_bwd_noalloc,
            "hga_route_attend_fwd": _m_route_attend_fwd,
            "hga_summarize_groups": _m_summarize_groups, "hga_route_groups": _m_route_groups,
            "hga_attend_fwd_groups": _m_attend_fwd_groups,
            "hga_route_attend_fwd_groups": _m_route_attend_fwd_groups,
            "hga_attend_bwd_groups": _m_attend_bwd_groups,
            "hga_diag_gather": _m_diag_gather, "hga_route_decode": _m_route_decode,
            "hga_attend_decode": _m_attend_decode,
            "hga_route_attend_decode": _m_route_attend_decode}


def hga_summarize(cfg: hga_config, K: torch.Tensor, tok_begin: int, n_tok: int,
                  summaries: torch.Tensor, stream=None) -> None:
    """K bf16 [Hkv][T_cap][D]; summaries f32 [Hkv][n_chunk_cap][D]."""
    _check("hga_summarize", lib().hga_summarize(
        *_m_summarize(cfg, K, tok_begin, n_tok, summaries, stream)))


def hga_route(cfg: hga_config, Q: torch.Tensor, p0: int, summaries: torch.Tensor,
              n_chunks_valid: int, ids: torch.Tensor, scores: torch.Tensor | None = None,
              stream=None) -> None:
    """Q bf16 [Hq][n_q][D]; ids int32 [U][n_q/64][k] (U = Hkv, or Hq with per-query-head
    routing); scores f32 like ids or None."""
    _check("hga_route", lib().hga_route(
        *_m_route(cfg, Q, p0, summaries, n_chunks_valid, ids, scores, stream)))


def hga_route_causal(cfg: hga_config, Q: torch.Tensor, Q_prev: torch.Tensor | None, p0: int,
                     summaries: torch.Tensor, n_chunks_valid: int, ids: torch.Tensor,
                     scores: torch.Tensor | None = None, stream=None) -> None:
    """Strictly causal routing: block b scores with the 64 queries before it
    (Q_prev bf16 [Hq][64][D] for the first block; None only when p0 == 0)."""
    _check("hga_route_causal", lib().hga_route_causal(
        *_m_route_causal(cfg, Q, Q_prev, p0, summaries, n_chunks_valid, ids, scores, stream)))


def hga_attend_fwd(cfg: hga_config, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                   p0: int, ids: torch.Tensor, O: torch.Tensor, lse: torch.Tensor,
                   stream=None) -> None:
    """O bf16 [Hq][n_q][D], lse f32 [Hq][n_q] are written."""
    _check("hga_attend_fwd", lib().hga_attend_fwd(
        *_m_attend_fwd(cfg, Q, K, V, p0, ids, O, lse, stream)))


def hga_attend_bwd_workspace_bytes(cfg: hga_config, n_q: int) -> int:
    return int(lib().hga_attend_bwd_workspace_bytes(ctypes.byref(cfg), n_q))


def hga_attend_bwd(cfg: hga_config, Q, K, V, p0: int, ids, O, lse, dO, dQ, dK, dV,
                   workspace: torch.Tensor, stream=None) -> None:
    """dQ f32 [Hq][n_q][D]; dK, dV f32 [Hkv][n_q][D] (active keys) are written."""
    _check("hga_attend_bwd", lib().hga_attend_bwd(
        *_m_attend_bwd(cfg, Q, K, V, p0, ids, O, lse, dO, dQ, dK, dV, workspace, stream)))


def hga_attend_bwd_noalloc(cfg: hga_config, Q, K, V, p0: int, ids, O, lse, dO, dQ, dK, dV,
                           stream=None) -> None:
    """hga_attend_bwd on the library's fixed scratch (no workspace argument)."""
    _check("hga_attend_bwd_noalloc", lib().hga_attend_bwd_noalloc(
        *_m_attend_bwd_noalloc(cfg, Q, K, V, p0, ids, O, lse, dO, dQ, dK, dV, stream)))


def hga_route_attend_fwd(cfg: hga_config, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                         p0: int, summaries: torch.Tensor, n_chunks_valid: int,
                         ids: torch.Tensor, O: torch.Tensor, lse: torch.Tensor,
                         scores: torch.Tensor | None = None, stream=None) -> None:
    """hga_route then hga_attend_fwd in one launch; ids (and scores) are
    written as hga_route writes them."""
    _check("hga_route_attend_fwd", lib().hga_route_attend_fwd(
        *_m_route_attend_fwd(cfg, Q, K, V, p0, summaries, n_chunks_valid, ids, O, lse, scores,
                             stream)))


def hga_summarize_groups(cfg: hga_config, K: torch.Tensor, tok_begin: int, n_tok: int,
                         group_summaries: torch.Tensor, stream=None) -> None:
    """K bf16 [Hkv][T_cap][D]; group_summaries f32 [Hkv][n_group_cap][D]."""
    _check("hga_summarize_groups", lib().hga_summarize_groups(
        *_m_summarize_groups(cfg, K, tok_begin, n_tok, group_summaries, stream)))


def hga_route_groups(cfg: hga_config, Q: torch.Tensor, p0: int, group_summaries: torch.Tensor,
                     chunk_ids: torch.Tensor, group_ids: torch.Tensor,
                     scores: torch.Tensor | None = None, stream=None) -> None:
    """chunk_ids int32 [Hkv][n_q/64][top_k] (from hga_route); group_ids int32
    [Hkv][n_q/64][group_top_k] is written (group_top_k = its last dimension)."""
    _check("hga_route_groups", lib().hga_route_groups(
        *_m_route_groups(cfg, Q, p0, group_summaries, chunk_ids, group_ids, scores, stream)))


def hga_attend_fwd_groups(cfg: hga_config, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                          p0: int, group_ids: torch.Tensor, O: torch.Tensor, lse: torch.Tensor,
                          stream=None) -> None:
    """Attention over routed 8-token groups plus the causal local block."""
    _check("hga_attend_fwd_groups", lib().hga_attend_fwd_groups(
        *_m_attend_fwd_groups(cfg, Q, K, V, p0, group_ids, O, lse, stream)))


def hga_route_attend_fwd_groups(cfg: hga_config, Q: torch.Tensor, K: torch.Tensor,
                                V: torch.Tensor, p0: int, summaries: torch.Tensor,
                                n_chunks_valid: int, group_summaries: torch.Tensor,
                                chunk_ids: torch.Tensor, group_ids: torch.Tensor, O: torch.Tensor,
                                lse: torch.Tensor, scores: torch.Tensor | None = None,
                                stream=None) -> None:
    """hga_route, hga_route_groups and hga_attend_fwd_groups in one call
    (one launch when 0 < top_k <= 32); chunk_ids [Hkv][n_q/64][top_k] and
    group_ids [Hkv][n_q/64][group_top_k] are written as those calls write them."""
    _check("hga_route_attend_fwd_groups", lib().hga_route_attend_fwd_groups(
        *_m_route_attend_fwd_groups(cfg, Q, K, V, p0, summaries, n_chunks_valid,
                                    group_summaries, chunk_ids, group_ids, O, lse, scores,
                                    stream)))


def hga_attend_bwd_groups(cfg: hga_config, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                          p0: int, group_ids: torch.Tensor, O, lse: torch.Tensor,
                          dO: torch.Tensor, dQ: torch.Tensor, dK: torch.Tensor, dV: torch.Tensor,
                          workspace: torch.Tensor, stream=None) -> None:
    """Gradients of hga_attend_fwd_groups (dQ; dK, dV of the active keys)."""
    _check("hga_attend_bwd_groups", lib().hga_attend_bwd_groups(
        *_m_attend_bwd_groups(cfg, Q, K, V, p0, group_ids, O, lse, dO, dQ, dK, dV, workspace,
                              stream)))


def hga_route_decode(cfg: hga_config, Q: torch.Tensor, p0: int, summaries: torch.Tensor,
                     n_chunks_valid: int, ids: torch.Tensor, workspace: torch.Tensor,
                     scores: torch.Tensor | None = None, stream=None) -> None:
    """Routing of a decode step, one token at a time (ids [Hkv][n_q][k])."""
    _check("hga_route_decode", lib().hga_route_decode(
        *_m_route_decode(cfg, Q, p0, summaries, n_chunks_valid, ids, workspace, scores,
                         stream)))


def hga_decode_workspace_bytes(cfg: hga_config, p0: int, n_q: int) -> int:
    return int(lib().hga_decode_workspace_bytes(ctypes.byref(cfg), p0, n_q))


def hga_attend_decode(cfg: hga_config, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                      p0: int, ids: torch.Tensor, O: torch.Tensor, lse: torch.Tensor,
                      workspace: torch.Tensor, stream=None) -> None:
    """Attention of a decode step (split over the routed chunks, then merged)."""
    _check("hga_attend_decode", lib().hga_attend_decode(
        *_m_attend_decode(cfg, Q, K, V, p0, ids, O, lse, workspace, stream)))


def hga_route_attend_decode_workspace_bytes(cfg: hga_config, p0: int, n_q: int) -> int:
    return int(lib().hga_route_attend_decode_workspace_bytes(ctypes.byref(cfg), p0, n_q))


def hga_route_attend_decode(cfg: hga_config, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                            p0: int, summaries: torch.Tensor, n_chunks_valid: int,
                            ids: torch.Tensor, O: torch.Tensor, lse: torch.Tensor,
                            workspace: torch.Tensor, scores: torch.Tensor | None = None,
                            stream=None) -> None:
    """Routing and attention of a decode step in one call (two launches)."""
    _check("hga_route_attend_decode", lib().hga_route_attend_decode(
        *_m_route_attend_decode(cfg, Q, K, V, p0, summaries, n_chunks_valid, ids, O, lse,
                                workspace, scores, stream)))


def hga_diag_gather_sink_words(cfg: hga_config, n_q: int) -> int:
    return int(lib().hga_diag_gather_sink_words(ctypes.byref(cfg), n_q))


def hga_diag_gather(cfg: hga_config, K: torch.Tensor, V: torch.Tensor, p0: int, n_q: int,
                    ids: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Diagnostic: read the rows hga_attend_fwd gathers, nothing else (sink is
    int32 scratch of hga_diag_gather_sink_words words)."""
    _check("hga_diag_gather", lib().hga_diag_gather(
        *_m_diag_gather(cfg, K, V, p0, n_q, ids, sink, stream)))


def hga_diag_bwd_second_pass(cfg: hga_config, n_q: int, workspace: torch.Tensor,
                             stream=None) -> tuple[int, int]:
    """Diagnostic: (dq workgroups that ran the second pass, dq workgroups) of
    the last backward call on `workspace`; waits for the stream."""
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" \
            or not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous GPU memory")
    n2, nw = ctypes.c_int64(0), ctypes.c_int64(0)
    _check("hga_diag_bwd_second_pass", lib().hga_diag_bwd_second_pass(
        ctypes.byref(cfg), n_q, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), ctypes.byref(n2), ctypes.byref(nw),
        _stream(stream)))
    return int(n2.value), int(nw.value)


def prepare(name: str, *args, **kwargs):
    """Marshal the arguments of entry point `name` once and return a
    zero-argument callable that repeats that exact C call (same pointers,
    sizes and stream) and raises HGAError on a non-OK status. The tensors
    passed must stay alive, unmoved, for as long as the callable is used.
    For launch loops where per-call argument checks would dominate."""
    fn = getattr(lib(), name)
    cfg = args[0]
    c_args = _MARSHAL[name](*args, **kwargs)

    def run(_fn=fn, _a=c_args, _keep=cfg):
        st = _fn(*_a)
        if st:
            raise HGAError(name, st, hga_last_error())
    return run
