"""Seeded synthetic workloads for the HGA hot path.

This module only draws random numbers and rounds them to the storage precision.
It holds none of the method's arithmetic (no pooling, scoring, selection or
attention), so both the CPU oracle and the GPU path can consume its arrays.

Recipe (one fixed draw order per workload, numpy PCG64, float32 normals):

  Q   [Hq][n_q][D]   ~ N(0, 1)
  K   [Hkv][T][D]    ~ N(0, 1)
  V   [Hkv][T][D]    ~ N(0, 1)
  off [Hkv][T/C]     ~ N(0, 1) * 0.5      one scalar per (kv head, chunk)
  dO  [Hq][n_q][D]   ~ N(0, 1)            backward workload only

  K[g][t][:] += off[g][t // C]            (the all-ones direction, so routing
                                           has structure to find)

bf16 workloads round every array to bfloat16 (round to nearest even) after the
offset is added; both sides then consume the widened values. The per-chunk
offset stands in for the topical structure of real long documents (the pages'
training corpus is a book collection); no dataset item is reproduced.

The five workloads mirror the Qwen3-8B attention layer layout (32 query heads,
8 key/value heads, head dim 128) and the chunk size 64 named on the pages
(arXiv 2607.15105, "Long-Context Fine-Tuning with Limited VRAM", technical
summary section 2.1, chunk selection).
"""
from __future__ import annotations

import dataclasses
import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: object
    Hq: int
    Hkv: int
    D: int
    p0: int          # absolute position of the first active query
    n_q: int         # active queries
    T: int           # tokens held in the K/V buffer
    C: int = 64      # chunk length
    Bq: int = 64     # query block length
    k: int = 16      # routed chunks per block
    m: int = 0       # routed 8-token groups per block (0: whole chunks)
    bf16: bool = True
    with_dO: bool = False

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def n_blocks(self) -> int:
        return self.n_q // self.Bq

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Tiny single-head check, fp32 draws (the GPU consumes bf16-rounded copies).
TINY = Workload("tiny-1h-2k", seed=0, Hq=1, Hkv=1, D=128, p0=1536, n_q=512,
                T=2048, k=4, bf16=False)
# Qwen3-8B layer, 2048 active queries over 14336 history tokens, top-16.
LAYER16K = Workload("qwen3-8b-layer-16k", seed=1, Hq=32, Hkv=8, D=128,
                    p0=14336, n_q=2048, T=16384, k=16)
# Long-context evaluation shape, 4096 active queries over 126976 history, top-32.
LAYER128K = Workload("qwen3-8b-layer-128k", seed=2, Hq=32, Hkv=8, D=128,
                     p0=126976, n_q=4096, T=131072, k=32)
# The 16K layer with the second routing level: of the 16 routed chunks (128
# groups of 8 tokens) each block keeps its best 64 groups, half the tokens.
LAYER16K_GROUPS = LAYER16K.replace(name="qwen3-8b-layer-16k-groups", m=64)
# Segment-wise backward at the 16K layer shape.
BWD16K = Workload("qwen3-8b-bwd-16k", seed=4, Hq=32, Hkv=8, D=128,
                  p0=14336, n_q=2048, T=16384, k=16, with_dO=True)

# Segment loop: 36 layers x 8 segments of 2048 tokens over a 16384-token sequence.
SEGLOOP_LAYERS = 36
SEGLOOP_SEGMENTS = 8
SEGLOOP_SEG_LEN = 2048
SEGLOOP_T = 16384


def seg_layer_workload(layer: int) -> Workload:
    """Per-layer draw of the segment-loop workload: Q covers all 16384 positions."""
    return Workload(f"qwen3-8b-segloop-l{layer}", seed=[3, layer], Hq=32, Hkv=8,
                    D=128, p0=0, n_q=SEGLOOP_T, T=SEGLOOP_T, k=16)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) & np.uint32(0xFFFF0000)).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def generate(w: Workload, *, bf16: bool | None = None) -> dict[str, np.ndarray]:
    """Draw one workload. Returns float32 arrays Q, K, V, off (and dO).

    ``bf16`` overrides the workload's storage precision (used to hand the GPU
    bf16-rounded copies of the fp32 tiny workload).
    """
    rng = np.random.default_rng(w.seed)
    Q = rng.standard_normal((w.Hq, w.n_q, w.D), dtype=np.float32)
    K = rng.standard_normal((w.Hkv, w.T, w.D), dtype=np.float32)
    V = rng.standard_normal((w.Hkv, w.T, w.D), dtype=np.float32)
    off = rng.standard_normal((w.Hkv, w.T // w.C), dtype=np.float32) * np.float32(0.5)
    out = {}
    if w.with_dO:
        out["dO"] = rng.standard_normal((w.Hq, w.n_q, w.D), dtype=np.float32)
    K += np.repeat(off, w.C, axis=1)[:, :, None]
    out.update(Q=Q, K=K, V=V, off=off)
    use_bf16 = w.bf16 if bf16 is None else bf16
    if use_bf16:
        for name in ("Q", "K", "V", "dO"):
            if name in out:
                out[name] = round_bf16(out[name])
    return out


def small_random(seed, Hq, Hkv, D, T, n_q, *, C=64, offset_sd=0.5, bf16=False,
                 with_dO=False) -> dict[str, np.ndarray]:
    """Same recipe at arbitrary (small) sizes, for tests."""
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((Hq, n_q, D), dtype=np.float32)
    K = rng.standard_normal((Hkv, T, D), dtype=np.float32)
    V = rng.standard_normal((Hkv, T, D), dtype=np.float32)
    off = rng.standard_normal((Hkv, T // C), dtype=np.float32) * np.float32(offset_sd)
    out = {}
    if with_dO:
        out["dO"] = rng.standard_normal((Hq, n_q, D), dtype=np.float32)
    K += np.repeat(off, C, axis=1)[:, :, None]
    out.update(Q=Q, K=K, V=V, off=off)
    if bf16:
        for name in ("Q", "K", "V", "dO"):
            if name in out:
                out[name] = round_bf16(out[name])
    return out
