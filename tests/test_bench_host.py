"""Host-side logic of bench.py: the algorithmic flop and byte counts that its
roofline figures divide by kernel time, and the one-GPU guard. Counts are
checked against pairs enumerated one by one on tiny id rows."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _pairs(ids, p0, unit, C=64):
    """(query, key) pairs one kv head's G heads attend, by enumeration."""
    Hkv, nb, _ = ids.shape
    n = 0
    for g in range(Hkv):
        for b in range(nb):
            P = p0 + b * C
            keys = set()
            for u in ids[g, b]:
                if 0 <= u < P // unit:
                    keys.update(range(u * unit, (u + 1) * unit))
            for i in range(C):
                n += len(keys) + (i + 1)          # routed keys + causal local keys
    return n


@pytest.mark.parametrize("unit", [64, 8])
def test_attend_counts_match_enumeration(unit):
    rng = np.random.default_rng(unit)
    p0, nb, k, G, D = 512, 3, 6, 4, 128
    ids = rng.integers(-3, (p0 + nb * 64) // unit + 4, (2, nb, k)).astype(np.int32)
    ids[0, 1, :3] = ids[0, 1, 3]                   # repeats count once
    fl = bench.attend_flops(ids, nb * 64, G, D, p0, unit=unit)
    assert fl == 4.0 * D * G * _pairs(ids, p0, unit)
    by = bench.attend_bytes(ids, nb * 64, 2 * G, D, p0, unit=unit)
    n_keys = _pairs(ids, p0, unit) - 2 * nb * (64 * 65 // 2)
    gathered = (n_keys // 64 + 2 * nb * 64) * D * 2 * 2   # routed keys per block + local
    assert by == gathered + 2 * G * nb * 64 * D * 4 + 2 * G * nb * 64 * 4


def test_bwd_counts_split_history_and_active():
    # p0 = 128: chunks 0, 1 are history (S, dP, dQ: 6D per pair), chunk 2 and
    # the local blocks are active (also dK, dV: 10D per pair)
    ids = np.array([[[0, 2, 2, -1], [1, 0, 9, 2]]], np.int32)
    G, D = 2, 128
    fl = bench.bwd_flops(ids, 128, G, D, 128)
    # block 0 (P/C = 2): {0}, chunk 2 is its own local chunk and is skipped;
    # block 1 (P/C = 3): {0, 1} history and chunk 2 active
    hist = (1 + 2) * 64 * 64
    act = 1 * 64 * 64 + 2 * (64 * 65 // 2)
    assert fl == G * (6 * D * hist + 10 * D * act)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_bwd_counts_for_groups():
    # p0 = 128: groups 0..15 are history, 16.. active; block 1 (P = 192) may
    # use groups < 24, block 0 (P = 128) groups < 16
    ids = np.array([[[3, 3, 15, 16, -1], [0, 17, 23, 24, 17]]], np.int32)
    G, D, U = 2, 128, 8
    fl = bench.bwd_flops(ids, 128, G, D, 128, unit=U)
    hist = (2 + 1) * U * 64            # block 0: {3, 15}; block 1: {0}
    act = 2 * U * 64 + 2 * (64 * 65 // 2)   # block 1: {17, 23}; both local blocks
    assert fl == G * (6 * D * hist + 10 * D * act)
