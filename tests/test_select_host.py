"""The router's top-k threshold search on the CPU.

route_core.h's select_threshold is compiled for the host (hipcc, host code
only, no GPU needed) and run on key sets that a sort checks: the chosen set
(every key > T, then the lowest-positioned keys == T, k in all) must be the k
largest keys with ties to the lowest position (the routing rule: score
descending, then lower chunk id). Cases cover random keys, heavy ties, every
key equal (an all-zero query block scores every chunk 0), keys differing in
the top bit only, and candidate counts past the register selection's 2048.
"""
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "select_threshold_main.cpp")
CSRC = os.path.join(ROOT, "sparse_long_context_summarize_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("sel") / "select_threshold")
    subprocess.run([HIPCC, "-x", "hip", "--offload-host-only", "-O1", "-std=c++17",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, SRC, "-o", exe],
                   check=True, capture_output=True)
    return exe


def _run(exe, cases):
    text = "".join(f"{k} {len(keys)} " + " ".join(str(int(x)) for x in keys) + "\n"
                   for k, keys in cases)
    out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
    return [int(x) for x in out.split()]


def _chosen(keys, k, T):
    keys = np.asarray(keys, dtype=np.uint64)
    gt = np.nonzero(keys > T)[0]
    eq = np.nonzero(keys == T)[0]
    return sorted(gt.tolist() + eq[:k - len(gt)].tolist()) if len(gt) <= k else None


def _expected(keys, k):
    order = sorted(range(len(keys)), key=lambda i: (-int(keys[i]), i))
    return sorted(order[:k])


def _score_keys(scores):
    """The router's order-preserving uint32 key of fp32 scores (-0 as +0)."""
    u = np.asarray(scores, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u[u == 0x80000000] = 0
    neg = (u & 0x80000000) != 0
    return np.where(neg, (~u) & 0xFFFFFFFF, u | 0x80000000).astype(np.uint64)


def _cases():
    rng = np.random.default_rng(7)
    cases = []
    for n, k in ((550, 16), (2200, 16), (300, 299), (65, 1), (2049, 256), (5000, 32)):
        cases.append((k, [0xBF800000] * n))                               # every key equal
        cases.append((k, _score_keys(np.zeros(n, np.float32))))           # all-zero scores
        cases.append((k, _score_keys(rng.standard_normal(n).astype(np.float32))))
        few = rng.integers(0, 3, n)                                       # heavy ties
        cases.append((k, _score_keys(few.astype(np.float32))))
        two = np.where(rng.random(n) < 0.5, 0x80000000, 0x7FFFFFFF)       # top bit only
        cases.append((k, two))
        cases.append((k, rng.integers(0, 2**32, n, dtype=np.uint64)))
    # tiny exhaustive-ish: every k for small patterned rows
    for n in (2, 3, 5, 9):
        for k in range(1, n):
            cases.append((k, [5] * n))
            cases.append((k, list(range(n))))
            cases.append((k, list(range(n, 0, -1))))
            cases.append((k, [(i * 7) % 3 for i in range(n)]))
    return cases


def test_select_threshold_matches_sort(driver):
    cases = _cases()
    Ts = _run(driver, cases)
    assert len(Ts) == len(cases)
    for (k, keys), T in zip(cases, Ts):
        got = _chosen(keys, k, T)
        assert got is not None, f"more than k={k} keys above T={T:#x} (n={len(keys)})"
        assert len(got) == k, (k, len(keys), T, len(got))
        assert got == _expected(keys, k), (k, len(keys), T)
