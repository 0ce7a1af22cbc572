"""The dQ kernel's acceptance rule for the Delta estimate, checked on the CPU.

The backward's dQ pass forms dS = P (dP - D) with D_i = dO_i . O_i taken from
the forward's bf16 output, while it sums the exact Delta_i = sum_j P_ij dP_ij
and M_i = sum_j P_ij |dP_ij - D_i|; a row keeps that dQ when
|Delta_i - D_i| <= 2^-8 M_i (bf16's unit roundoff), else it is recomputed with
Delta (the segment-wise backward of gist.science technical summary 2.2; the
softmax gradient dS = P (dP - Delta) is the standard one). Written out here in
fp64 with the forward's roundings emulated (P and O rounded to bf16):

* the one-pass dQ differs from the exact one by exactly
  +scale (Delta_i - D_i) sum_j P_ij K_j, so an accepted row moves by at most
  2^-8 M_i max_j |K_j| scale -- the identity and the bound;
* rows whose attention is spread over many keys (the 16K workload's kind) are
  all accepted, with margin;
* rows whose attention sits on one or two keys are mostly rejected; those
  let through stay within half the parity bar, and the row the estimate
  would have moved most is among the rejected.
"""
import numpy as np
import torch

TOL = 2.0 ** -8
ATOL, RTOL = 1e-2, 2e-2          # the elementwise bar of the GPU parity tests


def bf16(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(
        torch.bfloat16).double().numpy()


def rows(seed: int, n: int = 64, keys: int = 1024, d: int = 128, q_gain: float = 1.0):
    rng = np.random.default_rng(seed)
    q = bf16(rng.standard_normal((n, d)) * q_gain)
    k = bf16(rng.standard_normal((keys, d)))
    v = bf16(rng.standard_normal((keys, d)))
    do = bf16(rng.standard_normal((n, d)))
    scale = 1.0 / np.sqrt(d)
    s = scale * q @ k.T
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    o = bf16(bf16(p) @ v)                       # bf16 probabilities, bf16 output
    dp = do @ v.T
    delta = (p * dp).sum(1)                     # exact
    est = (do * o).sum(1)                       # the estimate from O
    m = (p * np.abs(dp - est[:, None])).sum(1)
    dq_fast = scale * (p * (dp - est[:, None])) @ k
    dq_exact = scale * (p * (dp - delta[:, None])) @ k
    return dict(k=k, p=p, scale=scale, delta=delta, est=est, m=m, dq_fast=dq_fast,
                dq_exact=dq_exact)


def test_identity_and_bound():
    for gain in (1.0, 16.0):
        r = rows(11, q_gain=gain)
        err = r["delta"] - r["est"]
        shift = r["scale"] * err[:, None] * (r["p"] @ r["k"])
        np.testing.assert_allclose(r["dq_fast"] - r["dq_exact"], shift, rtol=1e-9, atol=1e-12)
        ok = np.abs(err) <= TOL * r["m"]
        bound = TOL * r["m"] * np.abs(r["k"]).max() * r["scale"]
        moved = np.abs(r["dq_fast"] - r["dq_exact"]).max(1)
        assert np.all(moved[ok] <= bound[ok] * (1 + 1e-12))


def test_spread_rows_keep_the_first_pass():
    for seed in (12, 13, 14):
        r = rows(seed)
        ratio = np.abs(r["delta"] - r["est"]) / r["m"]
        assert ratio.max() <= TOL / 2, ratio.max()
        # and the one-pass dQ sits far inside the parity bar
        lim = ATOL + RTOL * np.abs(r["dq_exact"])
        assert np.all(np.abs(r["dq_fast"] - r["dq_exact"]) <= 0.1 * lim)


def test_peaked_rows_take_the_second_pass():
    r = rows(15, q_gain=16.0)
    err = np.abs(r["delta"] - r["est"])
    ok = err <= TOL * r["m"]
    assert np.median(r["p"].max(1)) > 0.9          # attention sits on one or two keys
    assert (~ok).sum() >= len(ok) // 2
    lim = ATOL + RTOL * np.abs(r["dq_exact"])
    frac = (np.abs(r["dq_fast"] - r["dq_exact"]) / lim).max(1)
    # what the rule lets through stays within half the parity bar, and the
    # row the estimate would have moved most is sent back
    assert frac[ok].max(initial=0.0) <= 0.5
    assert not ok[np.argmax(frac)]
