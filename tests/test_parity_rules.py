"""The id parity rule itself (tests/parity.py), on hand-made score rows.

The rule lets GPU ids differ from the oracle's only by chunks whose oracle
score lies within 1e-4 * M of the k-th best score. These cases pin that the
rule reads each chunk's own score, also when a sink window keeps the first
chunks out of the candidates (gist.science technical summary 2.1: the sink
and local windows are attended beside the routed chunks, so the sink chunks
are never routing candidates).
"""
import numpy as np
import pytest

from parity import check_ids, check_group_ids


def _row(scores, n_cap):
    sig = np.full((1, 1, n_cap), np.nan)
    sig[0, 0, :len(scores)] = scores
    return sig


def test_sink_far_off_id_rejected():
    # block 0 starts at 512: chunks 0..7 closed; sink of 2 chunks -> candidates 2..7.
    # Chunks 4, 5, 6 tie at 5.0 (k = 1: the oracle takes the lowest, 4). A
    # checker that read the score of chunk c + 2 for chunk c would see 5.0 for
    # the GPU's chunk 3 (score 0.2) and accept it.
    p0 = 512
    scores = [9.0, 9.0, 0.1, 0.2, 5.0, 5.0, 5.0, 0.3]
    sig = _row(scores, 8)
    ref = np.array([[[4]]], dtype=np.int32)
    gpu = np.array([[[3]]], dtype=np.int32)      # score 0.2, far below 5.0
    with pytest.raises(AssertionError):
        check_ids(gpu, ref, sig, p0, sink_chunks=2)
    # a true tie partner is accepted
    assert check_ids(np.array([[[5]]], dtype=np.int32), ref, sig, p0, sink_chunks=2) == 1


def test_sink_near_tie_accepted():
    p0, k = 384, 1
    scores = [9.0, 9.0, 0.1, 5.0 - 1e-5, 5.0, 0.3]
    sig = _row(scores, 8)
    ref = np.array([[[4]]], dtype=np.int32)
    gpu = np.array([[[3]]], dtype=np.int32)      # within 1e-4 * 5.0 of the k-th score
    assert check_ids(gpu, ref, sig, p0, sink_chunks=2) == 1


def test_sink_id_inside_window_rejected():
    p0 = 384
    scores = [9.0, 9.0, 0.1, 0.2, 5.0, 0.3]
    sig = _row(scores, 8)
    ref = np.array([[[4]]], dtype=np.int32)
    gpu = np.array([[[1]]], dtype=np.int32)      # a sink chunk is no candidate
    with pytest.raises(AssertionError):
        check_ids(gpu, ref, sig, p0, sink_chunks=2)


def test_no_sink_rules():
    p0 = 256                                      # chunks 0..3 closed
    scores = [1.0, 3.0, 2.0, 2.0 + 5e-5]
    sig = _row(scores, 4)
    ref = np.array([[[1, 3]]], dtype=np.int32)
    assert check_ids(ref.copy(), ref, sig, p0) == 0
    assert check_ids(np.array([[[1, 2]]], dtype=np.int32), ref, sig, p0) == 1
    with pytest.raises(AssertionError):          # 1.0 is far from the k-th score
        check_ids(np.array([[[0, 1]]], dtype=np.int32), ref, sig, p0)
    with pytest.raises(AssertionError):          # order
        check_ids(np.array([[[3, 1]]], dtype=np.int32), ref, sig, p0)
    with pytest.raises(AssertionError):          # count
        check_ids(np.array([[[1, -1]]], dtype=np.int32), ref, sig, p0)


def test_group_rule_reads_absolute_ids():
    # one chunk (id 2) routed; its groups 16..23 are the candidates
    p0 = 192
    n_gcap = 24
    sig = np.full((1, 1, n_gcap), np.nan)
    sig[0, 0, 16:24] = [0.1, 0.2, 4.0, 0.3, 0.0, 0.5, 0.6, 0.7]
    chunk_ids = np.array([[[2]]], dtype=np.int32)
    ref = np.array([[[18]]], dtype=np.int32)
    assert check_group_ids(ref.copy(), ref, sig, chunk_ids, p0) == 0
    with pytest.raises(AssertionError):
        check_group_ids(np.array([[[17]]], dtype=np.int32), ref, sig, chunk_ids, p0)
