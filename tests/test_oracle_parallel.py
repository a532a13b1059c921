"""Pins of the parallel-only drafting oracle (drafting without the
sequential head) against things other than itself: the Markov-head oracle
with a zero transition matrix, textbook argmax on hand-made rows with ties,
and the Gumbel-max property (sampling frequencies follow softmax)."""
import numpy as np

from oracle import dspark_oracle as orc
from semi_ar_drafter_amd import workloads as wl


def test_equals_markov_draft_with_zero_transition():
    for sampling in ("greedy", "gumbel"):
        cfg = wl.small_config(B=6, gamma=4, V=300, r=32, d=8, dtype="bf16", sampling=sampling)
        w = wl.make_workload(cfg)
        W2 = np.zeros_like(w["W2"])
        t_m, z_m, _, _ = orc.draft(w["anchor"], w["U"], w["h"], w["W1"], W2, w["conf_w"], w["conf_b"],
                                   w["sts_T"], sampling=sampling, seed=12345)
        t_p, z_p = orc.parallel_draft(w["U"], sampling=sampling, seed=12345)
        assert np.array_equal(t_m, t_p) and np.array_equal(z_m, z_p)


def test_lowest_index_among_equal_maxima_and_rows_subset():
    U = np.zeros((2, 3, 6), dtype=np.float32)
    U[0, 0] = [1, 5, 2, 5, 5, 0]        # ties at 1, 3, 4 -> 1
    U[0, 1] = [-3, -1, -2, -1, -9, -4]  # ties at 1, 3 -> 1
    U[0, 2] = [0, 0, 0, 0, 0, 0]        # all equal -> 0
    U[1, 0] = [7, 1, 1, 1, 1, 7.5]      # -> 5
    U[1, 1] = [2, 2, 3, 3, 3, 3]        # -> 2
    U[1, 2] = [-0.0, 0.0, -1, -1, -1, -1]  # -0 == +0 -> 0
    t, z = orc.parallel_draft(U)
    assert t.tolist() == [[1, 1, 0], [5, 2, 0]]
    assert z.tolist() == [[5, -1, 0], [7.5, 3, 0]]
    t1, z1 = orc.parallel_draft(U, rows=[1])
    assert t1.tolist() == [[5, 2, 0]]


def test_bf16_storage_is_decoded_exactly():
    vals = np.array([[[1.5, -2.25, 3.0, 2.9921875]]], dtype=np.float32)   # all exact in bf16
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    t, z = orc.parallel_draft(bits)
    assert t.tolist() == [[2]] and z.tolist() == [[3.0]]


def test_gumbel_max_samples_from_softmax():
    """Argmax of z + Gumbel noise is a draw from softmax(z): over many seeds the
    token frequencies match the probabilities (each within 4 standard errors)."""
    p = np.array([0.1, 0.2, 0.3, 0.4])
    z = np.log(p).astype(np.float32)
    U = np.broadcast_to(z, (1, 1, 4)).copy()
    n = 3000
    counts = np.zeros(4)
    for s in range(n):
        t, _ = orc.parallel_draft(U, sampling="gumbel", seed=0x9E3779B97F4A7C15 ^ (s * 0x100000001))
        counts[t[0, 0]] += 1
    freq = counts / n
    se = np.sqrt(p * (1 - p) / n)
    assert np.all(np.abs(freq - p) < 4 * se), (freq, p)
