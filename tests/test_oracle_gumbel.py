"""Pins for the oracle's counter-based hash and Gumbel-max sampling (CPU only).

* Philox4x32-10 against the published known-answer vectors.
* The uniform derived from the hash is uniform (chi-square).
* Gumbel-max over z + G samples from softmax(z) (chi-square), also through
  the full draft function (which exercises the seed / request / position /
  vocabulary-id plumbing).
"""
import os

import numpy as np
from scipy import stats

from oracle import dspark_oracle as orc
from semi_ar_drafter_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def test_philox_known_answer_vectors():
    n = 0
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        f = [int(x, 16) for x in line.split()]
        out = orc.philox4x32_10(f[0], f[1], f[2], f[3], f[4], f[5])
        assert [int(x) for x in out] == f[6:10]
        n += 1
    assert n == 3


def test_hash_word_uses_counter_layout():
    # v and v ^ 1 share a Philox block (same counter, other output word)
    seed, b, k = 0x1234ABCD5678, 3, 7
    v = np.arange(64)
    w = orc.gumbel_uniform_bits(seed, b, k, v)
    for base in range(0, 64, 4):
        blk = orc.philox4x32_10(base >> 2, k, b, 0, seed & 0xFFFFFFFF, seed >> 32)
        assert [int(x) for x in w[base:base + 4]] == [int(x) for x in blk]


def test_uniform_is_uniform_chi_square():
    v = np.arange(1 << 18)
    w = orc.gumbel_uniform_bits(99, 0, 1, v).astype(np.float64)
    u = (np.floor(w / 512) * 2 + 1) * 2.0 ** -24
    assert u.min() > 0 and u.max() < 1
    hist, _ = np.histogram(u, bins=1024, range=(0, 1))
    p = stats.chisquare(hist).pvalue
    assert p > 1e-4


def test_gumbel_max_samples_softmax():
    z = np.array([0.0, 1.0, -0.5, 2.0, 0.3, -2.0, 1.5, 0.9], dtype=np.float32)
    V = z.size
    n = 60_000
    seeds = np.arange(n, dtype=np.int64)
    counts = np.zeros(V, dtype=np.int64)
    for s0 in range(0, n, 2000):
        for seed in seeds[s0:s0 + 2000]:
            g = orc.gumbel_noise(int(seed), 0, 1, np.arange(V))
            counts[np.argmax(z + g)] += 1
    p = np.exp(z.astype(np.float64) - z.max())
    p /= p.sum()
    assert stats.chisquare(counts, p * n).pvalue > 1e-4


def test_gumbel_draft_samples_softmax_of_logits():
    """Through `draft`: with W2 = 0 the step-1 distribution is softmax(U_1)."""
    cfg = wl.small_config(B=1, gamma=1, V=8, r=16, d=4, dtype="f32", sampling="gumbel")
    w = wl.make_workload(cfg)
    w["W2"] = np.zeros_like(w["W2"])
    U = w["U"].copy()
    U[0, 0] = np.array([0.5, -1.0, 1.2, 0.0, 2.0, -0.3, 0.7, 1.9], dtype=np.float32)
    w["U"] = U
    n = 20_000
    counts = np.zeros(8, dtype=np.int64)
    for seed in range(n):
        t, _, _, _ = orc.draft_workload(w, seed=seed)
        counts[t[0, 0]] += 1
    p = np.exp(U[0, 0].astype(np.float64))
    p /= p.sum()
    assert stats.chisquare(counts, p * n).pvalue > 1e-4


def test_noise_differs_across_request_and_position():
    v = np.arange(4096)
    a = orc.gumbel_noise(5, 0, 1, v).astype(np.float64)
    b = orc.gumbel_noise(5, 1, 1, v).astype(np.float64)
    c = orc.gumbel_noise(5, 0, 2, v).astype(np.float64)
    d = orc.gumbel_noise(6, 0, 1, v).astype(np.float64)
    for other in (b, c, d):
        assert abs(np.corrcoef(a, other)[0, 1]) < 0.08
    # Gumbel(0, 1): mean = Euler-Mascheroni constant, variance = pi^2 / 6
    allg = np.concatenate([a, b, c, d])
    assert abs(allg.mean() - 0.5772156649) < 0.05
    assert abs(allg.var() - np.pi ** 2 / 6) < 0.1
