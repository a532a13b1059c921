"""Pins for the oracle's hardware-aware prefix scheduler (CPU only).

The oracle ranks gains and scans the top-M prefix sums.  It is checked
against exhaustive enumeration of every allocation l in {0..gamma}^B with
exact rational arithmetic, and against closed-form special cases.
"""
import itertools
import zlib
from fractions import Fraction

import numpy as np
import pytest

from oracle import dspark_oracle as orc

TWO32 = 2 ** 32


def _gain(s):
    # fixed point of one fp32 survival value (ties to even), as an exact integer
    return int(np.rint(np.float64(np.float32(s)) * TWO32))


def brute_force(surv, t_step, n_min):
    """Enumerate every allocation; objective (B*2^32 + sum of gains) / t exact."""
    B, g = surv.shape
    best = None
    for l in itertools.product(range(g + 1), repeat=B):
        M = sum(l)
        idx = B + M - n_min
        if idx >= len(t_step):
            continue
        num = B * TWO32 + sum(_gain(surv[i, k]) for i in range(B) for k in range(l[i]))
        phi = Fraction(num) / Fraction(float(t_step[idx]))
        key = (phi, -M)
        if best is None or key > best[0]:
            best = (key, [l])
        elif key == best[0]:
            best[1].append(l)
    (phi, negM), allocs = best
    return phi, -negM, allocs


def _monotone_surv(rng, B, g, mode):
    if mode == "random":
        c = rng.random((B, g)).astype(np.float32)
    elif mode == "ones":
        c = np.where(rng.random((B, g)) < 0.5, 1.0, rng.random((B, g))).astype(np.float32)
    elif mode == "ties":
        vals = np.array([1.0, 0.5, 0.25, 0.0], dtype=np.float32)
        c = vals[rng.integers(0, 4, size=(B, g))]
    elif mode == "zeros":
        c = rng.random((B, g)).astype(np.float32)
        c[:, g // 2:] = 0.0
    else:
        raise ValueError(mode)
    S = np.empty((B, g), dtype=np.float32)
    acc = np.ones(B, dtype=np.float32)
    for k in range(g):
        acc = (acc * c[:, k]).astype(np.float32)
        S[:, k] = acc
    return S


def _table(rng, B, g, kind):
    n = np.arange(B, B + B * g + 1, dtype=np.float64)
    if kind == "linear":
        return 1.0 + rng.uniform(0.001, 0.5) * n
    if kind == "quad":
        return 4.0 + 0.02 * n + rng.uniform(1e-4, 0.3) * n * n
    if kind == "flat":
        return np.full(n.size, 3.0)
    if kind == "step":   # piecewise, includes exact plateaus
        return 1.0 + np.floor(n / 3.0)
    raise ValueError(kind)


@pytest.mark.parametrize("mode", ["random", "ones", "ties", "zeros"])
@pytest.mark.parametrize("kind", ["linear", "quad", "flat", "step"])
def test_scheduler_matches_brute_force(mode, kind):
    rng = np.random.default_rng(zlib.crc32(f"{mode}/{kind}".encode()))
    for trial in range(12):
        B = int(rng.integers(1, 5))
        g = int(rng.integers(1, 5))
        if (g + 1) ** B > 700:
            g = 2
        S = _monotone_surv(rng, B, g, mode)
        t = _table(rng, B, g, kind)
        lens, m_star, obj = orc.schedule(S, t, B)
        phi, m_bf, allocs = brute_force(S, t, B)
        assert m_star == m_bf
        assert int(lens.sum()) == m_star
        assert tuple(int(x) for x in lens) in allocs
        assert obj * TWO32 == float(phi)          # one correctly rounded division


def test_scheduler_tie_order_prefers_lower_request():
    S = np.array([[0.5, 0.5], [0.5, 0.5]], dtype=np.float32)
    n = np.arange(2, 7, dtype=np.float64)
    # make exactly M = 3 optimal: cost jumps sharply after n = 5
    t = np.where(n <= 5, 1.0, 1e9)
    lens, m, _ = orc.schedule(S, t, 2)
    assert m == 3
    assert list(lens) == [2, 1]


def test_flat_table_takes_every_positive_gain():
    rng = np.random.default_rng(3)
    S = _monotone_surv(rng, 6, 5, "zeros")
    t = np.full(6 * 5 + 1, 2.5)
    lens, m, obj = orc.schedule(S, t, 6)
    gains = np.rint(S.astype(np.float64) * TWO32)
    assert m == int((gains > 0).sum())
    np.testing.assert_array_equal(lens, (gains > 0).sum(axis=1))


def test_steep_table_schedules_nothing():
    S = np.full((5, 4), 0.99, dtype=np.float32)
    t = 1.0 * 1e6 ** np.arange(21, dtype=np.float64) / 1e100
    t[0] = 1.0
    t[1:] = 1e12
    lens, m, obj = orc.schedule(S, t, 5)
    assert m == 0 and (lens == 0).all() and obj == 5.0


def test_linear_table_threshold_rule():
    """With t(n) = a + b n, at the optimum a token is scheduled iff its gain
    exceeds b * Phi* (marginal analysis of a ratio objective)."""
    rng = np.random.default_rng(11)
    for _ in range(20):
        B, g = 16, 8
        S = _monotone_surv(rng, B, g, "random")
        a, bb = 1.0, float(rng.uniform(0.001, 0.2))
        n = np.arange(B, B + B * g + 1, dtype=np.float64)
        lens, m, obj = orc.schedule(S, a + bb * n, B)
        gains = np.rint(S.astype(np.float64) * TWO32) / TWO32
        taken = np.arange(g)[None, :] < lens[:, None]
        thr = bb * obj
        assert (gains[taken] >= thr - 1e-9).all()
        assert (gains[~taken] <= thr + 1e-9).all()


def test_m_range_limited_by_table():
    S = np.full((4, 4), 0.9, dtype=np.float32)
    t = np.full(4 + 1, 1.0)            # covers n = 4..8 only: M <= 4
    lens, m, _ = orc.schedule(S, t, 4)
    assert m == 4 and list(lens) == [4, 0, 0, 0]
    with pytest.raises(ValueError):
        orc.schedule(S, t, 5)          # n_min > B
