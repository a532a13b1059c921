"""The ranking scheduler's compare rule, restated on the CPU (host logic, no
GPU): a key (h, i) with h = ~orderable(S) and i the flat index is ranked by
32-bit compares only, entries of 64-entry blocks wholly below the ranked
key's block lowered by one, plus a tie count inside that block.  The rule
must give exactly the ranks of a 64-bit key sort (descending survival, then
ascending flat index) for every non-NaN survival, including ties, signed
zeros, infinities and subnormals."""
import numpy as np
import pytest


def orderable(s):
    b = s.astype(np.float32).view(np.uint32).copy()
    b[b == 0x80000000] = 0                        # -0 ranks with +0
    neg = (b & 0x80000000) != 0
    return np.where(neg, ~b, b | 0x80000000).astype(np.uint32)


def ranks_by_sort(S):
    n = S.size
    key = ((~orderable(S)).astype(np.uint64) << np.uint64(32)) | np.arange(n, dtype=np.uint64)
    r = np.empty(n, np.int64)
    r[np.argsort(key, kind="stable")] = np.arange(n)
    return r


def ranks_by_rule(S, K):
    n = S.size
    h = (~orderable(S)).astype(np.uint32)
    block = np.arange(n) // 64 * 64
    out = np.empty(n, np.int64)
    for g0 in range(0, n, K):
        c0 = g0 & ~63                              # the 64-entry block holding keys g0 .. g0 + K - 1
        hw = (h - (block + 64 <= c0).astype(np.uint32)).astype(np.uint32)
        lanes = np.arange(c0, min(c0 + 64, n))
        for x in range(g0, min(g0 + K, n)):
            out[x] = int(np.sum(hw < h[x])) + int(np.sum((h[lanes] == h[x]) & (lanes < x)))
    return out


def survivals(rng, n, kind):
    if kind == "random":
        return rng.random(n).astype(np.float32)
    if kind == "ties":
        return (rng.integers(0, 5, n) / 4).astype(np.float32)
    if kind == "zeros":
        s = np.zeros(n, np.float32)
        s[rng.random(n) < 0.3] = -0.0
        s[rng.random(n) < 0.2] = 1.0
        return s
    s = rng.standard_normal(n).astype(np.float32) * np.float32(1e30)   # outside [0, 1]: still exact
    s[rng.random(n) < 0.05] = np.inf
    s[rng.random(n) < 0.05] = -np.inf
    s[rng.random(n) < 0.05] = np.float32(1e-45)
    return s


@pytest.mark.parametrize("n,K", [(1, 16), (63, 16), (64, 16), (65, 16), (1000, 16), (4096, 16), (5000, 64)])
@pytest.mark.parametrize("kind", ["random", "ties", "zeros", "wide"])
def test_rule_equals_sort(n, K, kind):
    S = survivals(np.random.default_rng(n * 7 + K), n, kind)
    assert np.array_equal(ranks_by_rule(S, K), ranks_by_sort(S))
