"""Pins for the oracle's prefix-match verify step (CPU only)."""
import numpy as np

from oracle import dspark_oracle as orc


def brute_force(tokens, target, lens):
    """Largest a <= lens with tokens[:a] == target[:a], searched from the top."""
    out_a, out_bonus = [], []
    for b in range(tokens.shape[0]):
        for a in range(int(lens[b]), -1, -1):
            if all(tokens[b, j] == target[b, j] for j in range(a)):
                break
        out_a.append(a)
        out_bonus.append(target[b, a])
    return np.array(out_a), np.array(out_bonus)


def test_verify_matches_brute_force_random():
    rng = np.random.default_rng(5)
    for _ in range(50):
        B, g = int(rng.integers(1, 40)), int(rng.integers(1, 17))
        V = int(rng.integers(2, 5))            # tiny vocab: many matches
        tokens = rng.integers(0, V, size=(B, g)).astype(np.int32)
        target = rng.integers(0, V, size=(B, g + 1)).astype(np.int32)
        lens = rng.integers(0, g + 1, size=B).astype(np.int32)
        a, bonus = orc.verify(tokens, target, lens)
        a2, bonus2 = brute_force(tokens, target, lens)
        np.testing.assert_array_equal(a, a2)
        np.testing.assert_array_equal(bonus, bonus2)


def test_verify_special_cases():
    tokens = np.array([[1, 2, 3, 4], [1, 2, 3, 4], [9, 9, 9, 9]], dtype=np.int32)
    target = np.array([[1, 2, 3, 4, 5], [1, 2, 3, 4, 5], [1, 2, 3, 4, 5]], dtype=np.int32)
    # lens = 0: nothing verified, bonus is the target's first token
    a, bonus = orc.verify(tokens, target, np.array([0, 4, 4], dtype=np.int32))
    assert list(a) == [0, 4, 0]
    assert list(bonus) == [1, 5, 1]
    # full match up to a shorter schedule: bonus is the next target token
    a, bonus = orc.verify(tokens, target, np.array([2, 3, 1], dtype=np.int32))
    assert list(a) == [2, 3, 0] and list(bonus) == [3, 4, 1]
    # a match after a mismatch does not count
    tk = np.array([[1, 7, 3, 4]], dtype=np.int32)
    a, bonus = orc.verify(tk, target[:1], np.array([4], dtype=np.int32))
    assert a[0] == 1 and bonus[0] == 2
