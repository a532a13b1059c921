"""Pins of the sequential-temperature-scaling oracle (fitting T_1..T_gamma
left to right by a grid search on the expected calibration error) against
things other than itself: a hand-worked calibration error, scikit-learn's
reliability curve, recovery of the temperatures of a known acceptance
process, closed forms for all-accepted and all-rejected data, the tie rule,
and exact invariances."""
import numpy as np
import pytest
from scipy.special import expit
from sklearn.calibration import calibration_curve

from oracle import dspark_oracle as orc
from semi_ar_drafter_amd import workloads as wl


def sklearn_ece(p, y, n_bins):
    """ECE from scikit-learn's uniform-bin reliability curve: the bin weights
    are the bin populations over the same edges."""
    prob_true, prob_pred = calibration_curve(y, p, n_bins=n_bins, strategy="uniform")
    edges = np.linspace(0.0, 1.0, n_bins + 1)
    counts = np.bincount(np.searchsorted(edges[1:-1], p), minlength=n_bins)
    counts = counts[counts > 0]
    return float(np.sum(counts / len(p) * np.abs(prob_true - prob_pred)))


def test_ece_hand_worked_example():
    # ten bins: 0.05 -> bin 0; 0.15, 0.12 -> bin 1; 0.55, 0.58 -> bin 5; 0.95 -> bin 9
    p = np.array([0.05, 0.15, 0.12, 0.95, 0.55, 0.58])
    y = np.array([0, 1, 0, 1, 1, 0])
    # bin gaps |sum(y - p)|: 0.05, |1 - 0.27| = 0.73, |1 - 1.13| = 0.13, 0.05 -> 0.96 / 6
    E, e = orc.ece_fixed(p, y, 10)
    assert abs(e - 0.16) < 1e-9
    # one bin: |sum y - sum p| / N = |3 - 2.40| / 6
    E1, e1 = orc.ece_fixed(p, y, 1)
    assert abs(e1 - 0.1) < 1e-9
    assert abs(int(E1) - 0.6 * 2 ** 32) <= 3     # six residuals, each rounded by <= 1/2


@pytest.mark.parametrize("n_bins", [1, 7, 15, 64])
def test_ece_agrees_with_sklearn_reliability_curve(n_bins):
    rng = np.random.default_rng(7 + n_bins)
    p = rng.random(5000) ** 2
    p[:7] = 1.0                                  # the top edge belongs to the last bin
    p[7:11] = 0.0
    y = (rng.random(5000) < np.clip(p * 1.2, 0, 1)).astype(np.int64)
    _, e = orc.ece_fixed(p, y, n_bins)
    assert abs(float(e) - sklearn_ece(p, y, n_bins)) < 1e-9
    # batched rows agree with one row at a time
    P = np.stack([p, p[::-1], np.sqrt(p)])
    E, eb = orc.ece_fixed(P, y, n_bins)
    for i in range(3):
        assert E[i] == orc.ece_fixed(P[i], y, n_bins)[0]
        assert abs(eb[i] - sklearn_ece(P[i], y, n_bins)) < 1e-9


def test_recovers_the_temperatures_of_the_acceptance_process():
    cfg = wl.STSConfig(210, "sts-recovery", 200000, 4, 128, 15, t_true=(1.4, 2.6))
    w = wl.make_sts_calibration(cfg)
    choice, T, ece = orc.sts_fit(w["logit"], w["accepted"], w["grid"], w["n_bins"])
    assert np.all(np.abs(T / w["t_true"] - 1.0) < 0.06), (T, w["t_true"])
    assert np.array_equal(T, w["grid"][choice])
    assert np.array_equal(ece[np.arange(4), choice], ece.min(axis=1))
    # an underconfident head (t_true < 1) is recovered too
    cfg2 = cfg.replace(cid=211, t_true=(0.6, 0.8))
    w2 = wl.make_sts_calibration(cfg2)
    _, T2, _ = orc.sts_fit(w2["logit"], w2["accepted"], w2["grid"], w2["n_bins"])
    assert np.all(np.abs(T2 / w2["t_true"] - 1.0) < 0.06), (T2, w2["t_true"])


def test_each_position_is_the_grid_argmin_of_sklearn_ece():
    w = wl.make_sts_calibration(wl.STS_WORKLOADS[0])
    L, a, grid, M = w["logit"].astype(np.float64), w["accepted"], w["grid"], w["n_bins"]
    choice, T, ece = orc.sts_fit(L.astype(np.float32), a, grid, M)
    prefix = np.ones(L.shape[0])
    for k in range(L.shape[1]):
        y = (a >= k + 1).astype(np.int64)
        ref = np.array([sklearn_ece(prefix * expit(L[:, k] / float(t)), y, M) for t in grid])
        assert np.max(np.abs(ref - ece[k])) < 1e-9
        order = np.sort(ref)
        assert order[1] - order[0] > 1e-8            # no near tie in this data
        assert choice[k] == int(np.argmin(ref))
        prefix = prefix * expit(L[:, k] / float(grid[choice[k]]))


def test_all_accepted_or_all_rejected_closed_forms():
    rng = np.random.default_rng(3)
    L = (np.abs(rng.standard_normal((500, 5))) + 0.1).astype(np.float32)   # positive logits
    grid = np.array([1.0, 0.5, 4.0, 2.0, 0.25, 8.0], dtype=np.float32)
    # every block fully accepted: ECE = mean(1 - p), smallest at the smallest T
    c, T, _ = orc.sts_fit(L, np.full(500, 5), grid, 10)
    assert np.all(T == 0.25) and np.all(c == 4)
    # every block rejected at once: ECE = mean(p), smallest at the largest T
    c, T, _ = orc.sts_fit(L, np.zeros(500, dtype=np.int32), grid, 10)
    assert np.all(T == 8.0) and np.all(c == 5)


def test_ties_resolved_to_the_first_entry_at_every_position():
    w = wl.make_sts_calibration(wl.STS_WORKLOADS[0])
    grid = np.repeat(w["grid"], 2)                # every candidate twice
    c, T, e = orc.sts_fit(w["logit"], w["accepted"], grid, w["n_bins"])
    assert np.all(c % 2 == 0)
    assert np.array_equal(e[:, 0::2], e[:, 1::2])
    c1, T1, _ = orc.sts_fit(w["logit"], w["accepted"], w["grid"], w["n_bins"])
    assert np.array_equal(c, 2 * c1) and np.array_equal(T, T1)


def test_invariant_under_scaling_logits_and_grid_by_two():
    w = wl.make_sts_calibration(wl.STS_WORKLOADS[0])
    c, T, e = orc.sts_fit(w["logit"], w["accepted"], w["grid"], w["n_bins"])
    c2, T2, e2 = orc.sts_fit(w["logit"] * np.float32(2), w["accepted"], w["grid"] * np.float32(2), w["n_bins"])
    assert np.array_equal(c, c2) and np.array_equal(T * 2, T2) and np.array_equal(e, e2)


def test_invariant_under_permuting_blocks():
    w = wl.make_sts_calibration(wl.STS_WORKLOADS[0])
    perm = np.random.default_rng(5).permutation(w["logit"].shape[0])
    c, T, e = orc.sts_fit(w["logit"], w["accepted"], w["grid"], w["n_bins"])
    cp, Tp, ep = orc.sts_fit(w["logit"][perm], w["accepted"][perm], w["grid"], w["n_bins"])
    assert np.array_equal(c, cp) and np.array_equal(e, ep)


def test_no_blocks():
    grid = np.array([2.0, 1.0, 3.0], dtype=np.float32)
    c, T, e = orc.sts_fit(np.zeros((0, 3), dtype=np.float32), np.zeros(0, dtype=np.int32), grid, 15)
    assert np.all(c == 0) and np.all(T == 2.0) and np.all(e == 0.0)


def test_accepted_counts_saturate_at_both_ends():
    w = wl.make_sts_calibration(wl.STS_WORKLOADS[0])
    a = w["accepted"].copy()
    gamma = w["logit"].shape[1]
    a2 = a.copy()
    a2[a == gamma] = gamma + 7
    a2[a == 0] = -3
    r1 = orc.sts_fit(w["logit"], a, w["grid"], w["n_bins"])
    r2 = orc.sts_fit(w["logit"], a2, w["grid"], w["n_bins"])
    for x, y in zip(r1, r2):
        assert np.array_equal(x, y)
