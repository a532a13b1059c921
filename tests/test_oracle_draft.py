"""Pins for the oracle's Markov-head draft (CPU only).

Each test checks the oracle against something other than its own code: the
explicit V x V transition matrix, numpy's first-occurrence argmax, scipy's
logistic function on an independently assembled dot product, the survival
process simulated by Monte Carlo, and closed-form special cases.
"""
import math

import numpy as np
import pytest
from scipy.special import expit

from oracle import dspark_oracle as orc
from semi_ar_drafter_amd import workloads as wl


def _small(dtype="f32", **kw):
    base = dict(B=3, gamma=5, V=300, r=16, d=40, dtype=dtype)
    base.update(kw)
    return wl.make_workload(wl.small_config(**base))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lowrank_bias_equals_explicit_transition_matrix(dtype):
    """B = W1 W2 is a V x V matrix; the bias at step k is row x_{k-1} of it."""
    w = wl.make_workload(wl.WORKLOADS[0]) if dtype == "f32" else _small("bf16", V=512, r=32)
    trace = []
    tokens, zsel, conf, surv = orc.draft_workload(w, trace=trace)
    W1 = orc.widen(w["W1"])
    W2 = orc.widen(w["W2"])
    Bmat = W1 @ W2                                  # full V x V transition
    U = orc.widen(w["U"])
    for st in trace:
        k = st["k"]
        prev = w["anchor"] if k == 1 else tokens[:, k - 2]
        np.testing.assert_array_equal(st["x_prev"], prev)
        expect = U[:, k - 1, :] + Bmat[prev, :]
        np.testing.assert_allclose(st["z64"], expect, rtol=0, atol=1e-10)
        # one entry by a plain Python sum over the rank dimension
        b, v = 0, 7
        s = math.fsum(W1[prev[b], j] * W2[j, v] for j in range(W1.shape[1]))
        assert abs(st["z64"][b, v] - (U[b, k - 1, v] + s)) < 1e-12


def test_argmax_is_numpy_first_occurrence_on_fp32_logits():
    w = wl.make_workload(wl.WORKLOADS[0])
    trace = []
    tokens, zsel, _, _ = orc.draft_workload(w, trace=trace)
    for st in trace:
        z32 = st["z64"].astype(np.float32)
        for b in range(z32.shape[0]):
            assert tokens[b, st["k"] - 1] == int(np.argmax(z32[b]))
            assert zsel[b, st["k"] - 1] == z32[b].max()


def test_argmax_ties_pick_lowest_index():
    """Exact ties: with W2 = 0 the logits are U; plant equal maxima."""
    w = _small("f32", B=2, gamma=2, V=64)
    w["W2"] = np.zeros_like(w["W2"])
    U = w["U"].copy()
    U[:] = -1.0
    U[0, 0, [5, 9, 40]] = 3.0
    U[1, 0, [63, 2]] = 3.0
    U[:, 1, 11] = 2.0
    w["U"] = U
    tokens, zsel, _, _ = orc.draft_workload(w)
    assert tokens[0, 0] == 5 and tokens[1, 0] == 2
    assert (tokens[:, 1] == 11).all()
    assert zsel[0, 0] == 3.0


def test_strong_plant_is_always_drafted():
    """Special case: a plant far above the noise is the argmax at every step.
    Catches an off-by-one between position k and U's slice."""
    cfg = wl.small_config(B=4, gamma=6, V=700, r=16, d=24, dtype="bf16", plant=(200.0, 200.0))
    w = wl.make_workload(cfg)
    tokens, _, _, _ = orc.draft_workload(w)
    np.testing.assert_array_equal(tokens, w["plant"])


def test_anchor_feeds_first_gather_only():
    """Changing the anchor changes step 1's bias and nothing that does not
    depend on it: with W2 = 0 the tokens must not move."""
    w = _small("f32")
    w2 = dict(w)
    w2["anchor"] = (w["anchor"] + 1) % w["cfg"].V
    w2["W2"] = np.zeros_like(w["W2"])
    w3 = dict(w2)
    w3["anchor"] = w["anchor"]
    t2, _, c2, _ = orc.draft_workload(w2)
    t3, _, c3, _ = orc.draft_workload(w3)
    np.testing.assert_array_equal(t2, t3)
    # the confidence uses the previous token's embedding: position 1 changes
    assert not np.allclose(c2[:, 0], c3[:, 0])
    np.testing.assert_array_equal(c2[:, 1:], c3[:, 1:])


def test_confidence_is_sigmoid_of_concatenated_linear_head_at_T1():
    """STS with T = 1 reproduces the raw sigmoid of w . [h_k ; W1[x_{k-1}]] + b."""
    w = _small("bf16", B=3, gamma=4, V=400, r=32, d=48)
    w["sts_T"] = np.ones_like(w["sts_T"])
    tokens, _, conf, surv = orc.draft_workload(w)
    H = orc.widen(w["h"])
    W1 = orc.widen(w["W1"])
    wv = w["conf_w"].astype(np.float64)
    for b in range(3):
        for k in range(1, 5):
            prev = w["anchor"][b] if k == 1 else tokens[b, k - 2]
            vec = np.concatenate([H[b, k - 1], W1[prev]])
            ell = math.fsum(vec * wv) + w["conf_b"]
            ref = np.float32(expit(ell))
            assert abs(float(conf[b, k - 1]) - float(ref)) <= 1e-7 * max(1.0, abs(float(ref)))


def test_sts_temperature_scaling_properties():
    w = _small("f32", B=2, gamma=3, V=128, r=16, d=8)
    ells = []
    _, _, c1, _ = orc.draft_workload(dict(w, sts_T=np.ones(3, np.float32)))
    for T in (2.0, 7.5):
        _, _, cT, _ = orc.draft_workload(dict(w, sts_T=np.full(3, T, np.float32)))
        # logit(c_T) * T == logit(c_1) (the temperature divides the whole logit)
        l1 = np.log(c1.astype(np.float64) / (1 - c1.astype(np.float64)))
        lT = np.log(cT.astype(np.float64) / (1 - cT.astype(np.float64)))
        np.testing.assert_allclose(lT * T, l1, rtol=2e-5, atol=2e-5)
    _, _, cinf, _ = orc.draft_workload(dict(w, sts_T=np.full(3, 1e30, np.float32)))
    np.testing.assert_allclose(cinf, 0.5, atol=1e-7)


def test_survival_invariants():
    for cid in (0,):
        w = wl.make_workload(wl.WORKLOADS[cid])
        _, _, conf, surv = orc.draft_workload(w)
        assert (surv[:, 0] == conf[:, 0]).all()
        assert (np.diff(surv, axis=1) <= 0).all()
        assert ((surv >= 0) & (surv <= 1)).all()
        np.testing.assert_array_equal(surv[:, 1:], (surv[:, :-1] * conf[:, 1:]).astype(np.float32))
    w = _small("bf16", B=8, gamma=8, V=256, r=32, d=64)
    _, _, conf, surv = orc.draft_workload(w)
    assert (np.diff(surv, axis=1) <= 0).all()


def test_survival_is_expected_accepted_length_monte_carlo():
    """Accepted length of a strict prefix-matching process with conditional
    acceptance c_k has expectation sum_k S_k."""
    w = _small("f32", B=4, gamma=6, V=256, r=16, d=4)
    w["conf_w"] = (w["conf_w"] * 0.3).astype(np.float32)   # keep c away from 0/1
    _, _, conf, surv = orc.draft_workload(w)
    rng = np.random.default_rng(7)
    n = 200_000
    for b in range(4):
        acc = rng.random((n, 6)) < conf[b][None, :].astype(np.float64)
        lengths = np.cumprod(acc, axis=1).sum(axis=1)
        se = lengths.std() / math.sqrt(n)
        assert abs(lengths.mean() - float(surv[b].sum())) < 5 * se + 1e-9


def test_end_to_end_acceptance_statistics_tiny_config():
    """Not a parity pin: with the plant dominating, acceptance at position k
    is close to p (target agrees with the plant) times P(draft = plant)."""
    cfg = wl.WORKLOADS[0].replace(B=400)
    w = wl.make_workload(cfg)
    tokens, _, _, _ = orc.draft_workload(w)
    hit = (tokens == w["plant"]).mean()
    agree = (tokens == w["target"][:, :cfg.gamma]).mean()
    assert hit > 0.8
    assert abs(agree - 0.85 * hit) < 0.06
