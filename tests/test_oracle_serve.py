"""Pins of the static-threshold scheduler and of the chained serving loop in
the oracle: closed forms, brute force, agreement with the hardware-aware
scheduler where marginal analysis says they coincide, the pages' threshold
sweep behaviour (a higher threshold raises the acceptance rate), and the loop
structure (anchors chain through bonus tokens; the delayed policy uses the
survivals of two iterations earlier)."""
import numpy as np
import pytest

from oracle import dspark_oracle as orc
from semi_ar_drafter_amd import workloads as wl

TWO32 = 2.0 ** 32


def brute_threshold(S, tau):
    lens = []
    for row in np.asarray(S, dtype=np.float32):
        l = 0
        while l < len(row) and row[l] >= np.float32(tau):
            l += 1
        lens.append(l)
    return np.array(lens, dtype=np.int32)


def test_threshold_closed_forms_and_prefix_rule():
    S = np.array([[0.9, 0.4, 0.8, 0.7],      # stops at the first survival below tau
                  [0.3, 0.9, 0.9, 0.9],      # nothing
                  [0.5, 0.5, 0.5, 0.49],     # equality counts
                  [1.0, 1.0, 1.0, 1.0]], dtype=np.float32)
    lens, M = orc.schedule_threshold(S, 0.5)
    assert lens.tolist() == [1, 0, 3, 4] and M == 8
    assert orc.schedule_threshold(S, 0.0)[0].tolist() == [4, 4, 4, 4]
    assert orc.schedule_threshold(S, 1.0000001)[0].tolist() == [0, 0, 0, 0]
    rng = np.random.default_rng(2)
    for _ in range(20):
        R = rng.random((13, 7)).astype(np.float32)
        R[rng.random(R.shape) < 0.2] = np.float32(0.25)
        for tau in (0.0, 0.25, 0.5, 0.9):
            assert np.array_equal(orc.schedule_threshold(R, tau)[0], brute_threshold(R, tau))


def test_threshold_equals_global_scheduler_on_a_linear_cost_table():
    """With t(n) = a + b n the hardware-aware optimum takes exactly the gains
    above b * Phi*, so a threshold placed between the smallest taken and the
    largest untaken survival reproduces its lengths."""
    rng = np.random.default_rng(21)
    checked = 0
    for _ in range(40):
        B, g = 32, 8
        S = np.sort(rng.random((B, g)), axis=1)[:, ::-1].astype(np.float32)
        a, bb = 1.0, float(rng.uniform(0.002, 0.1))
        n = np.arange(B, B + B * g + 1, dtype=np.float64)
        lens_g, m, obj = orc.schedule(S, a + bb * n, B)
        taken = np.arange(g)[None, :] < lens_g[:, None]
        if taken.all() or not taken.any():
            continue
        lo, hi = float(S[~taken].max()), float(S[taken].min())
        if not lo < hi:
            continue
        tau = np.float32((lo + hi) / 2)
        lens_t, M = orc.schedule_threshold(S, tau)
        assert np.array_equal(lens_t, lens_g) and M == m
        assert lo <= bb * obj + 1e-7 and bb * obj <= hi + 1e-7
        checked += 1
    assert checked >= 20


def test_higher_threshold_raises_the_acceptance_rate():
    """The pages' offline threshold sweep: with calibrated survivals, raising
    the threshold drops low-value suffix tokens, so the fraction of verified
    drafts that are accepted rises.  Acceptance is simulated as the strict
    prefix process with the drafts' own conditional probabilities."""
    rng = np.random.default_rng(9)
    B, g = 20000, 8
    c = rng.beta(6, 2, size=(B, g)).astype(np.float32)
    S = np.cumprod(c, axis=1).astype(np.float32)
    accepted_all = np.cumprod(rng.random((B, g)) < c, axis=1).sum(axis=1)
    rates = []
    for tau in (0.05, 0.2, 0.4, 0.6, 0.8):
        lens, M = orc.schedule_threshold(S, tau)
        acc = np.minimum(accepted_all, lens)
        rates.append(acc.sum() / max(M, 1))
    assert all(b > a for a, b in zip(rates, rates[1:])), rates


def _serve_inputs(cfg, iters):
    w0 = wl.make_workload(cfg)
    its = []
    for t in range(iters):
        x = wl.make_inputs(cfg, iteration=t)
        its.append(dict(U=x["U"], h=x["h"], target=x["target"], seed=x["seed"]))
    return w0, its


@pytest.mark.parametrize("sampling", ["greedy", "gumbel"])
def test_serve_structure(sampling):
    cfg = wl.small_config(B=6, gamma=4, V=300, r=32, d=8, dtype="bf16", sampling=sampling)
    w0, its = _serve_inputs(cfg, 5)
    res = {p: orc.serve(w0, its, w0["anchor"], w0["t_step"], w0["n_min"], policy=p, tau=0.4, sampling=sampling)
           for p in orc.SERVE_POLICIES}
    for p, r in res.items():
        anchor = w0["anchor"]
        for t in range(5):
            # the iteration drafted from the previous bonus tokens
            tok, zs, conf, surv = orc.draft(anchor, its[t]["U"], its[t]["h"], w0["W1"], w0["W2"], w0["conf_w"],
                                            w0["conf_b"], w0["sts_T"], sampling=sampling, seed=its[t]["seed"])
            assert np.array_equal(tok, r["tokens"][t]) and np.array_equal(surv, r["surv"][t])
            if p == "threshold":
                lens, M = orc.schedule_threshold(surv, 0.4)
            else:
                src = r["surv"][t - 2] if (p == "global_delayed2" and t >= 2) else surv
                lens, M, _ = orc.schedule(src, w0["t_step"], w0["n_min"])
            assert np.array_equal(lens, r["lens"][t]) and M == r["M"][t]
            acc, bonus = orc.verify(tok, its[t]["target"], lens)
            assert np.array_equal(acc, r["accepted"][t]) and np.array_equal(bonus, r["bonus"][t])
            assert np.all(acc <= lens) and np.all(lens <= cfg.gamma)
            anchor = bonus
    # the delayed policy matches the synchronous one on the first two iterations
    for k in ("lens", "accepted", "bonus", "tokens"):
        assert np.array_equal(res["global"][k][:2], res["global_delayed2"][k][:2])
    # a zero threshold verifies every draft
    r0 = orc.serve(w0, its[:2], w0["anchor"], w0["t_step"], w0["n_min"], policy="threshold", tau=0.0,
                   sampling=sampling)
    assert np.all(r0["lens"] == cfg.gamma)
