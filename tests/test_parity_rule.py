"""The parity checker's near-tie rule, exercised on the CPU with fabricated
GPU outputs (no GPU needed).

Rule under test (tests/parity.py): token ids must equal the oracle's, except
at a (request, position) where the oracle's top-2 score gap is below 2e-2;
there a different token is accepted if the oracle scores it within 2e-2 of
the maximum, and the oracle's chain then continues from that token (the next
position's gathered embedding is the replayed token's row).

The workload is a tiny fp32 case, so base logits can be set to exact values:
a near tie is planted at request 1, position 1, and position 2's base logits
are flattened so that its token is decided by the transition row of the
position-1 token alone, which makes the two chains differ after the tie.
"""
import numpy as np
import pytest

from oracle import dspark_oracle as orc
from parity import TIE_TOL, check_draft
from semi_ar_drafter_amd import workloads as wl


def _workload():
    cfg = wl.small_config(B=3, gamma=4, V=64, r=16, d=8, dtype="f32")
    w = wl.make_workload(cfg)
    U = w["U"].copy()
    trace = []
    orc.draft_workload(w, trace=trace)
    z = trace[0]["z64"][1]                      # request 1, position 1 (fp64 logits)
    bias = z - U[1, 0].astype(np.float64)
    top = int(np.argmax(z))
    runner = (top + 7) % cfg.V
    far = (top + 13) % cfg.V
    # the runner-up 0.005 below the maximum (a near tie); one token 0.3 below
    U[1, 0, runner] = np.float32(z[top] - 0.005 - bias[runner])
    U[1, 0, far] = np.float32(z[top] - 0.3 - bias[far])
    # every other logit of that row well below both
    others = np.setdiff1d(np.arange(cfg.V), [top, runner, far])
    U[1, 0, others] = np.float32(z[top] - 5.0) - bias[others].astype(np.float32)
    # position 2 decided by the transition row of x_1 only
    U[1, 1, :] = 0.0
    w = dict(w, U=U)
    return w, top, runner, far


def _chain(w, forced):
    """Oracle outputs with the tokens of `forced` {(request, k): token} imposed."""
    def choose(k, rows, s, x):
        x = x.copy()
        for i, b in enumerate(rows):
            if (int(b), k) in forced:
                x[i] = forced[(int(b), k)]
        return x
    return orc.draft_workload(w, choose=choose)


def test_planted_tie_is_where_intended():
    w, top, runner, far = _workload()
    trace = []
    orc.draft_workload(w, trace=trace)
    s = trace[0]["s"][1].astype(np.float64)
    assert int(np.argmax(s)) == top
    gap = s[top] - s[runner]
    assert 0.0 < gap < TIE_TOL
    assert s[top] - s[far] > TIE_TOL
    # the two continuations differ at position 2, so a checker that did not
    # replay the GPU's token would see a mismatch there
    own = orc.draft_workload(w)[0]
    alt = _chain(w, {(1, 1): runner})[0]
    assert own[1, 0] == top and alt[1, 0] == runner
    assert own[1, 1] != alt[1, 1]


def test_near_tie_alternative_is_replayed():
    w, top, runner, far = _workload()
    fake = _chain(w, {(1, 1): runner})          # a GPU that picked the runner-up
    st = check_draft(w, fake)
    assert st.replays == 1
    assert st.mismatches == 0
    assert st.ok(), st
    assert st.max_dlogit == 0.0 and st.max_dconf == 0.0 and st.max_dsurv == 0.0


def test_token_outside_tolerance_is_a_mismatch():
    w, top, runner, far = _workload()
    # at the near-tie position, a token 0.3 below the maximum
    fake = _chain(w, {(1, 1): far})
    st = check_draft(w, fake)
    assert st.mismatches >= 1 and not st.ok()
    assert st.first_mismatch[:2] == (1, 1)
    # at a position without a near tie, any other token
    own = orc.draft_workload(w)
    k0 = int(own[0][0, 0])
    fake = _chain(w, {(0, 1): (k0 + 1) % w["cfg"].V})
    st = check_draft(w, fake)
    assert st.replays == 0 and st.mismatches >= 1 and not st.ok()


@pytest.mark.parametrize("bad", [-1, 64, 1 << 20])
def test_out_of_range_id_is_a_mismatch(bad):
    w, top, runner, far = _workload()
    tok, zs, conf, surv = orc.draft_workload(w)
    tok = tok.copy()
    tok[1, 0] = bad                               # at the near-tie position
    st = check_draft(w, (tok, zs, conf, surv))
    assert st.mismatches >= 1 and not st.ok()


def test_logit_and_confidence_tolerances():
    w, top, runner, far = _workload()
    tok, zs, conf, surv = orc.draft_workload(w)
    st = check_draft(w, (tok, zs + np.float32(0.009), conf, surv))
    assert st.ok(), st
    st = check_draft(w, (tok, zs + np.float32(0.011), conf, surv))
    assert not st.ok()
    st = check_draft(w, (tok, zs, conf + np.float32(2e-4), surv))
    assert not st.ok()
    st = check_draft(w, (tok, zs, conf, surv - np.float32(2e-4)))
    assert not st.ok()
