"""Pins of the oracle's RNN sequential head (reading of "DSpark: DeepSeek's new
speculative decoding work", §4 "Two instantiations of the sequential block",
RNN head, whose state carries every earlier position of the draft block).

The pages give no equations, so the reading (state s_k = bf16(fp32(a * s_{k-1})
+ W1[x_{k-1}]), s_0 = 0, bias = s_k W2) is checked here against what it must
reduce to and against independent arithmetic: the Markov head at a = 0,
brute-force prefix sums at a = 1 and dyadic closed forms at a = 1/2 (all exact
in bf16), and torch's IEEE fp32 operations and bfloat16 rounding for the
state step itself.
"""
import numpy as np
import pytest
import torch

from oracle import dspark_oracle as orc
from semi_ar_drafter_amd import workloads as wl


def _bits(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200000) * rng.choice([1e-3, 1.0, 1e3], 200000)).astype(np.float32)
    # exact halfway cases between two bf16 values (ties to even)
    base = rng.integers(0, 0x7F00, 5000).astype(np.uint32) << np.uint32(16)   # finite: exponent < 0xFF
    ties = (base | np.uint32(0x8000)).view(np.float32)
    for v in (x, ties, np.array([0.0, -0.0, 1.0, -1.0, 3.0e38], dtype=np.float32)):
        assert np.array_equal(orc.bf16_round(v), _bits(v))


def test_state_step_matches_torch_fp32_ops():
    rng = np.random.default_rng(6)
    n, r = 64, 256
    sp = _bits(rng.standard_normal((n, r)).astype(np.float32))
    e = _bits((rng.standard_normal((n, r)) * 0.25).astype(np.float32))
    a = (0.5 + 0.45 * rng.random(r)).astype(np.float32)
    ts = torch.from_numpy(sp.view(np.int16)).view(torch.bfloat16).float()
    te = torch.from_numpy(e.view(np.int16)).view(torch.bfloat16).float()
    want = ((torch.from_numpy(a) * ts) + te).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.rnn_state_step(sp, a, e), want)
    # a = 0: the state is the embedding itself
    assert np.array_equal(orc.rnn_state_step(sp, np.zeros(r, np.float32), e), e)


def _small(B=5, gamma=6, V=96, r=16, d=24, seed=11):
    cfg = wl.small_config(B=B, gamma=gamma, V=V, r=r, d=d, dtype="bf16")
    w = wl.make_workload(cfg)
    return cfg, w


def test_zero_decay_is_the_markov_head():
    cfg, w = _small()
    a = orc.draft_workload(w)
    w0 = dict(w, decay=np.zeros(cfg.r, np.float32))
    b = orc.draft_workload(w0, head="rnn")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def _integer_workload(decay_value):
    """bf16 weights with small integer (or dyadic) values so that every sum
    below is exact; U plants make the chain move through different tokens."""
    cfg, w = _small(B=3, gamma=5, V=40, r=8, d=8)
    rng = np.random.default_rng(3)
    W1 = rng.integers(-3, 4, size=(cfg.V, cfg.r)).astype(np.float32)
    W2 = rng.integers(-2, 3, size=(cfg.r, cfg.V)).astype(np.float32)
    U = (rng.integers(-8, 9, size=(cfg.B, cfg.gamma, cfg.V)) * 4).astype(np.float32)
    w = dict(w, W1=_bits(W1), W2=_bits(W2), U=_bits(U), decay=np.full(cfg.r, decay_value, np.float32))
    return cfg, w, W1, W2, U


@pytest.mark.parametrize("decay", [1.0, 0.5])
def test_state_is_the_decayed_prefix_sum(decay):
    cfg, w, W1, W2, U = _integer_workload(decay)
    trace = []
    tok, zsel, _, _ = orc.draft_workload(w, head="rnn", trace=trace)
    for b in range(cfg.B):
        prefix = [int(w["anchor"][b])] + [int(t) for t in tok[b]]
        for k in range(1, cfg.gamma + 1):
            # s_k = sum_{j<k} decay^(k-1-j) W1[x_j], written out term by term
            s = [0.0] * cfg.r
            for j in range(k):
                for c in range(cfg.r):
                    s[c] += decay ** (k - 1 - j) * float(W1[prefix[j], c])
            st = trace[k - 1]
            assert np.array_equal(st["q"][b], np.array(s))
            # logits z_k(v) = U_k(v) + sum_c s[c] W2[c, v]
            z = [float(U[b, k - 1, v]) + sum(s[c] * float(W2[c, v]) for c in range(cfg.r)) for v in range(cfg.V)]
            assert np.array_equal(st["z64"][b], np.array(z))
            # the drafted token is the first maximiser
            assert tok[b, k - 1] == int(np.argmax(np.array(z, dtype=np.float32)))
            assert zsel[b, k - 1] == np.float32(z[tok[b, k - 1]])


def test_prefix_dependence_beyond_the_previous_token():
    # with a != 0 the logits at k = 2 move with the anchor even when x_1 is
    # held fixed; with a = 0 (Markov) they do not
    cfg, w, W1, W2, U = _integer_workload(1.0)
    x1 = 7

    def z2(wd, anchor):
        ww = dict(wd, anchor=np.full(cfg.B, anchor, np.int32))
        tr = []
        orc.draft_workload(ww, head="rnn", trace=tr, choose=lambda k, rows, s, x: np.full_like(x, x1) if k == 1 else x)
        return tr[1]["z64"]

    anchors = [a for a in range(cfg.V) if np.any(W1[a] != W1[0])][:1] + [0]
    assert not np.array_equal(z2(w, anchors[0]), z2(w, anchors[1]))
    w0 = dict(w, decay=np.zeros(cfg.r, np.float32))
    assert np.array_equal(z2(w0, anchors[0]), z2(w0, anchors[1]))


def test_confidence_keeps_the_markov_embedding():
    # the confidence head reads [h_k; W1[x_{k-1}]] under either head: with the
    # same drafted tokens, the confidences of the two heads coincide
    cfg, w = _small()
    tok_r, _, conf_r, surv_r = orc.draft_workload(w, head="rnn")
    forced = lambda k, rows, s, x: tok_r[rows, k - 1]  # noqa: E731
    _, _, conf_m, surv_m = orc.draft_workload(w, choose=forced)
    assert np.array_equal(conf_r, conf_m) and np.array_equal(surv_r, surv_m)


def test_rnn_head_needs_bf16_storage():
    cfg = wl.small_config(B=2, gamma=3, V=64, r=16, d=8, dtype="f32")
    w = wl.make_workload(cfg)
    with pytest.raises(TypeError):
        orc.draft_workload(w, head="rnn")
