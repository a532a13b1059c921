"""Exact ties in the drafting argmax (GPU, through the C ABI): with W2 = 0 the
logits are the bf16 base logits exactly, and each (request, position) gets
the same largest value planted at several vocabulary ids, placed in the same
lane, the same tile, different waves and different workgroups.  The drafted
token must be the lowest of those ids (the rule at every reduction level:
lanes, waves, workgroups), for the Markov and the RNN head, on the guarded
and the whole-tile kernels.  No near-tie replay applies here: tokens are
compared exactly with the oracle's first-maximum argmax.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from oracle import dspark_oracle as orc  # noqa: E402
from semi_ar_drafter_amd import workloads as wl  # noqa: E402

from parity import gpu_draft, gpu_rnn_draft, to_device  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from semi_ar_drafter_amd import binding
    binding.load()


def tied_workload(B, gamma, V, r, seed):
    cfg = wl.small_config(B=B, gamma=gamma, V=V, r=r, d=16, dtype="bf16")
    w = wl.make_workload(cfg)
    rng = np.random.default_rng(seed)
    U = wl.f32_to_bf16_bits((rng.standard_normal((B, gamma, V)) * 1.4).astype(np.float32))
    top = wl.f32_to_bf16_bits(np.array([20.0], np.float32))[0]
    ids = np.zeros((B, gamma, 4), dtype=np.int64)
    for b in range(B):
        for k in range(gamma):
            v0 = int(rng.integers(0, V - 64))
            cand = [v0,                              # ...
                    v0 + 1 + int(rng.integers(0, 3)),  # same 4-id lane group or the next one
                    v0 + 16 + int(rng.integers(0, 32)),  # a later tile (same or another wave)
                    int(rng.integers(0, V))]            # anywhere (another workgroup, often lower)
            ids[b, k] = cand
            U[b, k, cand] = top
    w = dict(w, U=U, W2=np.zeros_like(w["W2"]))
    return cfg, w, ids


@pytest.mark.parametrize("V", [3000, 69632])
@pytest.mark.parametrize("head", ["markov", "rnn"])
def test_lowest_id_wins_exact_ties(V, head):
    cfg, w, ids = tied_workload(B=40, gamma=3, V=V, r=64 if V < 10000 else 256, seed=V + (head == "rnn"))
    d = to_device(w)
    tok = (gpu_rnn_draft(d) if head == "rnn" else gpu_draft(d))[0]
    want = ids.min(axis=2)
    o_tok = orc.draft_workload(w, head=head)[0]
    assert np.array_equal(o_tok, want)          # the oracle's first maximum is the lowest tied id
    assert np.array_equal(tok, want)
