"""GPU parity of the RNN-head drafting (dspark_rnn_draft, through the C ABI)
against the CPU oracle's RNN head on the same seeded inputs: token ids
bit-exact, logits within 1e-2, confidences and survivals within 1e-4, near
ties replayed (the rule of the Markov-head parity tests).  Cases cover the
guarded kernel (small and ragged vocabularies, one and two request groups)
and the whole-tile kernel (vocabularies of 4352 tiles and more, two groups),
greedy and Gumbel-max drafting, and the full-size B=256, gamma=16,
V=151936, r=256 workload on sampled requests.  With zero decay the RNN head
must reproduce the Markov-head kernel's outputs bit for bit.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from semi_ar_drafter_amd import workloads as wl  # noqa: E402

from parity import check_draft, gpu_draft, gpu_rnn_draft, to_device  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from semi_ar_drafter_amd import binding
    binding.load()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = [
    # (B, gamma, V, r, d, sampling)
    (2, 4, 1024, 32, 64, "greedy"),
    (40, 6, 3000, 64, 48, "greedy"),          # guarded kernel, ragged vocabulary tail
    (200, 5, 4096, 32, 40, "greedy"),         # two groups, ragged last group
    (40, 5, 5003, 128, 32, "gumbel"),
    (140, 4, 69632, 256, 64, "greedy"),       # whole-tile kernel, two groups
    (130, 3, 69632, 256, 64, "gumbel"),
    (64, 4, 70001, 256, 64, "greedy"),        # guarded kernel at a large, odd vocabulary
    (1, 8, 151936, 256, 64, "greedy"),        # one request at the full vocabulary (latency shape)
    (3, 64, 2048, 32, 16, "greedy"),          # the longest block (gamma = 64): 63 state steps
    (256, 2, 151936, 256, 32, "gumbel"),      # whole-tile kernel, two full groups, Gumbel-max
    (17, 3, 69648, 64, 16, "greedy"),         # whole-tile kernel, rank 64, ragged single group
    (140, 3, 69632, 256, 0, "greedy"),        # whole-tile kernel without a hidden state (d = 0)
    # batches of at most 16 requests (rank 256): synchronised through the winner keys
    (4, 5, 70016, 256, 32, "gumbel"),         # whole tiles, four slots
    (2, 3, 3001, 256, 16, "greedy"),          # guarded kernel
    (8, 4, 65536, 256, 16, "greedy"),
    (16, 3, 65536, 256, 16, "gumbel"),        # the largest such batch: two requests per wave
    (2, 4, 151936, 256, 16, "gumbel"),        # five slots per wave
]


@pytest.mark.parametrize("B,gamma,V,r,d,sampling", CASES)
def test_rnn_draft_parity(B, gamma, V, r, d, sampling):
    cfg = wl.small_config(B=B, gamma=gamma, V=V, r=r, d=d, dtype="bf16")
    if sampling == "gumbel":
        cfg = cfg.replace(sampling="gumbel")
    w = wl.make_workload(cfg)
    say(f"[case] rnn B={B} gamma={gamma} V={V} r={r} d={d} {sampling}")
    dv = to_device(w)
    out = gpu_rnn_draft(dv)
    st = check_draft(w, out, head="rnn")
    say(f"  replays={st.replays} mismatches={st.mismatches} first={st.first_mismatch} "
        f"dlogit={st.max_dlogit:.2e} dconf={st.max_dconf:.2e} dsurv={st.max_dsurv:.2e}")
    assert st.ok(), st
    tok, _, _, surv = out
    assert ((tok >= 0) & (tok < V)).all()
    assert (np.diff(surv, axis=1) <= 0).all()


@pytest.mark.parametrize("B,gamma,V,r", [(40, 6, 3000, 64), (140, 4, 69632, 256), (3, 5, 65536, 256)])
def test_zero_decay_equals_markov_kernel(B, gamma, V, r):
    cfg = wl.small_config(B=B, gamma=gamma, V=V, r=r, d=32, dtype="bf16")
    w = wl.make_workload(cfg)
    say(f"[case] rnn zero decay B={B} gamma={gamma} V={V} r={r}")
    dv = to_device(w)
    dv["decay"] = torch.zeros_like(dv["decay"])
    a = gpu_rnn_draft(dv)
    b = gpu_draft(dv)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_repeated_calls_are_identical():
    cfg = wl.small_config(B=140, gamma=4, V=69632, r=256, d=32, dtype="bf16")
    w = wl.make_workload(cfg)
    dv = to_device(w)
    a = gpu_rnn_draft(dv)
    gpu_draft(dv)                 # a Markov call in between shares the workspace
    b = gpu_rnn_draft(dv)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_full_size_all_rows():
    """The B=256, gamma=16, V=151936 configuration: every request's chain
    against the RNN-head oracle."""
    cfg = wl.WORKLOADS[3]
    w = wl.make_workload(cfg)
    say(f"[case] rnn full size {cfg.name} B={cfg.B} gamma={cfg.gamma} V={cfg.V} r={cfg.r} d={cfg.d}")
    dv = to_device(w)
    out = gpu_rnn_draft(dv)
    st = check_draft(w, out, head="rnn")
    say(f"  replays={st.replays} mismatches={st.mismatches} dlogit={st.max_dlogit:.2e} dconf={st.max_dconf:.2e}")
    assert st.ok(), st
    del dv
    torch.cuda.empty_cache()


def test_rejects_fp32_storage():
    from semi_ar_drafter_amd import binding
    cfg = wl.small_config(B=4, gamma=2, V=256, r=32, d=8, dtype="f32")
    w = wl.make_workload(cfg)
    dv = to_device(w)
    with pytest.raises(TypeError):
        gpu_rnn_draft(dv)
    lib = binding.load()
    f = torch.zeros(4, dtype=torch.float32, device="cuda")
    st = lib.dspark_rnn_draft(4, 2, 256, 32, 8, binding.DSPARK_F32, *([binding._ptr(f)] * 6), binding._ptr(f),
                              binding.ctypes.c_float(1.0), binding._ptr(f), binding.DSPARK_GREEDY,
                              binding.ctypes.c_uint64(0), *([binding._ptr(f)] * 5), binding.ctypes.c_size_t(1 << 20),
                              binding._stream())
    assert st == binding.DSPARK_ERR_UNSUPPORTED
