"""The allocation-free draft entry point (dspark_markov_draft_noalloc, static
per-device scratch) against the workspace entry point (dspark_markov_draft)
on the same inputs: two calls in a row, the second with a smaller input,
then the first shape again (the scratch must have been left clean).  Both
entry points run the same kernels, so every output is compared bit for bit.
Host-side rejection of shapes beyond the scratch is checked too."""
import ctypes
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from semi_ar_drafter_amd import binding  # noqa: E402
from semi_ar_drafter_amd import workloads as wl  # noqa: E402

from parity import to_device  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def both(shape, seed=None):
    shape = dict(shape)
    sampling = shape.pop("sampling", "greedy")
    w = wl.make_workload(wl.small_config(sampling=sampling, **shape))
    if seed is not None:
        w["seed"] = seed
    cfg = w["cfg"]
    say(f"[case] noalloc vs workspace B={cfg.B} gamma={cfg.gamma} V={cfg.V} r={cfg.r} d={cfg.d} "
        f"{cfg.dtype} {cfg.sampling}")
    d = to_device(w)
    args = (d["anchor"], d["U"], d["h"], d["W1"], d["W2"], d["conf_w"], d["conf_b"], d["sts_T"])
    ref = binding.markov_draft(*args, mode=d["mode"], seed=d["seed"])
    got = binding.markov_draft_noalloc(*args, mode=d["mode"], seed=d["seed"])
    torch.cuda.synchronize()
    ref = [x.cpu().numpy() for x in ref]
    got = [x.cpu().numpy() for x in got]
    for name, a, b in zip(("tokens", "logit", "conf", "surv"), ref, got):
        assert a.shape == b.shape, name
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), name
    assert ((got[0] >= 0) & (got[0] < cfg.V)).all()
    return got


FIRST = dict(B=96, gamma=6, V=69632, r=256, d=48, dtype="bf16")                        # whole-tile kernel
SECOND = dict(B=10, gamma=3, V=3001, r=32, d=20, dtype="bf16", sampling="gumbel")     # guarded kernel, smaller
THIRD = dict(B=5, gamma=4, V=1030, r=16, d=12, dtype="f32")                           # fp32 storage


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    first = both(FIRST)
    both(SECOND, seed=0x5EED)
    both(THIRD)
    again = both(FIRST)   # the scratch was left zero-filled by the calls before
    for a, b in zip(first, again):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_noalloc_rejects_shapes_beyond_the_scratch():
    lib = binding.load()
    B, gamma, V, r = 4096, 64, 151936, 256
    assert lib.dspark_draft_workspace_bytes(B, gamma, V, r) > binding.NOALLOC_SCRATCH_BYTES
    P = ctypes.c_void_p(0x10000)
    st = lib.dspark_markov_draft_noalloc(B, gamma, V, r, 64, binding.DSPARK_BF16, P, P, P, P, P, P,
                                         ctypes.c_float(0.0), P, binding.DSPARK_GREEDY, ctypes.c_uint64(0),
                                         P, P, P, P, ctypes.c_void_p(0))
    assert st == binding.DSPARK_ERR_UNSUPPORTED
    assert "scratch" in lib.dspark_last_error().decode()
