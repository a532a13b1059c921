"""GPU parity of the static-threshold scheduler and of the chained serving
loop (dspark_serve) against the oracle.

The threshold lengths are bit-exact.  The serving loop is checked iteration
by iteration on the GPU's own intermediate outputs, so that a near tie in one
iteration cannot cascade: the draft of iteration t must match the oracle's
draft (tests/parity.py rule) from the anchors the GPU's verify produced at
t - 1; the verify lengths must equal the oracle's policy applied to the GPU
survivals the policy names (this iteration's, or those of t - 2); verify
outputs must equal the oracle's on the GPU tokens and lengths."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from oracle import dspark_oracle as orc  # noqa: E402
from semi_ar_drafter_amd import workloads as wl  # noqa: E402

from parity import check_draft  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from semi_ar_drafter_amd import binding
    binding.load()


def say(*a):
    print(*a, flush=True)


def dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_threshold_empty_batch():
    from semi_ar_drafter_amd import schedule_threshold
    lens, m = schedule_threshold(torch.zeros((0, 4), dtype=torch.float32, device="cuda:0"), 0.5)
    torch.cuda.synchronize()
    assert lens.numel() == 0 and int(m.cpu().numpy()[0]) == 0


@pytest.mark.parametrize("B,gamma", [(1, 1), (5, 4), (256, 16), (1000, 7), (3000, 16)])
def test_threshold_bit_exact(B, gamma):
    from semi_ar_drafter_amd import schedule_threshold
    rng = np.random.default_rng(B * 31 + gamma)
    mono = np.cumprod(rng.beta(5, 2, size=(B, gamma)), axis=1).astype(np.float32)
    rough = rng.random((B, gamma)).astype(np.float32)          # not monotone: the prefix rule decides
    for S in (mono, rough):
        S[rng.random(S.shape) < 0.05] = np.float32(0.5)        # exact equality with tau
        Sd = dev(S)
        for tau in (0.0, 0.25, 0.5, 0.9, 1.5):
            lens, m = schedule_threshold(Sd, tau)
            torch.cuda.synchronize()
            o_lens, o_m = orc.schedule_threshold(S, tau)
            assert np.array_equal(lens.cpu().numpy(), o_lens)
            assert int(m.cpu().numpy()[0]) == o_m


def serve_case(cfg, iters, policy, tau=0.4, rows=None):
    from semi_ar_drafter_amd import serve
    w0 = wl.make_workload(cfg)
    its = [w0] + [wl.make_inputs(cfg, iteration=t) for t in range(1, iters)]
    say(f"[serve] {cfg.name} iters={iters} policy={policy} sampling={cfg.sampling}")
    U = dev(np.stack([x["U"] for x in its]))
    h = dev(np.stack([x["h"] for x in its]))
    target = dev(np.stack([x["target"] for x in its]))
    out = serve(dev(w0["anchor"]), U, h, dev(w0["W1"]), dev(w0["W2"]), dev(w0["conf_w"]), w0["conf_b"],
                dev(w0["sts_T"]), target, dev(w0["t_step"]), w0["n_min"], policy=policy, tau=tau,
                mode=cfg.sampling, seed=w0["seed"])
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items()}
    del U, h
    replays = 0
    for t in range(iters):
        anchor = w0["anchor"] if t == 0 else g["bonus"][t - 1]
        wt = dict(w0)
        wt.update(anchor=np.ascontiguousarray(anchor, dtype=np.int32), U=its[t]["U"], h=its[t]["h"],
                  seed=its[t]["seed"])
        st = check_draft(wt, (g["tokens"][t], g["logit"][t], g["conf"][t], g["surv"][t]), rows=rows)
        assert st.ok(), (t, st)
        replays += st.replays
        if policy == "threshold":
            lens, M = orc.schedule_threshold(g["surv"][t], tau)
        else:
            src = g["surv"][t - 2] if (policy == "global_delayed2" and t >= 2) else g["surv"][t]
            lens, M, _ = orc.schedule(src, w0["t_step"], w0["n_min"])
        assert np.array_equal(g["lens"][t], lens) and int(g["m"][t]) == M, t
        acc, bonus = orc.verify(g["tokens"][t], its[t]["target"], g["lens"][t])
        assert np.array_equal(g["accepted"][t], acc) and np.array_equal(g["bonus"][t], bonus), t
    say(f"[serve]   M per iteration {g['m'].tolist()}  accepted {g['accepted'].sum(axis=1).tolist()}  "
        f"replays {replays}")
    return g


@pytest.mark.parametrize("policy", ["global", "global_delayed2", "threshold"])
@pytest.mark.parametrize("sampling,dtype", [("greedy", "bf16"), ("gumbel", "bf16"), ("greedy", "f32")])
def test_serve_small(policy, sampling, dtype):
    cfg = wl.small_config(B=6, gamma=4, V=300, r=32, d=8, dtype=dtype, sampling=sampling)
    serve_case(cfg, 5, policy)


def test_serve_ragged_vocabulary_and_many_requests():
    cfg = wl.small_config(B=40, gamma=8, V=4099, r=64, d=96, dtype="bf16", cid=131)
    g = serve_case(cfg, 4, "global_delayed2")
    assert np.all(g["accepted"] <= g["lens"])


def test_serve_qwen3_8b_shape():
    """B=64, gamma=16, V=151936, r=256, d=4096, three chained iterations;
    the draft is checked on a sample of requests, schedule and verify on all."""
    g = serve_case(wl.WORKLOADS[2], 3, "global", rows=[0, 17, 33, 63])
    assert g["m"].min() > 0


@pytest.mark.parametrize("sampling,dtype,r,policy", [("greedy", "bf16", 256, "global"),
                                                     ("gumbel", "bf16", 256, "global_delayed2"),
                                                     ("greedy", "f32", 16, "threshold")])
def test_serve_small_batch(sampling, dtype, r, policy):
    """Batches of at most 16 requests: the drafting kernels synchronise through
    the workgroups' winner keys, chained over iterations on one workspace."""
    cfg = wl.small_config(B=4, gamma=6, V=5000, r=r, d=16, dtype=dtype, sampling=sampling)
    serve_case(cfg, 5, policy)
