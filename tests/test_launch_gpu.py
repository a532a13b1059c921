"""The drafting kernel under the exclusive launch mode (plain launch, the
caller guaranteeing an otherwise idle device, which a test process is) gives
the same parity as the default cooperative launch, bit for bit in tokens."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from semi_ar_drafter_amd import workloads as wl  # noqa: E402

from parity import check_draft, gpu_draft, to_device  # noqa: E402


@pytest.fixture(autouse=True)
def exclusive_launch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from semi_ar_drafter_amd import get_draft_launch, set_draft_launch
    set_draft_launch("exclusive")
    yield
    set_draft_launch("cooperative")
    assert get_draft_launch() == "cooperative"


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("B,gamma,V,r,d,dtype,sampling", [
    (6, 4, 300, 32, 8, "bf16", "greedy"),
    (40, 8, 4099, 64, 96, "bf16", "gumbel"),
    (24, 5, 3000, 32, 40, "f32", "greedy"),
])
def test_small_shapes_match_the_oracle_and_the_cooperative_launch(B, gamma, V, r, d, dtype, sampling):
    from semi_ar_drafter_amd import set_draft_launch
    cfg = wl.small_config(B=B, gamma=gamma, V=V, r=r, d=d, dtype=dtype, sampling=sampling, cid=300 + B)
    w = wl.make_workload(cfg)
    dv = to_device(w)
    say(f"[launch] exclusive {cfg.name} {sampling}")
    out = gpu_draft(dv)
    st = check_draft(w, out)
    assert st.ok(), st
    set_draft_launch("cooperative")
    ref = gpu_draft(dv)
    set_draft_launch("exclusive")
    for a, b in zip(out, ref):
        assert np.array_equal(a, b)


def test_full_size_step_all_rows():
    """B=256, gamma=16, V=151936: every token equals the cooperative launch's,
    and every request matches the oracle."""
    from semi_ar_drafter_amd import set_draft_launch
    w = wl.make_workload(wl.WORKLOADS[3])
    dv = to_device(w)
    say("[launch] exclusive full-size step")
    outs = [gpu_draft(dv) for _ in range(3)]          # back-to-back calls reuse the workspace
    set_draft_launch("cooperative")
    ref = gpu_draft(dv)
    set_draft_launch("exclusive")
    for o in outs:
        for a, b in zip(o, ref):
            assert np.array_equal(a, b)
    st = check_draft(w, outs[-1])
    assert st.ok(), st


def _dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_serving_loop_same_in_both_modes():
    from semi_ar_drafter_amd import serve, set_draft_launch
    cfg = wl.small_config(B=6, gamma=4, V=300, r=32, d=8, dtype="bf16")
    w0 = wl.make_workload(cfg)
    its = [w0] + [wl.make_inputs(cfg, iteration=t) for t in range(1, 4)]
    U = _dev(np.stack([x["U"] for x in its]))
    h = _dev(np.stack([x["h"] for x in its]))
    target = _dev(np.stack([x["target"] for x in its]))
    d = to_device(w0)

    def run():
        out = serve(d["anchor"], U, h, d["W1"], d["W2"], d["conf_w"], d["conf_b"], d["sts_T"], target, d["t_step"],
                    d["n_min"], policy="global_delayed2")
        torch.cuda.synchronize()
        return {k: v.cpu().numpy() for k, v in out.items()}

    a = run()
    set_draft_launch("cooperative")
    b = run()
    set_draft_launch("exclusive")
    for k in a:
        assert np.array_equal(a[k], b[k]), k
