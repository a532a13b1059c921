"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Token ids, scheduled lengths and verify outputs are
bit-exact; logits within 1e-2, confidences and survivals within 1e-4; near
ties (oracle top-2 gap < 2e-2) replay the GPU's token in the oracle.

Small cases span several vocabulary tiles, several request tiles, two
request groups and ragged tails.  The five named configurations run at full
size in the launch configuration the benchmark times, and every request of
every one of them is compared with the oracle (the stochastic B=512 case in
four chunks of 128 requests that share one GPU launch, plus a second chained
iteration whose anchors are the first iteration's bonus tokens).
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from oracle import dspark_oracle as orc  # noqa: E402
from semi_ar_drafter_amd import workloads as wl  # noqa: E402

from parity import check_draft, gpu_draft, to_device  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from semi_ar_drafter_amd import binding
    binding.load()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_case(w, rows=None):
    cfg = w["cfg"]
    say(f"[case] {cfg.name} B={cfg.B} gamma={cfg.gamma} V={cfg.V} r={cfg.r} d={cfg.d} "
        f"{cfg.dtype} {cfg.sampling} seed={w['seed']}")
    d = to_device(w)
    out = gpu_draft(d)
    st = check_draft(w, out, rows=rows)
    say(f"  replays={st.replays} mismatches={st.mismatches} first={st.first_mismatch} "
        f"dlogit={st.max_dlogit:.2e} dconf={st.max_dconf:.2e} dsurv={st.max_dsurv:.2e}")
    assert st.ok(), st
    tok, logit, conf, surv = out
    assert ((tok >= 0) & (tok < cfg.V)).all()
    assert (np.diff(surv, axis=1) <= 0).all() and ((surv >= 0) & (surv <= 1)).all()
    return d, out


def gpu_schedule(d, surv_np, path="ranked", workspace=None):
    """dspark_schedule with a workspace (the multi-workgroup ranking kernel)
    or without one (the one-workgroup sorting kernel)."""
    from semi_ar_drafter_amd import schedule
    surv = torch.from_numpy(surv_np).to("cuda:0")
    lens, m, obj = schedule(surv, d["t_step"], d["n_min"], workspace=workspace, one_workgroup=path == "one_workgroup")
    torch.cuda.synchronize()
    return lens.cpu().numpy(), int(m.cpu()[0]), float(obj.cpu()[0])


def gpu_verify(tok_np, target_np, lens_np):
    from semi_ar_drafter_amd import verify
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")
    acc, bonus = verify(dev(tok_np), dev(target_np), dev(lens_np))
    torch.cuda.synchronize()
    return acc.cpu().numpy(), bonus.cpu().numpy()


def end_to_end(w, d, out):
    """Scheduler and verify on identical inputs (the GPU's own draft outputs)."""
    tok, _, _, surv = out
    lens, m, obj = gpu_schedule(d, surv)
    o_lens, o_m, o_obj = orc.schedule(surv, w["t_step"], w["n_min"])
    assert m == o_m and (lens == o_lens).all() and obj == o_obj
    acc, bonus = gpu_verify(tok, w["target"], lens)
    o_acc, o_bonus = orc.verify(tok, w["target"], lens)
    assert (acc == o_acc).all() and (bonus == o_bonus).all()
    say(f"  schedule M*={m} objective={obj:.6f} mean accepted={acc.mean():.3f}")
    return lens, acc, bonus


# --------------------------------------------------------------------------
# small cases: whole batch against the oracle
# --------------------------------------------------------------------------
def test_tiny_fp32_config():
    w = wl.make_workload(wl.WORKLOADS[0])
    d, out = run_case(w)
    end_to_end(w, d, out)


SMALL = [
    dict(B=37, gamma=5, V=1000, r=64, d=100, dtype="bf16"),            # ragged V tile, ragged request tile
    dict(B=300, gamma=3, V=4099, r=32, d=33, dtype="bf16"),            # two request groups, V % 4 != 0
    dict(B=16, gamma=4, V=8192, r=256, d=64, dtype="bf16"),            # full rank, exact tiles
    dict(B=5, gamma=6, V=2051, r=128, d=8, dtype="bf16"),
    dict(B=9, gamma=4, V=777, r=16, d=20, dtype="f32"),
    dict(B=33, gamma=3, V=3000, r=64, d=40, dtype="f32"),
    dict(B=20, gamma=3, V=3000, r=64, d=0, dtype="bf16"),              # no hidden state (d = 0)
    dict(B=140, gamma=3, V=69632, r=256, d=0, dtype="bf16"),           # whole-tile kernel, d = 0
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(str(v) for v in s.values()))
def test_small_greedy(shape):
    w = wl.make_workload(wl.small_config(**shape))
    d, out = run_case(w)
    end_to_end(w, d, out)


@pytest.mark.parametrize("shape", [dict(B=20, gamma=4, V=3000, r=64, d=32, dtype="bf16"),
                                   dict(B=7, gamma=5, V=1234, r=32, d=16, dtype="f32")],
                         ids=["bf16", "f32"])
def test_small_gumbel(shape):
    cfg = wl.small_config(sampling="gumbel", **shape)
    w = wl.make_workload(cfg)
    w["seed"] = 0x123456789AB
    d, out = run_case(w)
    end_to_end(w, d, out)


# Batches of at most 16 requests synchronise the draft positions through each
# workgroup's winner keys instead of arrival counters (bf16 at rank 256, fp32
# at rank 16): every kernel instance of that path, both samplings, one and two
# requests per wave.
SMALL_BATCH = [
    (dict(B=3, gamma=5, V=3001, r=256, d=24, dtype="bf16"), "greedy"),       # guarded kernel, ragged tile
    (dict(B=1, gamma=6, V=3001, r=256, d=8, dtype="bf16"), "gumbel"),
    (dict(B=8, gamma=4, V=65536, r=256, d=16, dtype="bf16"), "greedy"),      # whole tiles, four slots; largest B
    (dict(B=4, gamma=4, V=70016, r=256, d=16, dtype="bf16"), "gumbel"),
    (dict(B=2, gamma=3, V=151936, r=256, d=16, dtype="bf16"), "gumbel"),     # five slots
    (dict(B=2, gamma=3, V=777, r=16, d=8, dtype="f32"), "greedy"),
    (dict(B=3, gamma=4, V=1030, r=16, d=12, dtype="f32"), "gumbel"),
    (dict(B=16, gamma=4, V=65536, r=256, d=16, dtype="bf16"), "greedy"),     # two requests per wave; largest B
    (dict(B=12, gamma=3, V=5003, r=256, d=16, dtype="bf16"), "gumbel"),
    (dict(B=9, gamma=3, V=151936, r=256, d=16, dtype="bf16"), "greedy"),
    (dict(B=16, gamma=3, V=2000, r=16, d=8, dtype="f32"), "greedy"),
    # tiny vocabularies: one workgroup owning every request, ten owning up to two each
    (dict(B=16, gamma=3, V=16, r=16, d=8, dtype="f32"), "greedy"),
    (dict(B=16, gamma=2, V=160, r=256, d=8, dtype="bf16"), "gumbel"),
]


@pytest.mark.parametrize("shape,sampling", SMALL_BATCH,
                         ids=lambda v: "x".join(str(x) for x in v.values()) if isinstance(v, dict) else v)
def test_small_batch(shape, sampling):
    w = wl.make_workload(wl.small_config(sampling=sampling, **shape))
    if sampling == "gumbel":
        w["seed"] = 0x5EED0001
    d, out = run_case(w)
    end_to_end(w, d, out)


@pytest.mark.parametrize("V,sampling", [(70016, "greedy"), (100000, "greedy"), (131072, "greedy"),
                                        (100000, "gumbel"), (140000, "greedy"), (140000, "gumbel")])
def test_vocab_splits_of_the_whole_tile_path(V, sampling):
    """V % 16 == 0 and at least two tiles per wave: the branch-free path with
    paired tiles.  On a 256-CU GPU the first four vocabularies take the
    four-slot kernel with waves owning {2, 3}, {3, 4} and exactly 4 tiles
    (odd counts use the overlapping last pair), the last two the five-slot
    kernel with waves owning {4, 5} tiles (spare last slot)."""
    cfg = wl.small_config(B=24, gamma=3, V=V, r=256, d=64, dtype="bf16", sampling=sampling)
    w = wl.make_workload(cfg)
    if sampling == "gumbel":
        w["seed"] = 0xBADC0FFEE
    d, out = run_case(w)
    end_to_end(w, d, out)


def test_small_weak_plant_many_near_ties():
    """No plant: logits are pure noise, so the oracle meets top-2 score gaps
    below the near-tie tolerance at many positions; the GPU must still agree
    under the replay rule."""
    from parity import TIE_TOL
    cfg = wl.small_config(B=64, gamma=4, V=20000, r=64, d=16, dtype="bf16", plant=(0.0, 0.0))
    w = wl.make_workload(cfg)
    trace = []
    orc.draft_workload(w, trace=trace)
    near = sum(int((np.diff(np.sort(t["s"], axis=1)[:, -2:], axis=1)[:, 0] < TIE_TOL).sum()) for t in trace)
    say(f"  oracle positions with a top-2 gap below {TIE_TOL}: {near} of {cfg.B * cfg.gamma}")
    assert near > 0
    run_case(w)


def test_out_of_range_anchors_are_clamped():
    cfg = wl.small_config(B=6, gamma=3, V=500, r=32, d=8, dtype="bf16")
    w = wl.make_workload(cfg)
    bad = w["anchor"].copy()
    bad[:3] = [-7, 500, 10 ** 6]
    w["anchor"] = bad
    d = to_device(w)
    out = gpu_draft(d)
    w_ref = dict(w, anchor=np.clip(bad, 0, cfg.V - 1).astype(np.int32))
    st = check_draft(w_ref, out)
    assert st.ok(), st


def test_determinism_bitwise():
    w = wl.make_workload(wl.small_config(B=70, gamma=4, V=5000, r=64, d=24, dtype="bf16"))
    d = to_device(w)
    a = gpu_draft(d)
    b = gpu_draft(d)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_empty_batch_is_noop():
    from semi_ar_drafter_amd import markov_draft
    w = wl.make_workload(wl.small_config(B=0, gamma=4, V=256, r=32, d=8, dtype="bf16"))
    d = to_device(w)
    tok, logit, conf, surv = markov_draft(d["anchor"], d["U"], d["h"], d["W1"], d["W2"], d["conf_w"],
                                          1.0, d["sts_T"])
    assert tok.shape == (0, 4)


# --------------------------------------------------------------------------
# scheduler and verify alone, on random inputs
# --------------------------------------------------------------------------
def _rand_surv(rng, B, g, mode):
    if mode == "ties":
        c = np.array([1.0, 0.5, 0.25, 0.0], np.float32)[rng.integers(0, 4, size=(B, g))]
    elif mode == "saturated":
        c = np.where(rng.random((B, g)) < 0.7, 1.0, rng.random((B, g)) * 1e-6).astype(np.float32)
    else:
        c = rng.random((B, g)).astype(np.float32)
    S = np.cumprod(c, axis=1, dtype=np.float32)
    for k in range(1, g):       # exact fp32 running product
        S[:, k] = (S[:, k - 1] * c[:, k]).astype(np.float32)
    return S


SCHED_PATHS = ["ranked", "one_workgroup"]


@pytest.mark.parametrize("path", SCHED_PATHS)
@pytest.mark.parametrize("B,g", [(1, 1), (3, 5), (64, 16), (256, 16), (512, 16), (1024, 16), (100, 3)])
@pytest.mark.parametrize("mode", ["random", "ties", "saturated"])
def test_schedule_parity(B, g, mode, path):
    rng = np.random.default_rng(B * 131 + g * 7 + len(mode))
    S = _rand_surv(rng, B, g, mode)
    for table in ("linear", "quad"):
        n = np.arange(B, B + B * g + 1, dtype=np.float64)
        t = 1.0 + 0.01 * n if table == "linear" else 4.0 + 0.02 * n + 2e-5 * n * n
        d = dict(t_step=torch.from_numpy(t).to("cuda:0"), n_min=B)
        lens, m, obj = gpu_schedule(d, S, path)
        o_lens, o_m, o_obj = orc.schedule(S, t, B)
        assert m == o_m and (lens == o_lens).all() and obj == o_obj, (table, m, o_m)


@pytest.mark.parametrize("path", SCHED_PATHS)
@pytest.mark.parametrize("B,g", [(7, 5), (256, 16), (512, 16), (333, 21), (1024, 16), (3000, 5)])
def test_schedule_parity_rows_not_monotone(B, g, path):
    """Both kernels order all entries (a full sort, or ranks over all
    entries): survivals in any order (outside the documented contract)
    still give the oracle's top-M set."""
    rng = np.random.default_rng(B * 7 + g)
    S = rng.random((B, g)).astype(np.float32)
    S[rng.random((B, g)) < 0.1] = np.float32(0.5)
    n = np.arange(B, B + B * g + 1, dtype=np.float64)
    t = 4.0 + 0.02 * n + 2e-5 * n * n
    d = dict(t_step=torch.from_numpy(t).to("cuda:0"), n_min=B)
    lens, m, obj = gpu_schedule(d, S, path)
    o_lens, o_m, o_obj = orc.schedule(S, t, B)
    assert m == o_m and (lens == o_lens).all() and obj == o_obj


@pytest.mark.parametrize("path", SCHED_PATHS)
def test_schedule_table_offset_and_short_table(path):
    rng = np.random.default_rng(3)
    S = _rand_surv(rng, 40, 8, "random")
    n_min = 10
    t = 2.0 + 0.05 * np.arange(n_min, 40 + 100, dtype=np.float64)   # covers M <= 99 only
    d = dict(t_step=torch.from_numpy(t).to("cuda:0"), n_min=n_min)
    lens, m, obj = gpu_schedule(d, S, path)
    o_lens, o_m, o_obj = orc.schedule(S, t, n_min)
    assert m == o_m and (lens == o_lens).all() and obj == o_obj


@pytest.mark.parametrize("path", SCHED_PATHS)
@pytest.mark.parametrize("B,g", [(1, 300), (3, 1000), (16, 1024), (16384, 1), (4096, 4), (2, 8192)])
def test_schedule_extreme_shapes(B, g, path):
    """Long rows (gamma > 255: one LDS counter per request instead of four
    per word), the most requests (B = 16384), and a table shorter than the
    drafts for the widest rows."""
    rng = np.random.default_rng(B + 3 * g)
    S = _rand_surv(rng, B, g, "random" if B % 2 else "ties")
    n_all = B * g
    cnt = min(n_all + 1, 5000) if g >= 1000 else n_all + 1
    t = 4.0 + 0.02 * np.arange(B, B + cnt, dtype=np.float64) + 3e-6 * np.arange(cnt, dtype=np.float64) ** 2
    d = dict(t_step=torch.from_numpy(t).to("cuda:0"), n_min=B)
    lens, m, obj = gpu_schedule(d, S, path)
    o_lens, o_m, o_obj = orc.schedule(S, t, B)
    assert m == o_m and (lens == o_lens).all() and obj == o_obj, (B, g, m, o_m)


def test_schedule_workspace_reused_across_shapes():
    """One workspace, consecutive calls of different sizes: each call puts the
    ticket counter back to zero, so every call's last workgroup is the one
    that sees all ranks."""
    from semi_ar_drafter_amd import binding
    ws = torch.zeros(binding.schedule_workspace_bytes(1024, 16), dtype=torch.uint8, device="cuda:0")
    rng = np.random.default_rng(21)
    for B, g in [(1024, 16), (5, 3), (256, 16), (1, 1), (700, 7), (1024, 16)]:
        S = _rand_surv(rng, B, g, "random")
        t = 4.0 + 0.02 * np.arange(B, B + B * g + 1, dtype=np.float64) + 1e-5 * np.arange(B * g + 1) ** 2
        d = dict(t_step=torch.from_numpy(t).to("cuda:0"), n_min=B)
        lens, m, obj = gpu_schedule(d, S, "ranked", workspace=ws)
        o_lens, o_m, o_obj = orc.schedule(S, t, B)
        assert m == o_m and (lens == o_lens).all() and obj == o_obj, (B, g)
    assert int(ws[:4].view(torch.int32).cpu()[0]) == 0


@pytest.mark.parametrize("path", SCHED_PATHS)
def test_schedule_no_drafts(path):
    """gamma = 0: nothing to schedule, M* = 0 and every length 0."""
    S = np.zeros((6, 0), dtype=np.float32)
    t = np.array([3.0, 3.5], dtype=np.float64)
    d = dict(t_step=torch.from_numpy(t).to("cuda:0"), n_min=6)
    lens, m, obj = gpu_schedule(d, S, path)
    o_lens, o_m, o_obj = orc.schedule(S, t, 6)
    assert m == o_m == 0 and (lens == o_lens).all() and (lens == 0).all() and obj == o_obj


def test_verify_parity_random():
    rng = np.random.default_rng(9)
    # gamma < 64 runs one lane per position (segments of 4..64 lanes), gamma >= 64 one thread per request
    for B, g, V in [(1, 1, 2), (1000, 16, 3), (513, 7, 2), (64, 16, 5), (100, 0, 2), (50, 63, 2), (20, 64, 2),
                    (10, 100, 2), (300, 31, 2), (70, 32, 2), (5, 3, 2), (4097, 16, 2)]:
        tok = rng.integers(0, V, size=(B, g)).astype(np.int32)
        tgt = rng.integers(0, V, size=(B, g + 1)).astype(np.int32)
        lens = rng.integers(-2, g + 3, size=B).astype(np.int32)     # out-of-range lengths are clamped
        acc, bonus = gpu_verify(tok, tgt, lens)
        o_acc, o_bonus = orc.verify(tok, tgt, np.clip(lens, 0, g))
        assert (acc == o_acc).all() and (bonus == o_bonus).all()
        # drafts that mostly agree with the target: long accepted prefixes
        tok2 = tgt[:, :g].copy()
        flip = rng.random((B, g)) < 0.03
        tok2[flip] = (tok2[flip] + 1) % V
        acc, bonus = gpu_verify(tok2, tgt, lens)
        o_acc, o_bonus = orc.verify(tok2, tgt, np.clip(lens, 0, g))
        assert (acc == o_acc).all() and (bonus == o_bonus).all(), (B, g)


# --------------------------------------------------------------------------
# full-size configurations
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cid", [1, 2, 3])
def test_full_size_config(cid):
    """Every request of the full-size configuration against the oracle."""
    cfg = wl.WORKLOADS[cid]
    say(f"[gen] config {cid} ...")
    w = wl.make_workload(cfg)
    d, out = run_case(w)
    end_to_end(w, d, out)


_CFG4 = {}


def _config4_iteration0():
    """One GPU launch of the stochastic B=512 configuration, shared by the
    chunked comparisons below (generated once per test session)."""
    if "w" not in _CFG4:
        cfg = wl.WORKLOADS[4]
        say("[gen] config 4 iteration 0 ...")
        w = wl.make_workload(cfg)
        d = to_device(w)
        say(f"[case] {cfg.name} B={cfg.B} gamma={cfg.gamma} V={cfg.V} {cfg.sampling} seed={w['seed']}")
        out = gpu_draft(d)
        tok, _, _, surv = out
        assert ((tok >= 0) & (tok < cfg.V)).all()
        lens, acc, bonus = end_to_end(w, d, out)
        _CFG4.update(w=w, d=d, out=out, bonus=bonus)
    return _CFG4


@pytest.mark.parametrize("chunk", range(4))
def test_full_size_config4_all_rows(chunk):
    """Config 4 (B=512, V=129280, Gumbel-max), requests 128*chunk .. +127:
    together the four chunks compare every request with the oracle."""
    c = _config4_iteration0()
    rows = np.arange(128 * chunk, 128 * (chunk + 1))
    st = check_draft(c["w"], c["out"], rows=rows)
    say(f"  rows {rows[0]}..{rows[-1]}: replays={st.replays} mismatches={st.mismatches} "
        f"first={st.first_mismatch} dlogit={st.max_dlogit:.2e} dconf={st.max_dconf:.2e}")
    assert st.ok(), st


def test_full_size_config4_chained_iteration():
    """Iteration 1 of config 4 at full size: anchors are the bonus tokens the
    GPU verify step returned for iteration 0, the Gumbel seed is seed0 + 1.
    Two requests from every 16-request tile (first and last, so every tile
    of every request group and both ends of each) are compared."""
    c = _config4_iteration0()
    cfg = wl.WORKLOADS[4]
    w1 = wl.make_workload(cfg, iteration=1, anchor=c["bonus"])
    assert w1["seed"] == c["w"]["seed"] + 1
    d1 = to_device(w1)
    out1 = gpu_draft(d1)
    rows = np.sort(np.concatenate([np.arange(0, cfg.B, 16), np.arange(15, cfg.B, 16)]))
    st = check_draft(w1, out1, rows=rows)
    say(f"  iteration 1, {rows.size} rows: replays={st.replays} mismatches={st.mismatches} "
        f"first={st.first_mismatch} dlogit={st.max_dlogit:.2e}")
    assert st.ok(), st
    end_to_end(w1, d1, out1)


def test_chained_gumbel_iterations():
    """Config 4 semantics at reduced batch: iteration t+1's anchor is
    iteration t's bonus token and its seed is seed0 + t."""
    cfg = wl.WORKLOADS[4].replace(B=24, cid=40)
    anchor = None
    for it in range(4):
        w = wl.make_workload(cfg, iteration=it, anchor=anchor)
        d, out = run_case(w)
        lens, acc, bonus = end_to_end(w, d, out)
        anchor = bonus


def test_dirty_workspace_is_flagged_and_cleaned():
    """A workspace that was not zero-filled is detected (all tokens -1) and the
    call leaves it clean, so the next call is correct."""
    from semi_ar_drafter_amd import binding, markov_draft
    w = wl.make_workload(wl.small_config(B=20, gamma=3, V=2000, r=32, d=16, dtype="bf16"))
    d = to_device(w)
    nb = binding.workspace_bytes(20, 3, 2000, 32)
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda:0")
    args = (d["anchor"], d["U"], d["h"], d["W1"], d["W2"], d["conf_w"], d["conf_b"], d["sts_T"])
    tok, _, _, _ = markov_draft(*args, workspace=ws)
    torch.cuda.synchronize()
    assert (tok.cpu().numpy() == -1).all()
    out = markov_draft(*args, workspace=ws)
    torch.cuda.synchronize()
    st = check_draft(w, tuple(x.cpu().numpy() for x in out))
    assert st.ok(), st


def test_dirty_small_batch_workspace_is_flagged_and_cleaned():
    """Batches of at most 16 requests do not use the barrier counters: stale
    winner keys are what is detected.  The control words and the counters
    (the first 512 bytes for such a batch) are left clean and everything
    after them dirty: the call returns all -1 and leaves the workspace clean."""
    from semi_ar_drafter_amd import binding, markov_draft
    w = wl.make_workload(wl.small_config(B=3, gamma=3, V=3001, r=256, d=16, dtype="bf16"))
    d = to_device(w)
    nb = binding.workspace_bytes(3, 3, 3001, 256)
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda:0")
    ws[:512] = 0
    args = (d["anchor"], d["U"], d["h"], d["W1"], d["W2"], d["conf_w"], d["conf_b"], d["sts_T"])
    tok, _, _, _ = markov_draft(*args, workspace=ws)
    torch.cuda.synchronize()
    assert (tok.cpu().numpy() == -1).all()
    out = markov_draft(*args, workspace=ws)
    torch.cuda.synchronize()
    st = check_draft(w, tuple(x.cpu().numpy() for x in out))
    assert st.ok(), st
