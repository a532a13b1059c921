"""GPU parity of the parallel-only drafting kernel (no sequential head)
against its CPU oracle, on the same seeded inputs.  Greedy tokens and logits
are bit-exact (the scores are the stored values themselves); with Gumbel
noise a token may differ only where the oracle's best two scores are within
2e-2 (the noise is computed with different logarithm implementations)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from oracle import dspark_oracle as orc  # noqa: E402
from semi_ar_drafter_amd import workloads as wl  # noqa: E402

from parity import to_device  # noqa: E402

TIE_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from semi_ar_drafter_amd import binding
    binding.load()


def say(*a):
    print(*a, flush=True)


def gpu_parallel(Ud, mode="greedy", seed=0):
    from semi_ar_drafter_amd import parallel_draft
    tok, logit = parallel_draft(Ud, mode=mode, seed=seed)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), logit.cpu().numpy()


def check(U_np, tok, logit, mode, seed, rows=None):
    o_tok, o_z = orc.parallel_draft(U_np, sampling=mode, seed=seed, rows=rows)
    if rows is not None:
        tok, logit = tok[rows], logit[rows]
    if mode == "greedy":
        assert np.array_equal(tok, o_tok)
        assert np.array_equal(logit, o_z)
        return 0
    rows_a = np.arange(U_np.shape[0]) if rows is None else np.asarray(rows)
    V = U_np.shape[2]
    replays = 0
    for i, b in enumerate(rows_a):
        for k in range(U_np.shape[1]):
            if tok[i, k] == o_tok[i, k]:
                assert logit[i, k] == o_z[i, k]
                continue
            z = orc.widen(U_np[b, k]).astype(np.float32)
            s = z + orc.gumbel_noise(seed, np.full(V, b), k + 1, np.arange(V))
            gap = abs(float(s[o_tok[i, k]]) - float(s[tok[i, k]]))
            assert gap < TIE_TOL, (b, k, tok[i, k], o_tok[i, k], gap)
            assert logit[i, k] == z[tok[i, k]]
            replays += 1
    return replays


SHAPES = [
    dict(B=3, gamma=4, V=1000, dtype="bf16"),    # 16-byte path, ragged last chunk round
    dict(B=5, gamma=3, V=1003, dtype="bf16"),    # element path (V % 8 != 0)
    dict(B=4, gamma=2, V=1024, dtype="f32"),     # 16-byte path
    dict(B=2, gamma=5, V=777, dtype="f32"),      # element path
    dict(B=1, gamma=1, V=1, dtype="bf16"),       # a single id
]


@pytest.mark.parametrize("mode", ["greedy", "gumbel"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(str(v) for v in s.values()))
def test_small(shape, mode):
    cfg = wl.small_config(B=shape["B"], gamma=shape["gamma"], V=shape["V"], r=32 if shape["dtype"] == "bf16" else 16,
                          d=8, dtype=shape["dtype"], sampling=mode)
    w = wl.make_workload(cfg)
    d = to_device(w)
    seed = 0xC0FFEE1234567
    say(f"[case] parallel {shape} {mode}")
    tok, logit = gpu_parallel(d["U"], mode, seed)
    check(w["U"], tok, logit, mode, seed)


def test_ties_take_the_lowest_id():
    B, g, V = 2, 3, 4096
    U = np.zeros((B, g, V), dtype=np.float32)
    U[0, 0, [5, 77, 4000]] = 3.0           # equal maxima in different chunks and threads
    U[0, 1, :] = -1.0                      # all equal: id 0
    U[0, 2, [4095, 4094]] = 2.0
    U[1, 0, [1023, 1024, 2047]] = 1.0
    U[1, 1, [8, 9, 10, 11, 12, 13, 14, 15]] = 9.0
    U[1, 2, [4090]] = 0.5
    for dt in ("f32", "bf16"):
        if dt == "f32":
            Ud = torch.from_numpy(U).cuda()
        else:
            Ud = torch.from_numpy((U.view(np.uint32) >> 16).astype(np.uint16).view(np.int16)).cuda().view(torch.bfloat16)
        tok, logit = gpu_parallel(Ud)
        assert tok.tolist() == [[5, 0, 4094], [1023, 8, 4090]], (dt, tok.tolist())


def test_matches_markov_draft_with_zero_transition():
    from semi_ar_drafter_amd import markov_draft
    for mode in ("greedy", "gumbel"):
        cfg = wl.small_config(B=20, gamma=4, V=3000, r=64, d=16, dtype="bf16", sampling=mode)
        w = wl.make_workload(cfg)
        d = to_device(w)
        W2z = torch.zeros_like(d["W2"])
        t_m, z_m, _, _ = markov_draft(d["anchor"], d["U"], d["h"], d["W1"], W2z, d["conf_w"], d["conf_b"],
                                      d["sts_T"], mode=mode, seed=777)
        t_p, z_p = gpu_parallel(d["U"], mode, 777)
        assert np.array_equal(t_m.cpu().numpy(), t_p), mode
        assert np.array_equal(z_m.cpu().numpy(), z_p), mode


_PAR4 = {}


@pytest.mark.parametrize("cid,mode,chunk", [(3, "greedy", None)] + [(4, "gumbel", c) for c in range(2)])
def test_full_size(cid, mode, chunk):
    """Every request of the full-size configuration against the oracle (the
    stochastic B=512 case in two halves that share one GPU launch)."""
    cfg = wl.WORKLOADS[cid]
    if cid == 4 and "w" in _PAR4:
        w, tok, logit = _PAR4["w"], _PAR4["tok"], _PAR4["logit"]
    else:
        say(f"[gen] config {cid} ...")
        w = wl.make_workload(cfg)
        d = to_device(w)
        say(f"[case] parallel config {cid} {mode}")
        tok, logit = gpu_parallel(d["U"], mode, int(w["seed"]))
        del d
        if cid == 4:
            _PAR4.update(w=w, tok=tok, logit=logit)
    rows = None if chunk is None else np.arange(chunk * cfg.B // 2, (chunk + 1) * cfg.B // 2)
    r = check(w["U"], tok, logit, mode, int(w["seed"]), rows=rows)
    say(f"  replays={r}")
