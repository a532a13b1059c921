"""GPU parity of the sequential-temperature fit against its CPU oracle on the
same seeded calibration sets.

Both sides take the decision on exact integer sums of the residuals rounded
to 2^-32, so the chosen temperatures agree exactly unless two candidates'
sums are within a few quanta.  The only difference between the sides is in
the fp64 sigmoid: the kernel multiplies by 1/T and uses the device exp, the
oracle divides by T and uses numpy's exp, a few ulps apart.  A residual
rounded to 2^-32 then moves by one quantum once in about 2^19 evaluations,
so each candidate's integer sum moves by a few quanta at most; TOL_Q = 1024
quanta covers that with a wide margin.  Where the GPU's choice differs, the
oracle's sum for it must be within TOL_Q of the minimum, and the oracle
continues from the GPU's choice.  ECE values agree within (TOL_Q + 16) /
(2^32 N) (16 more for rounding the sum to fp64)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from oracle import dspark_oracle as orc  # noqa: E402
from semi_ar_drafter_amd import workloads as wl  # noqa: E402

TOL_Q = 1024


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from semi_ar_drafter_amd import binding
    binding.load()


def say(*a):
    print(*a, flush=True)


def gpu_fit(logit, accepted, grid, n_bins, workspace=None):
    from semi_ar_drafter_amd import sts_fit
    dev = torch.device("cuda:0")
    lo = torch.from_numpy(np.ascontiguousarray(logit)).to(dev)
    ac = torch.from_numpy(np.ascontiguousarray(accepted, dtype=np.int32)).to(dev)
    gr = torch.from_numpy(np.ascontiguousarray(grid, dtype=np.float32)).to(dev)
    c, T, e = sts_fit(lo, ac, gr, n_bins, workspace=workspace)
    torch.cuda.synchronize()
    return c.cpu().numpy(), T.cpu().numpy(), e.cpu().numpy()


def check_fit(logit, accepted, grid, n_bins, got):
    choice, T, ece = got
    N = logit.shape[0]
    near = []

    def follow(k, E, g):
        gg = int(choice[k - 1])
        if gg != g:
            assert int(E[gg]) - int(E[g]) <= TOL_Q, (k, g, gg, int(E[gg]) - int(E[g]))
            near.append(k)
        return gg

    oc, oT, oe = orc.sts_fit(logit, accepted, grid, n_bins, choose=follow)
    assert np.array_equal(oc, choice)
    assert np.array_equal(oT, T)
    assert np.array_equal(T, np.asarray(grid, dtype=np.float32)[choice])
    tol = (TOL_Q + 16) / (2.0 ** 32 * max(N, 1))
    err = float(np.max(np.abs(oe - ece))) if ece.size else 0.0
    assert err <= tol, (err, tol)
    return near, float(np.mean(oe == ece)) if ece.size else 1.0


def run_case(cfg):
    w = wl.make_sts_calibration(cfg)
    say(f"[sts] {cfg.name}: N={cfg.N} gamma={cfg.gamma} G={cfg.G} bins={cfg.n_bins}")
    got = gpu_fit(w["logit"], w["accepted"], w["grid"], w["n_bins"])
    near, exact = check_fit(w["logit"], w["accepted"], w["grid"], w["n_bins"], got)
    say(f"[sts]   choices {got[0].tolist()}  near ties {near}  bit-exact ECE {exact:.4f}")
    return w, got


def test_small_calibration_set():
    run_case(wl.STS_WORKLOADS[0])


@pytest.mark.parametrize("N,gamma,G,n_bins", [
    (1, 3, 5, 15),          # a single block
    (1023, 2, 7, 10),       # one short chunk
    (1025, 3, 100, 15),     # ragged chunk; G does not divide the workgroup
    (4099, 2, 1000, 8),     # 8000 histogram entries
    (2000, 2, 1500, 5),     # G above the workgroup size: each lane takes two candidates
    (3000, 2, 4096, 2),     # the largest grid
    (5000, 3, 32, 256),     # the most bins
    (2500, 2, 64, 1),       # one bin: |sum of residuals| / N
    (70000, 4, 128, 15),    # more chunks than compute units
])
def test_shapes(N, gamma, G, n_bins):
    cid = 400 + (N * 7 + G * 3 + n_bins) % 997
    run_case(wl.STSConfig(cid, f"sts-{N}x{gamma}x{G}x{n_bins}", N, gamma, G, n_bins))


def test_no_blocks():
    grid = np.array([2.0, 1.0, 3.0, 0.5, 4.0], dtype=np.float32)
    c, T, e = gpu_fit(np.zeros((0, 3), dtype=np.float32), np.zeros(0, dtype=np.int32), grid, 15)
    assert np.all(c == 0) and np.all(T == 2.0) and np.all(e == 0.0)


def test_equal_candidates_choose_the_first():
    w = wl.make_sts_calibration(wl.STS_WORKLOADS[0])
    grid = np.repeat(w["grid"], 2)
    c, T, e = gpu_fit(w["logit"], w["accepted"], grid, w["n_bins"])
    assert np.all(c % 2 == 0)
    assert np.array_equal(e[:, 0::2], e[:, 1::2])
    check_fit(w["logit"], w["accepted"], grid, w["n_bins"], (c, T, e))


def test_repeatable_for_any_workspace_contents():
    big = wl.make_sts_calibration(wl.STSConfig(450, "sts-repeat", 20000, 5, 48, 15))
    small = wl.make_sts_calibration(wl.STS_WORKLOADS[0])
    r1 = gpu_fit(big["logit"], big["accepted"], big["grid"], big["n_bins"])
    r2 = gpu_fit(small["logit"], small["accepted"], small["grid"], small["n_bins"])
    r3 = gpu_fit(big["logit"], big["accepted"], big["grid"], big["n_bins"])
    for a, b in zip(r1, r3):
        assert np.array_equal(a, b)
    check_fit(small["logit"], small["accepted"], small["grid"], small["n_bins"], r2)
    # a workspace full of garbage gives the same result: the call clears what it needs
    from semi_ar_drafter_amd import binding
    nbytes = binding.load().dspark_sts_workspace_bytes(20000, 48, 15)
    junk = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda:0")
    r4 = gpu_fit(big["logit"], big["accepted"], big["grid"], big["n_bins"], workspace=junk)
    for a, b in zip(r1, r4):
        assert np.array_equal(a, b)


def test_labels_saturate_at_both_ends():
    w = wl.make_sts_calibration(wl.STS_WORKLOADS[0])
    a = w["accepted"].copy()
    a[a == w["cfg"].gamma] = 1000
    a[a == 0] = -5
    got = gpu_fit(w["logit"], a, w["grid"], w["n_bins"])
    ref = gpu_fit(w["logit"], w["accepted"], w["grid"], w["n_bins"])
    for x, y in zip(got, ref):
        assert np.array_equal(x, y)


def test_full_calibration_set():
    """262144 blocks x 16 positions x 128 candidates x 15 bins: the whole
    oracle (about 20 s on one core) against the GPU."""
    w, got = run_case(wl.STS_WORKLOADS[1])
    # the fit recovers the acceptance process's temperatures where labels are plentiful
    T, t_true = got[1], w["t_true"]
    assert np.all(np.abs(T[:10] / t_true[:10] - 1.0) < 0.08)
