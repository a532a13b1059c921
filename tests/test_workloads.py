"""Checks of the seeded input generator (CPU only)."""
import numpy as np
import torch

from semi_ar_drafter_amd import workloads as wl


def test_generator_is_deterministic():
    a = wl.make_workload(wl.WORKLOADS[0])
    b = wl.make_workload(wl.WORKLOADS[0])
    for key in ("anchor", "U", "h", "W1", "W2", "conf_w", "sts_T", "target", "t_step", "plant"):
        assert np.array_equal(a[key], b[key]), key
    c = wl.make_workload(wl.WORKLOADS[0], iteration=1)
    assert not np.array_equal(a["U"], c["U"])
    assert np.array_equal(a["W1"], c["W1"])       # weights do not change per iteration


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100_000).astype(np.float32) * 3
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]   # exact halfway cases
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_config_shapes_and_tables():
    cfg = wl.WORKLOADS[0]
    w = wl.make_workload(cfg)
    assert w["U"].shape == (2, 4, 1024) and w["U"].dtype == np.float32
    assert w["t_step"].shape == (2 * 4 + 1,) and w["n_min"] == 2
    np.testing.assert_allclose(w["t_step"], 1 + 0.01 * np.arange(2, 11))
    np.testing.assert_allclose(w["sts_T"], [1.1, 1.2, 1.3, 1.4], rtol=1e-6)
    c3 = wl.WORKLOADS[3]
    t, n_min = wl.sps_table(c3)
    assert n_min == 256 and t.size == 4097
    f = lambda n: 4 + 0.02 * n + 2e-5 * n * n
    assert abs(t[0] - f(256)) < 1e-9 and abs(t[-1] - f(4352)) < 1e-9
    assert (np.diff(t) > 0).all()


def test_plants_and_targets():
    cfg = wl.small_config(B=50, gamma=16, V=1000, r=16, d=8, dtype="bf16")
    w = wl.make_workload(cfg)
    U = wl.bf16_bits_to_f32(w["U"])
    got = np.take_along_axis(U, w["plant"][:, :, None].astype(np.int64), axis=2)[:, :, 0]
    assert got[:, 0].mean() > 7.5 and got[:, -1].mean() < 6.0      # 9 -> 5 decay
    agree = (w["target"][:, :16] == w["plant"]).mean(axis=0)
    assert agree[0] > 0.8 and agree[-1] < 0.8


def test_sts_calibration_set_is_deterministic_and_well_formed():
    cfg = wl.STS_WORKLOADS[0]
    a = wl.make_sts_calibration(cfg)
    b = wl.make_sts_calibration(cfg)
    for key in ("logit", "accepted", "grid"):
        assert np.array_equal(a[key], b[key])
    assert a["logit"].shape == (cfg.N, cfg.gamma) and a["logit"].dtype == np.float32
    assert a["accepted"].dtype == np.int32
    assert a["accepted"].min() >= 0 and a["accepted"].max() <= cfg.gamma
    assert a["grid"].shape == (cfg.G,) and np.all(np.diff(a["grid"]) > 0)
    assert a["grid"][0] == np.float32(cfg.grid[0])
    # a different config id gives a different set
    c = wl.make_sts_calibration(cfg.replace(cid=cfg.cid + 1))
    assert not np.array_equal(a["logit"], c["logit"])
