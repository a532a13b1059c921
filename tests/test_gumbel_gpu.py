"""The drafting kernels' Gumbel noise on its own (dspark_gumbel_from_words,
the same device function the kernels use) against the oracle's G = -ln(-ln u)
in fp64: every one of the 2^23 values u = (2m + 1) 2^-24 the hash words can
give, including both ends (u next to 0 and next to 1, where 1 - u is tiny)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_noise_matches_the_definition_on_every_grid_value():
    from oracle import dspark_oracle as orc
    from semi_ar_drafter_amd import binding
    m = np.arange(1 << 23, dtype=np.uint64)
    rng = np.random.default_rng(9)
    words = ((m << np.uint64(9)) | rng.integers(0, 512, m.size).astype(np.uint64)).astype(np.uint32)
    g = binding.gumbel_from_words(torch.from_numpy(words.view(np.int32)).cuda()).cpu().numpy()
    u = (2.0 * m.astype(np.float64) + 1.0) * 2.0 ** -24
    ref = -np.log(-np.log(u))
    err = np.abs(g.astype(np.float64) - ref)
    print(f"max |dG| = {err.max():.3e} at m = {int(err.argmax())}; G range [{ref.min():.2f}, {ref.max():.2f}]", flush=True)
    assert err.max() < 1e-5
    # the oracle's own noise (rounded to fp32) agrees with the definition too
    w_o = orc.gumbel_uniform_bits(123, np.arange(8), 3, np.arange(8))
    assert np.allclose(orc.gumbel_noise(123, np.arange(8), 3, np.arange(8)),
                       -np.log(-np.log((np.floor(w_o / 512.0) * 2 + 1) * 2.0 ** -24)), atol=1e-6)
