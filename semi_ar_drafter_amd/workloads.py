"""Seeded synthetic workloads for the Markov-head draft / schedule / verify path.

This module only *creates inputs*.  It holds none of the method's arithmetic:
no logits, no argmax, no confidence, no scheduling, no verification.  Both the
HIP path (through the tests and the benchmark) and the CPU oracle read the
arrays it returns, so the two sides always see identical bytes.

Shapes follow the pages' statement of the problem: base logits U_k and hidden
states h_k per draft position from the parallel backbone
("DSpark: DeepSeek's new speculative decoding work", §4 "Semi-Autoregressive
Generation", parallel stage), the low-rank transition factors W1 [V, r] and
W2 [r, V] (same page, §4, Markov head), a linear confidence head over the
backbone hidden state and the Markov embedding (same page, §5), per-position
temperatures (same page, §5, Sequential Temperature Scaling) and a step-cost
table standing in for the serving system's steps-per-second curve
("DSpark: Overcoming the Efficiency Wall in LLM Speculative Decoding",
"2. The Hardware-Aware Prefix Scheduler").

Value recipe (the trained models and datasets behind the pages are not
available, so these distributions stand in for them):

* N(mu, s) in a config description is read as mean mu and *variance* s.
  U ~ N(0, 2);  W1, W2 ~ N(0, 1/sqrt(r)) so that one Markov bias entry has unit
  variance;  h ~ N(0, 1);  conf_w ~ N(0, 0.05);  conf_b = 1.0;
  T_k = 1 + 0.1 k for k = 1..gamma.
* One "planted" token per (request, position), uniform over the vocabulary,
  gets an additive offset s_k on top of its U sample.  s_k is constant or
  decays linearly in k between the configured end points.
* Target tokens: position k (1-based) equals the planted token with
  probability p_k (constant or linear in k), otherwise a uniform token (which
  may coincide with the plant).  Column gamma (position gamma + 1, the token
  the target emits after a fully accepted block) is uniform.  Anchors are
  uniform.
* bf16 tensors are fp32 samples rounded to bfloat16 by round-to-nearest-even
  and stored as uint16 bit patterns.
* Step-cost table: dense fp64 array over every integer n in [B, B + B*gamma].
  "linear" tables evaluate a + b*n at every n.  "quad64" tables sample
  f(n) = a + b*n + c*n^2 at 64 real points n_j = B + B*gamma*j/63 and
  interpolate linearly to each integer n.

Randomness: numpy PCG64 streams spawned from
SeedSequence([20260629, config id, tag, iteration]) with one fixed tag per
tensor, so each tensor is reproducible on its own.  Weights (W1, W2, conf_w)
do not depend on the iteration; per-iteration inputs do.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SEED_ROOT = 20260629

# Fixed per-tensor stream tags (never reorder: they define the bytes).
_TAG_W1, _TAG_W2, _TAG_CONFW = 1, 2, 3
_TAG_ANCHOR, _TAG_U, _TAG_PLANT, _TAG_H, _TAG_TGT_COIN, _TAG_TGT_UNI = 10, 11, 12, 13, 14, 15
_TAG_STS_LOGIT, _TAG_STS_NOISE = 20, 21
_TAG_DECAY = 30


@dataclasses.dataclass(frozen=True)
class Config:
    cid: int
    name: str
    B: int
    gamma: int
    V: int
    r: int
    d: int
    dtype: str                  # "f32" or "bf16": storage type of U, h, W1, W2
    plant: tuple                # (s at k=1, s at k=gamma)
    p_target: tuple             # (p at k=1, p at k=gamma)
    sps: tuple                  # ("linear", a, b) or ("quad64", a, b, c)
    sampling: str = "greedy"    # "greedy" or "gumbel"
    gumbel_seed0: int = 0x5EED  # iteration t uses gumbel_seed0 + t

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    0: Config(0, "tiny-fp32", 2, 4, 1024, 16, 64, "f32", (8.0, 8.0), (0.85, 0.85),
              ("linear", 1.0, 0.01)),
    1: Config(1, "qwen3-4b-latency", 1, 8, 151936, 256, 2560, "bf16", (8.0, 8.0),
              (0.85, 0.85), ("linear", 1.0, 0.01)),
    2: Config(2, "qwen3-8b", 64, 16, 151936, 256, 4096, "bf16", (9.0, 5.0),
              (0.9, 0.7), ("linear", 1.0, 0.01)),
    3: Config(3, "qwen3-14b-sched", 256, 16, 151936, 256, 5120, "bf16", (9.0, 5.0),
              (0.9, 0.7), ("quad64", 4.0, 0.02, 2e-5)),
    4: Config(4, "large-vocab-gumbel", 512, 16, 129280, 256, 7168, "bf16", (9.0, 5.0),
              (0.9, 0.7), ("quad64", 4.0, 0.02, 2e-5), sampling="gumbel"),
}


def _rng(cfg: Config, tag: int, iteration: int = -1) -> np.random.Generator:
    key = [SEED_ROOT, cfg.cid, tag] if iteration < 0 else [SEED_ROOT, cfg.cid, tag, iteration]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns.

    Inputs are finite by construction (normal samples plus small offsets).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to fp32 (for host-side helpers)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def linear_in_k(first: float, last: float, gamma: int) -> np.ndarray:
    """Per-position parameter for k = 1..gamma, linear from `first` to `last`."""
    if gamma == 1:
        return np.array([first], dtype=np.float64)
    k = np.arange(gamma, dtype=np.float64)
    return first + (last - first) * k / (gamma - 1)


def sps_table(cfg: Config):
    """Dense step-cost table t_step[n - n_min] for n in [B, B + B*gamma]; returns (t, n_min)."""
    B, g = cfg.B, cfg.gamma
    n = np.arange(B, B + B * g + 1, dtype=np.float64)
    kind = cfg.sps[0]
    if kind == "linear":
        _, a, b = cfg.sps
        t = a + b * n
    elif kind == "quad64":
        _, a, b, c = cfg.sps
        nj = B + (B * g) * np.arange(64, dtype=np.float64) / 63.0
        tj = a + b * nj + c * nj * nj
        t = np.interp(n, nj, tj)
    else:
        raise ValueError(kind)
    return np.ascontiguousarray(t, dtype=np.float64), B


def make_weights(cfg: Config) -> dict:
    """Markov-head weights and confidence head (iteration independent)."""
    V, r, d = cfg.V, cfg.r, cfg.d
    sd = float(r) ** -0.25
    W1 = _store(_rng(cfg, _TAG_W1).standard_normal((V, r), dtype=np.float32) * np.float32(sd), cfg.dtype)
    W2 = _store(_rng(cfg, _TAG_W2).standard_normal((r, V), dtype=np.float32) * np.float32(sd), cfg.dtype)
    conf_w = (_rng(cfg, _TAG_CONFW).standard_normal(d + r, dtype=np.float32)
              * np.float32(np.sqrt(0.05))).astype(np.float32)
    sts_T = (1.0 + 0.1 * np.arange(1, cfg.gamma + 1)).astype(np.float32)
    # per-channel decay of the RNN head's recurrent state, uniform in [0.5, 0.95)
    decay = (0.5 + 0.45 * _rng(cfg, _TAG_DECAY).random(r, dtype=np.float32)).astype(np.float32)
    return dict(W1=W1, W2=W2, conf_w=conf_w, conf_b=1.0, sts_T=sts_T, decay=decay)


def make_inputs(cfg: Config, iteration: int = 0, anchor: Optional[np.ndarray] = None, progress=None) -> dict:
    """Per-iteration inputs: anchor, U (with plants), h, plant ids, targets.
    `progress(b)`, if given, is called every 64 requests of the U loop."""
    B, g, V, d = cfg.B, cfg.gamma, cfg.V, cfg.d
    if anchor is None:
        anchor = _rng(cfg, _TAG_ANCHOR, iteration).integers(0, V, size=B, dtype=np.int64)
    anchor = np.ascontiguousarray(anchor, dtype=np.int32)
    plant = _rng(cfg, _TAG_PLANT, iteration).integers(0, V, size=(B, g), dtype=np.int64).astype(np.int32)
    s_k = linear_in_k(cfg.plant[0], cfg.plant[1], g).astype(np.float32)
    store_dt = np.uint16 if cfg.dtype == "bf16" else np.float32
    U = np.empty((B, g, V), dtype=store_dt)
    ru = _rng(cfg, _TAG_U, iteration)
    su = np.float32(np.sqrt(2.0))
    rows = np.arange(g)
    for b in range(B):          # one request at a time bounds host memory
        if progress is not None and b % 64 == 0:
            progress(b)
        x = ru.standard_normal((g, V), dtype=np.float32) * su
        x[rows, plant[b]] += s_k
        U[b] = _store(x, cfg.dtype)
    rh = _rng(cfg, _TAG_H, iteration)
    h = np.empty((B, g, d), dtype=store_dt)
    for b in range(B):
        h[b] = _store(rh.standard_normal((g, d), dtype=np.float32), cfg.dtype)
    p_k = linear_in_k(cfg.p_target[0], cfg.p_target[1], g)
    coin = _rng(cfg, _TAG_TGT_COIN, iteration).random((B, g))
    uni = _rng(cfg, _TAG_TGT_UNI, iteration).integers(0, V, size=(B, g + 1), dtype=np.int64).astype(np.int32)
    target = uni.copy()
    hit = coin < p_k[None, :]
    target[:, :g][hit] = plant[hit]
    t_step, n_min = sps_table(cfg)
    seed = (cfg.gumbel_seed0 + iteration) if cfg.sampling == "gumbel" else 0
    return dict(anchor=anchor, U=U, h=h, plant=plant, target=np.ascontiguousarray(target),
                t_step=t_step, n_min=n_min, seed=int(seed), iteration=iteration)


def make_workload(cfg: Config, iteration: int = 0, anchor: Optional[np.ndarray] = None, progress=None) -> dict:
    w = make_weights(cfg)
    w.update(make_inputs(cfg, iteration, anchor, progress))
    w["cfg"] = cfg
    return w


def small_config(B: int, gamma: int, V: int, r: int, d: int, dtype: str = "bf16",
                 sampling: str = "greedy", cid: int = 100, plant=(9.0, 5.0),
                 p_target=(0.9, 0.7), sps=("linear", 1.0, 0.01)) -> Config:
    """Ad-hoc shape with the same value recipe (for parity cases that span
    several tiles and ragged tails at sizes the oracle finishes quickly)."""
    return Config(cid, f"custom-{B}x{gamma}x{V}x{r}x{d}-{dtype}", B, gamma, V, r, d, dtype,
                  plant, p_target, sps, sampling=sampling)


# ----------------------------------------------------------------------------
# Calibration sets for fitting the sequential temperatures
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class STSConfig:
    cid: int
    name: str
    N: int                      # calibration blocks
    gamma: int                  # draft positions per block
    G: int                      # candidate temperatures (geometric grid)
    n_bins: int                 # calibration-error bins
    mu: tuple = (3.5, 1.0)      # mean raw confidence logit at k = 1 and k = gamma
    sd: float = 2.0             # its standard deviation
    t_true: tuple = (1.4, 2.6)  # temperature of the acceptance process, k = 1 and k = gamma
    grid: tuple = (0.25, 8.0)   # first and last candidate temperature

    def replace(self, **kw) -> "STSConfig":
        return dataclasses.replace(self, **kw)


STS_WORKLOADS = {
    0: STSConfig(200, "sts-small", 3000, 4, 24, 15),
    1: STSConfig(201, "sts-calibration-256k", 262144, 16, 128, 15),
}


def make_sts_calibration(cfg: STSConfig) -> dict:
    """Synthetic calibration set: raw confidence logits and accepted lengths.

    logit[n][k-1] ~ N(mu_k, sd^2) in fp32 (mu linear in k).  Acceptance is a
    strict prefix process: draft k of block n is accepted, given drafts
    1..k-1 were, when logit/t_true_k + L > 0 for a standard logistic L, i.e.
    with probability sigmoid(logit / t_true_k); accepted[n] counts the leading
    accepted drafts.  t_true > 1 makes the raw scores overconfident.  The
    candidate temperatures are a geometric fp32 grid.
    """
    N, g = cfg.N, cfg.gamma
    mu = linear_in_k(cfg.mu[0], cfg.mu[1], g).astype(np.float32)
    t_true = linear_in_k(cfg.t_true[0], cfg.t_true[1], g)
    logit = (_rng(cfg, _TAG_STS_LOGIT).standard_normal((N, g), dtype=np.float32) * np.float32(cfg.sd)
             + mu[None, :]).astype(np.float32)
    noise = _rng(cfg, _TAG_STS_NOISE).logistic(size=(N, g))
    ok = logit.astype(np.float64) / t_true[None, :] + noise > 0.0
    accepted = np.cumprod(ok, axis=1).sum(axis=1).astype(np.int32)
    grid = np.geomspace(cfg.grid[0], cfg.grid[1], cfg.G).astype(np.float32)
    return dict(logit=np.ascontiguousarray(logit), accepted=accepted, grid=grid,
                n_bins=cfg.n_bins, t_true=t_true, cfg=cfg)
