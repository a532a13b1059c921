"""CPU oracle for the DSpark Markov-head draft, prefix scheduler and verify
step, parallel-only drafting and the sequential-temperature fit.

TEST INFRASTRUCTURE.  Only the tests, the package entry's smoke check and the
benchmark's CPU-baseline leg may import this module.  The library never does:
it shares no code, table or helper with the HIP path.

Plain, slow and written to be checked against the pages by eye: numpy in fp64,
one vocabulary-wide matrix product per draft step (a library primitive), no
blocking or fusion.  Where a floating-point value decides an integer (the
argmax that picks a draft token) the decision is taken on the value rounded to
fp32, the precision the GPU kernel decides in.

Pages cited (titles and sections only):
  [P-blog]  "DSpark: DeepSeek's new speculative decoding work (Video + Blog)"
  [P-wisp]  "DSpark: Overcoming the Efficiency Wall in LLM Speculative Decoding"
  [P-news]  "DeepSeek's DSpark just fixed the two things that held back faster
             AI inference"

Readings taken where the pages are silent or garbled are listed in the
repository's design notes; the ones that matter for a function are restated in
its docstring.  Every function here is pinned by a "not gpu" test against
something other than itself (explicit V x V matrix, textbook routines, brute
force, closed forms, published Philox known-answer vectors, statistics).
"""
from __future__ import annotations

import math
from typing import Callable, Optional

import numpy as np

TWO32 = float(2 ** 32)


# ----------------------------------------------------------------------------
# storage decoding
# ----------------------------------------------------------------------------
def widen(a: np.ndarray) -> np.ndarray:
    """Exact fp64 value of a stored tensor: uint16 arrays hold bfloat16 bit
    patterns (sign, 8-bit exponent, 7-bit mantissa: the top half of an fp32),
    float32 arrays are widened as is."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    raise TypeError(f"unsupported storage dtype {a.dtype}")


# ----------------------------------------------------------------------------
# Philox4x32-10 and Gumbel noise (stochastic drafting)
# ----------------------------------------------------------------------------
_PHILOX_M0 = 0xD2511F53
_PHILOX_M1 = 0xCD9E8D57
_PHILOX_W0 = 0x9E3779B9
_PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random
    numbers: as easy as 1, 2, 3", SC'11, section on the Philox family).

    One round maps the counter (c0, c1, c2, c3) under key (k0, k1) to
    (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)) where
    hi/lo are the upper/lower 32 bits of the 64-bit product; between rounds
    the key is advanced by the Weyl constants (W0, W1).  Arrays broadcast.
    Returns four uint32 arrays."""
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & _MASK32 for x in (c0, c1, c2, c3))
    k0 = np.uint64(int(k0) & 0xFFFFFFFF)
    k1 = np.uint64(int(k1) & 0xFFFFFFFF)
    m0, m1 = np.uint64(_PHILOX_M0), np.uint64(_PHILOX_M1)
    for rnd in range(10):
        if rnd:
            k0 = np.uint64((int(k0) + _PHILOX_W0) & 0xFFFFFFFF)
            k1 = np.uint64((int(k1) + _PHILOX_W1) & 0xFFFFFFFF)
        p0 = m0 * c0
        p1 = m1 * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & _MASK32,
                          (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & _MASK32)
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def gumbel_uniform_bits(seed: int, b, k: int, v):
    """Raw 32-bit hash word for (seed, request b (0-based), position k
    (1-based), vocabulary id v (0-based)).

    Reading: counter = (v >> 2, k, b, 0), key = (low, high 32 bits of seed),
    and the word used is output word (v & 3), so one Philox evaluation serves
    four neighbouring vocabulary ids."""
    v = np.asarray(v, dtype=np.int64)
    b = np.asarray(b, dtype=np.int64)
    words = philox4x32_10(v >> 2, np.full_like(v, k), b, np.zeros_like(v),
                          seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    sel = (v & 3).astype(np.int64)
    w = np.choose(sel, words)
    return w.astype(np.uint32)


def gumbel_noise(seed: int, b, k: int, v) -> np.ndarray:
    """G = -ln(-ln u) with u = (2*(word >> 9) + 1) * 2^-24, an odd multiple of
    2^-24 in (0, 1) (exact in fp32).  Evaluated in fp64, rounded to fp32."""
    w = gumbel_uniform_bits(seed, b, k, v).astype(np.float64)
    u = (np.floor(w / 512.0) * 2.0 + 1.0) * 2.0 ** -24
    return (-np.log(-np.log(u))).astype(np.float32)


# ----------------------------------------------------------------------------
# Draft: Markov head + confidence head + STS + prefix survival
# ----------------------------------------------------------------------------
def sigmoid64(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def bf16_round(x32: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bfloat16 (ties to even), returned as
    uint16 bit patterns: add 0x7FFF plus the lowest kept bit to the fp32 bit
    pattern and keep the top 16 bits (finite inputs)."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)).astype(np.uint16)


def rnn_state_step(s_prev_bits: np.ndarray, decay: np.ndarray, e_bits: np.ndarray) -> np.ndarray:
    """One step of the RNN head's recurrent state (reading of [P-blog] §4
    "Two instantiations of the sequential block", RNN head: its state carries
    every earlier position of the draft block; the pages give no equations).  Per rank channel j:

        s_k[j] = bf16( fp32( fp32(a[j] * s_{k-1}[j]) + e_k[j] ) )

    with e_k = W1[x_{k-1}] the embedding of the previous draft token, a the
    per-channel decay (fp32, an input), s_0 = 0 and the state stored in bf16.
    The product and the sum are separate fp32 operations (each rounded to
    nearest).  a = 0 gives s_k = e_k, the Markov head; a = 1 sums the
    embeddings of x_0 .. x_{k-1}.  bf16 inputs and output as uint16 bits."""
    sp = widen(s_prev_bits).astype(np.float32)
    e = widen(e_bits).astype(np.float32)
    a = np.asarray(decay, dtype=np.float32)
    t = (a * sp).astype(np.float32)
    u = (t + e).astype(np.float32)
    return bf16_round(u)


def draft(anchor, U, h, W1, W2, conf_w, conf_b, sts_T, sampling: str = "greedy",
          seed: int = 0, rows=None, choose: Optional[Callable] = None,
          trace: Optional[list] = None, decay=None):
    """Semi-autoregressive drafting with the Markov head (decay None) or the
    RNN head (decay = the per-channel decay a of rnn_state_step; bf16
    storage only).

    For each request b (rows of the batch; every request's chain is
    independent) and each draft position k = 1..gamma:

    1. Gather e = W1[x_{k-1}], the Markov embedding of the previous draft
       token, with x_0 the anchor ([P-blog] §4, "Two instantiations of the
       sequential block", Markov head: W1 is an embedding lookup table; the
       anchor is the first prediction position, §4 parallel stage).
    2. Transition bias row B(x_{k-1}, .) = e @ W2, the low-rank factorisation
       B = W1 W2 of the first-order V x V transition ([P-blog] §4 Markov head;
       [P-news] "How DSpark combines the best of both worlds").
    3. Logits z_k = U_k + bias, U_k the backbone's base logits at position k
       ([P-blog] §4 sequential stage).  Computed in fp64, rounded to fp32.
    4. Draft token x_k = the lowest vocabulary id with the largest score, the
       score being z_k (greedy) or z_k + G(seed, b, k, v) in fp32 (Gumbel-max
       sampling from softmax(z_k)).  Reading: the pages lose the formula of
       the drafting distribution; p_k(v) is taken proportional to exp(z_k(v)).
    5. Confidence c_k = sigmoid((w . [h_k ; e] + b) / T_k): a linear
       projection of the backbone hidden state at k and the Markov embedding
       of the previous draft token, then a sigmoid ([P-blog] §5), with the
       sequential temperature T_k dividing the whole pre-sigmoid value
       ([P-blog] §5 "Sequential Temperature Scaling"; [P-wisp] "Critical
       Insights").  The dot product is accumulated in fp64; c_k is rounded to
       fp32.
    6. Prefix survival S_k = S_{k-1} * c_k with S_0 = 1, one fp32 multiply
       ([P-blog] §5 "cumulative product"; [P-news] "strict prefix-matching
       survival process").

    `choose(k, rows, s, x)` may replace the oracle's token choice at step k
    (s: fp32 scores [n, V], x: the oracle's argmax); the chain continues from
    whatever it returns.  `trace`, if a list, receives per-step dicts with the
    fp64 logits and the gathered embeddings.

    RNN head ([P-blog] §4 sequential stage: the transition bias
    B_k(x_0, x_{<k}, x_k) may depend on the whole prefix): steps 2-3 use the
    recurrent state s_k of rnn_state_step in place of e, bias = s_k @ W2 (the
    same logits projection); the confidence head keeps the Markov embedding e
    of the previous draft token as its input ([P-blog] §5 names that input).

    Returns (tokens int32 [n, gamma], zsel fp32 [n, gamma], conf fp32,
    surv fp32), zsel being the unperturbed logit z_k(x_k).
    """
    U = np.asarray(U)
    B, gamma, V = U.shape
    r = W1.shape[1]
    d = h.shape[2]
    rows = np.arange(B) if rows is None else np.asarray(rows, dtype=np.int64)
    n = rows.size
    W2f = widen(W2)
    wf = np.asarray(conf_w, dtype=np.float32).astype(np.float64)
    w_h, w_e = wf[:d], wf[d:d + r]
    T = np.asarray(sts_T, dtype=np.float32).astype(np.float64)
    tokens = np.zeros((n, gamma), dtype=np.int32)
    zsel = np.zeros((n, gamma), dtype=np.float32)
    conf = np.zeros((n, gamma), dtype=np.float32)
    surv = np.zeros((n, gamma), dtype=np.float32)
    x_prev = np.asarray(anchor, dtype=np.int64)[rows]
    S = np.ones(n, dtype=np.float32)
    vv = np.arange(V, dtype=np.int64)
    ar = np.arange(n)
    if decay is not None:
        if np.asarray(W1).dtype != np.uint16:
            raise TypeError("the RNN head is defined for bf16 storage")
        state = np.zeros((n, r), dtype=np.uint16)               # s_0 = 0
    for k in range(1, gamma + 1):
        e = widen(W1[x_prev])                                   # step 1
        if decay is None:
            q = e
        else:
            state = rnn_state_step(state, decay, W1[x_prev])
            q = widen(state)
        z64 = widen(U[rows, k - 1]) + q @ W2f                   # steps 2-3
        z = z64.astype(np.float32)
        if sampling == "greedy":
            s = z
        elif sampling == "gumbel":
            G = gumbel_noise(seed, rows[:, None], k, vv[None, :])
            s = z + G                                           # fp32 add
        else:
            raise ValueError(sampling)
        x = np.argmax(s, axis=1)                                # step 4 (first max)
        if choose is not None:
            x = np.asarray(choose(k, rows, s, x), dtype=np.int64)
        ell = conf_b + (widen(h[rows, k - 1]) @ w_h + e @ w_e)  # step 5
        c = sigmoid64(ell / T[k - 1]).astype(np.float32)
        S = (S * c).astype(np.float32)                          # step 6
        tokens[:, k - 1] = x
        zsel[:, k - 1] = z[ar, x]
        conf[:, k - 1] = c
        surv[:, k - 1] = S
        if trace is not None:
            trace.append(dict(k=k, z64=z64, z=z, s=s, e=e, q=q, ell=ell, x_prev=x_prev.copy()))
        x_prev = x
    return tokens, zsel, conf, surv


# ----------------------------------------------------------------------------
# Parallel-only drafting (the baseline without a sequential head)
# ----------------------------------------------------------------------------
def parallel_draft(U, sampling: str = "greedy", seed: int = 0, rows=None):
    """Drafting with the parallel stage alone: every position's token comes
    from its own base logits, with no transition bias and no dependence on
    the earlier draft tokens ([P-blog] §1 "Autoregressive vs Parallel
    Drafting", the parallel drafters that emit logits for all positions in
    one pass; §4 "Semi-Autoregressive Generation", parallel stage, U_k; §2
    "Speedup formula": the sequential head is the lever on acceptance, paid
    for in drafting time).

    For each request b and k = 1..gamma: z_k = U_k (exact in fp32 for bf16 or
    fp32 storage); x_k = the lowest vocabulary id with the largest score,
    the score being z_k (greedy) or z_k + G(seed, b, k, v) in fp32, with the
    same Gumbel noise as the Markov-head draft.  Reading: the baseline is the
    Markov-head step with the transition bias removed, so the tokens are those
    of draft() with W2 = 0; it drafts only (no confidence head).

    Returns (tokens int32 [n, gamma], zsel fp32 [n, gamma]), zsel = z_k(x_k).
    """
    U = np.asarray(U)
    B, gamma, V = U.shape
    rows = np.arange(B) if rows is None else np.asarray(rows, dtype=np.int64)
    n = rows.size
    tokens = np.zeros((n, gamma), dtype=np.int32)
    zsel = np.zeros((n, gamma), dtype=np.float32)
    vv = np.arange(V, dtype=np.int64)
    ar = np.arange(n)
    for k in range(1, gamma + 1):
        z = widen(U[rows, k - 1]).astype(np.float32)
        if sampling == "greedy":
            s = z
        elif sampling == "gumbel":
            s = z + gumbel_noise(seed, rows[:, None], k, vv[None, :])
        else:
            raise ValueError(sampling)
        x = np.argmax(s, axis=1)                                 # first max
        tokens[:, k - 1] = x
        zsel[:, k - 1] = z[ar, x]
    return tokens, zsel


# ----------------------------------------------------------------------------
# Hardware-aware prefix scheduler
# ----------------------------------------------------------------------------
def schedule(surv, t_step, n_min: int):
    """Global throughput maximisation over per-request verify lengths
    ([P-wisp] "2. The Hardware-Aware Prefix Scheduler"; [P-blog] §6; [P-news]
    "Confidence-scheduled verification").

    Objective (reading): every request commits one token from its verify pass
    whatever happens (the correction or bonus token), and its expected number
    of accepted drafts is the sum of its prefix survivals over the verified
    positions.  With n = B + M tokens in the verify step (each request's
    anchor plus M scheduled drafts) and t_step[n - n_min] the step cost,
    maximise  Phi(l) = (B + sum_i sum_{k <= l_i} S_{i,k}) / t_step(B + sum_i l_i)
    over all l in {0..gamma}^B.

    Survival is non-increasing along each request, so for every total M the
    best set is the M largest gains, and that set is prefix-closed: ranking
    all (i, k) by (S desc, i asc, k asc) and taking the top M is optimal.
    Numerics (reading): gains are fixed point g = rint(S * 2^32) (ties to
    even), sums are exact int64, and Phi(M) is one IEEE fp64 division of
    (B * 2^32 + sum of the top-M gains) by t_step.  M* is the smallest M
    attaining the largest Phi; M ranges over 0..min(B*gamma, n_max - B).

    Returns (lens int32 [B], M*, objective = Phi(M*) / 2^32).
    """
    surv = np.asarray(surv, dtype=np.float32)
    B, gamma = surv.shape
    t_step = np.asarray(t_step, dtype=np.float64)
    if n_min > B or n_min + t_step.size - 1 < B:
        raise ValueError("step-cost table must cover n = B")
    m_max = min(B * gamma, n_min + t_step.size - 1 - B)
    S = surv.reshape(-1).astype(np.float64)
    flat = np.arange(B * gamma)
    order = np.lexsort((flat, -S))          # primary: S descending; then flat id
    gains = np.rint(S * TWO32).astype(np.int64)
    G = np.zeros(m_max + 1, dtype=np.int64)
    G[1:] = np.cumsum(gains[order[:m_max]])
    num = (np.int64(B) * np.int64(2 ** 32) + G).astype(np.float64)
    phi = num / t_step[B + np.arange(m_max + 1) - n_min]
    m_star = int(np.argmax(phi))            # first occurrence: smallest M
    lens = np.bincount(order[:m_star] // gamma, minlength=B).astype(np.int32)
    return lens, m_star, float(phi[m_star]) / TWO32


def schedule_threshold(surv, tau: float):
    """Static confidence threshold: the baseline the hardware-aware scheduler
    replaces ([P-blog] §6 "Hardware-Aware Prefix Scheduler": existing work
    verifies by a fixed confidence threshold; [P-news] "Confidence-scheduled
    verification": offline threshold sweeps).

    Reading: a request verifies the longest prefix of its drafts whose prefix
    survival S_k is at least tau (compared in fp32); the threshold ignores
    the batch and the step cost.  Returns (lens int32 [B], M = sum of lens)."""
    S = np.asarray(surv, dtype=np.float32)
    ok = S >= np.float32(tau)
    lens = np.cumprod(ok, axis=1).sum(axis=1).astype(np.int32)
    return lens, int(lens.sum())


SERVE_POLICIES = ("global", "global_delayed2", "threshold")


def serve(weights: dict, iters: list, anchor0, t_step, n_min: int, policy: str = "global", tau: float = 0.5,
          sampling: str = "greedy"):
    """Several drafting iterations of one batch chained as in serving: the
    target's bonus token of iteration t is the anchor (first prediction
    position) of iteration t + 1 ([P-blog] §3 "Speculative decoding" loop;
    §4 parallel stage).  Each iteration drafts, schedules and verifies.

    Policies for the verify lengths:
      global          - the hardware-aware scheduler on this iteration's survivals;
      global_delayed2 - the same scheduler on the survivals of iteration t - 2
                        (scheduling from predictions two steps old, so the
                        decision never waits for the current draft: [P-wisp]
                        "Key Takeaways", asynchrony); iterations 0 and 1 use
                        their own survivals (reading: no older predictions);
      threshold       - schedule_threshold on this iteration's survivals.
    `iters[t]` holds U, h, target and seed of iteration t.  Returns a dict of
    per-iteration arrays (tokens, logit, conf, surv, lens, M, accepted,
    bonus)."""
    if policy not in SERVE_POLICIES:
        raise ValueError(policy)
    anchor = np.asarray(anchor0, dtype=np.int32)
    out = {k: [] for k in ("tokens", "logit", "conf", "surv", "lens", "M", "accepted", "bonus")}
    for t, it in enumerate(iters):
        tok, zs, conf, surv = draft(anchor, it["U"], it["h"], weights["W1"], weights["W2"], weights["conf_w"],
                                   weights["conf_b"], weights["sts_T"], sampling=sampling, seed=it["seed"])
        if policy == "threshold":
            lens, M = schedule_threshold(surv, tau)
        else:
            src = out["surv"][t - 2] if (policy == "global_delayed2" and t >= 2) else surv
            lens, M, _ = schedule(src, t_step, n_min)
        acc, bonus = verify(tok, it["target"], lens)
        for k, v in (("tokens", tok), ("logit", zs), ("conf", conf), ("surv", surv), ("lens", lens), ("M", M),
                     ("accepted", acc), ("bonus", bonus)):
            out[k].append(v)
        anchor = bonus
    return {k: np.asarray(v) for k, v in out.items()}


# ----------------------------------------------------------------------------
# Verification
# ----------------------------------------------------------------------------
def verify(tokens, target, lens):
    """Strict prefix match ([P-news] opening: the drafts are kept up to the
    first one the target disagrees with, which is discarded together with all
    later drafts; [P-blog] §3: the
    target verifies the scheduled prefix).

    accepted_b = number of leading scheduled drafts equal to the target's
    tokens (scan left to right, stop at the first mismatch or at lens_b);
    bonus_b = target[b][accepted_b], the target's own token at the first
    rejected position, or after the last verified one.  Reading: exact token
    match in every sampling mode."""
    tokens = np.asarray(tokens)
    target = np.asarray(target)
    B = tokens.shape[0]
    accepted = np.zeros(B, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    for b in range(B):
        a = 0
        while a < int(lens[b]) and int(tokens[b, a]) == int(target[b, a]):
            a += 1
        accepted[b] = a
        bonus[b] = target[b, a]
    return accepted, bonus


# ----------------------------------------------------------------------------
# Sequential temperature scaling: fitting the per-position temperatures
# ----------------------------------------------------------------------------
def ece_fixed(p, y, n_bins: int):
    """Expected calibration error of predicted probabilities p against 0/1
    labels y: the samples are split into n_bins equal-width bins of p, and
    each bin contributes its share of the samples times the gap between its
    mean label and its mean prediction ([P-blog] §5 "Sequential Temperature
    Scaling" names ECE as the objective; the pages give no bin count or rule).

    Since (n_m / N) |mean y - mean p| = |sum over the bin of (y - p)| / N,
    ECE = sum_m |sum_{n in bin m} (y_n - p_n)| / N.  Readings: bin(p) =
    min(floor(p * n_bins), n_bins - 1), so p = 1 falls in the last bin; each
    residual y - p is rounded to a multiple of 2^-32 (ties to even) and the
    bin sums are exact integers, so comparing two candidates is exact.  The
    last axis of p (and y, broadcast) runs over samples.

    Returns (E, ece): E = sum_m |sum rint((y - p) 2^32)| as int64 per leading
    index, ece = E / (2^32 N), and 0 when there are no samples.

    The bin sums are taken by a weighted histogram in fp64, exact here: every
    residual is an integer of magnitude <= 2^32, so with N <= 2^20 samples
    every partial sum is an integer below 2^53.
    """
    p = np.asarray(p, dtype=np.float64)
    y = np.broadcast_to(np.asarray(y, dtype=np.float64), p.shape)
    N = p.shape[-1]
    if N > 2 ** 20:
        raise ValueError("ece_fixed: more than 2^20 samples")
    lead = p.shape[:-1]
    R = int(np.prod(lead, dtype=np.int64))
    bins = np.minimum(np.floor(p * n_bins), n_bins - 1).astype(np.int64)
    q = np.rint((y - p) * TWO32)                                 # integers, |q| <= 2^32
    key = (np.arange(R, dtype=np.int64).reshape(lead + (1,)) * n_bins + bins).ravel()
    sums = np.bincount(key, weights=q.ravel(), minlength=R * n_bins).reshape(R, n_bins)
    E = np.abs(sums.astype(np.int64)).sum(axis=1).reshape(lead)
    ece = E / (TWO32 * N) if N > 0 else np.zeros(E.shape, dtype=np.float64)
    return E, ece


def sts_fit(logit, accepted, grid, n_bins: int, choose: Optional[Callable] = None,
            g_chunk: int = 16):
    """Sequential temperature scaling fitted left to right ([P-blog] §5
    "Sequential Temperature Scaling"; [P-wisp] "Critical Insights"; [P-news]
    on post-hoc calibration against empirical acceptance).

    logit[n][k-1] is block n's raw confidence logit at draft position k (the
    pre-sigmoid value of the confidence head, bias included, read as fp32);
    accepted[n] is how many leading drafts of block n the target accepted.
    For k = 1..gamma, in order:
      * y_n = 1 when accepted[n] >= k: the survival label, since the
        calibrated quantity is the cumulative product S_k, the probability
        that drafts 1..k are all accepted (reading);
      * for every candidate T of the grid, p_n(T) = S_{n,k-1} sigmoid(logit
        / T), the earlier positions held at their fitted temperatures
        (S_{n,0} = 1; T divides the whole logit, as in the draft step);
      * T_k = the candidate with the smallest ECE of p(T) against y (a 1-D
        grid search); among equal ECE the first in grid order (reading);
      * S_{n,k} = p_n(T_k).
    fp64 throughout; the comparison uses ece_fixed's exact integer sums.

    `choose(k, E, g)` may replace the chosen grid index at position k (E: the
    integer objective per candidate, g: the oracle's choice); the fit goes on
    from whatever it returns.

    Returns (choice int32 [gamma], T fp32 [gamma], ece fp64 [gamma][G]).
    """
    L = widen(np.asarray(logit, dtype=np.float32))
    N, gamma = L.shape
    T_grid = np.asarray(grid, dtype=np.float32)
    Tg = T_grid.astype(np.float64)
    G = Tg.size
    a = np.asarray(accepted, dtype=np.int64)
    S = np.ones(N, dtype=np.float64)
    choice = np.zeros(gamma, dtype=np.int32)
    T_out = np.zeros(gamma, dtype=np.float32)
    ece = np.zeros((gamma, G), dtype=np.float64)
    for k in range(1, gamma + 1):
        y = (a >= k).astype(np.float64)
        E = np.zeros(G, dtype=np.int64)
        for g0 in range(0, G, g_chunk):                         # bounds host memory
            P = S[None, :] * sigmoid64(L[:, k - 1][None, :] / Tg[g0:g0 + g_chunk, None])
            E[g0:g0 + g_chunk], ece[k - 1, g0:g0 + g_chunk] = ece_fixed(P, y, n_bins)
        g = int(np.argmin(E))                                   # first minimum
        if choose is not None:
            g = int(choose(k, E, g))
        choice[k - 1] = g
        T_out[k - 1] = T_grid[g]
        S = S * sigmoid64(L[:, k - 1] / Tg[g])
    return choice, T_out, ece


def draft_workload(w: dict, rows=None, choose=None, trace=None, seed=None, head: str = "markov"):
    """Convenience wrapper over `draft` for a workload dictionary (head
    "markov" or "rnn"; the RNN head takes the workload's decay)."""
    cfg = w["cfg"]
    return draft(w["anchor"], w["U"], w["h"], w["W1"], w["W2"], w["conf_w"], w["conf_b"],
                 w["sts_T"], sampling=cfg.sampling, seed=w["seed"] if seed is None else seed,
                 rows=rows, choose=choose, trace=trace, decay=w["decay"] if head == "rnn" else None)
