"""Benchmark of the DSpark Markov-head draft -> prefix schedule -> verify path
on one MI355X.

Before timing, steps run untimed for 0.2 s (clock ramp-up), then the W
warm-up steps.  One step = one pass of the whole path over one batch: dspark_markov_draft
(gamma dependent Markov-head steps with the confidence epilogue), then
dspark_schedule on the drafted survivals, then dspark_verify against the
target tokens.  Inputs are resident in HBM before timing starts.

Workload: B=256 requests, gamma=16, V=151936, r=256, d=5120, bf16 storage,
greedy drafting, 64-point step-cost table 4 + 0.02 n + 2e-5 n^2 over
n in [256, 4352] (synthetic inputs from the seeded generator).

Prints one JSON line.  `value` = drafted tokens per second of the whole step
(B * gamma / step time), with the drafting kernel in the exclusive launch mode
(a plain launch: the benchmark is the only work on the device; named in
`config.draft_launch`); the step and draft times under the library's default
cooperative launch are reported beside it (`draft_launch`).  The timed
tokens are checked to lie in [0, V) (`outputs_valid`; exit status 3
otherwise).  `schedule_us` / `verify_us` are the device time per call of those
two calls alone (50 calls captured in a graph and replayed);
`schedule_verify_timing` adds the per-call latency as the step issues them
and the scheduler's one-workgroup (no workspace) kernel.  `roofline` rates the draft kernel against HBM
bandwidth with its algorithmic bytes; `cpu_baseline` times the CPU oracle on
a bounded sample of requests of the same workload; `ablation` times
dspark_parallel_draft (drafting without the sequential head) on the same U,
outside the timed step; `sts_fit` times dspark_sts_fit (fitting the 16
confidence temperatures on 262144 synthetic calibration blocks, 128 candidate
temperatures, 15 bins), also outside the step, against the VALU issue rate;
`serve` runs dspark_serve (4 chained iterations of the same batch, anchors
taken from the previous bonus tokens) under each verify-length policy;
`rnn_head` times dspark_rnn_draft (the RNN sequential head) on the same inputs;
`latency_case` times the one-request, gamma = 8 workload (the draft call, and
the whole step as one dspark_step call).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
# VALU issue rate: 256 CUs x 4 SIMDs x 16 lanes per cycle x 2.4 GHz (one fp64
# or fp32 vector op per lane per cycle; 78.6 TFLOP/s fp64 counts an FMA as 2)
VALU_PEAK_GOPS = 256 * 64 * 2.4
# Operations one candidate evaluation of the temperature fit needs: scale by
# 1/T (1); e^x: range reduction (4), degree-13 polynomial (13), scaling (1);
# 1 + e^x (1); reciprocal estimate + two Newton steps (5); p = S sigmoid (1);
# y - p (1); rounding to 2^-32 (2); bin index (3); histogram address (1);
# histogram add (1).
STS_OPS_PER_EVAL = 34
# operations the fit needs per evaluation whatever the implementation, the
# exponential and the reciprocal counted as one each
STS_ALG_OPS_PER_EVAL = 8
SETTLE_S = 0.2   # untimed steps before the warm-up: long enough for the clocks to settle
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
# the draft kernel's device code (the traffic summary is tied to these files)
DRAFT_SOURCES = [os.path.join(ROOT, "semi_ar_drafter_amd", "csrc", f) for f in ("markov_draft.hip", "device_util.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "markov_draft_hbm_traffic.txt")


def source_digest(paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        h.update(open(path, "rb").read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per draft launch from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by the factor a plain copy
    kernel of known size gives), or None if the summary is missing or was
    taken on a different version of the draft kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    try:
        if vals.get("kernel_source_sha256") != source_digest(DRAFT_SOURCES):
            return None
        fetch = float(vals["fetch_kib_per_launch"]) * 1024 * float(vals["fetch_scale"])
        write = float(vals["write_kib_per_launch"]) * 1024 * float(vals["write_scale"])
        return int(round(fetch + write))
    except (KeyError, ValueError):
        return None


GUMBEL_PROFILE = os.path.join(ROOT, "profiles", "markov_draft_cfg4_gumbel.md")


def profiled_valu_fraction():
    """VALU and MFMA fractions of the draft kernel on the large-vocabulary
    Gumbel-max workload, from the committed rocprofv3 counter summary, or
    None if it is missing or was taken on other draft kernel sources."""
    if not os.path.exists(GUMBEL_PROFILE):
        return None
    text = open(GUMBEL_PROFILE).read()
    import re
    sha = re.search(r"kernel_source_sha256: ([0-9a-f]+)", text)
    valu = re.search(r"VALU fraction = .* = ([0-9.]+) %", text)
    mfma = re.search(r"MFMA utilisation = .* = ([0-9.]+) %", text)
    if not (sha and valu and mfma) or sha.group(1) != source_digest(DRAFT_SOURCES):
        return None
    return {"frac": round(float(valu.group(1)) / 100, 4), "mfma_busy_frac": round(float(mfma.group(1)) / 100, 4),
            "definition": "4 x SQ_ACTIVE_INST_VALU (quad-cycles, summed over waves) / (busy cycles x 1024 SIMDs); "
                          "two waves per SIMD, so up to 2",
            "source": "profiles/markov_draft_cfg4_gumbel.md (rocprofv3 counters of the same kernel sources)"}


def copy_calibration(nbytes: int, reps: int):
    """A plain device-to-device copy of known size, for scaling the HBM
    counters (each launch reads and writes `nbytes`)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def algorithmic_bytes(cfg) -> int:
    """Bytes the draft call must move at minimum: every base logit once, W2
    once, one gathered W1 row and one hidden-state row per (request,
    position), the confidence head, temperatures, anchors and the four
    [B, gamma] outputs."""
    e = 2 if cfg.dtype == "bf16" else 4
    B, g, V, r, d = cfg.B, cfg.gamma, cfg.V, cfg.r, cfg.d
    return (B * g * V * e + r * V * e + B * g * r * e + B * g * d * e
            + (d + r) * 4 + g * 4 + B * 4 + B * g * 16)


def flops(cfg) -> int:
    return 2 * cfg.B * cfg.gamma * cfg.r * cfg.V


def cpu_baseline(w, rows: int, min_seconds: float):
    """The oracle as it stands, drafting the first `rows` requests through all
    gamma steps (requests are independent, so the sample is a fixed fraction
    of the call's work), repeated until at least `min_seconds` have passed."""
    import numpy as np
    from oracle import dspark_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    reps = 0
    t0 = time.perf_counter()
    while True:
        orc.draft_workload(w, rows=np.arange(rows))
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    t1 = time.perf_counter()
    return dict(seconds=t1 - t0, tokens=reps * rows * w["cfg"].gamma, threads=threads, reps=reps)


def time_sts_fit(torch, wl, sts_fit, reps: int = 10):
    """Times dspark_sts_fit on the 262144-block calibration set (inputs in HBM)."""
    c = wl.STS_WORKLOADS[1]
    cal = wl.make_sts_calibration(c)
    lo = torch.from_numpy(cal["logit"]).cuda()
    ac = torch.from_numpy(cal["accepted"]).cuda()
    gr = torch.from_numpy(cal["grid"]).cuda()
    out = (torch.empty(c.gamma, dtype=torch.int32, device="cuda"),
           torch.empty(c.gamma, dtype=torch.float32, device="cuda"),
           torch.empty((c.gamma, c.G), dtype=torch.float64, device="cuda"))
    for _ in range(2):
        sts_fit(lo, ac, gr, c.n_bins, out=out)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        sts_fit(lo, ac, gr, c.n_bins, out=out)
        b.record()
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)[reps // 2]
    evals = c.N * c.gamma * c.G
    gops = evals * STS_OPS_PER_EVAL / (us / 1e6) / 1e9
    # the same rate against the operations the fit cannot do without, each
    # counted once (the fp64 exponential and reciprocal as one operation each)
    alg_gops = evals * STS_ALG_OPS_PER_EVAL / (us / 1e6) / 1e9
    return {"workload": f"calibration N={c.N} gamma={c.gamma} G={c.G} bins={c.n_bins}",
            "us_per_fit": round(us, 1), "evals_per_s": round(evals / (us / 1e6), 1),
            "roofline": {"bound": "alu", "achieved": round(gops, 1), "peak": VALU_PEAK_GOPS, "unit": "Gop/s",
                         "frac": round(gops / VALU_PEAK_GOPS, 4), "ops_per_eval": STS_OPS_PER_EVAL,
                         "ops_note": "operations of this implementation (its exponential is 18 of them): frac is "
                                     "the fraction of the VALU issue rate its instruction stream reaches",
                         "algorithmic_ops_per_eval": STS_ALG_OPS_PER_EVAL,
                         "frac_algorithmic": round(alg_gops / VALU_PEAK_GOPS, 4),
                         "algorithmic_note": "scale, exponential, 1 + e, reciprocal, S * sigma, y - p, bin, "
                                             "histogram add: one operation each",
                         "kernel": f"sts_pass_kernel ({c.gamma} launches + 1 clear per fit)"}}


def time_serve(torch, serve, w, anchor, U, h, W1, W2, conf_w, sts_T, target, t_step, mode, seed,
               iters: int = 4, taus=(0.3, 0.5, 0.7), runs_per_policy: int = 20):
    """dspark_serve under each verify-length policy: `iters` chained
    iterations of the benchmark batch (U, h and target repeated on the
    device; the anchors chain through the bonus tokens).  Each policy is
    timed over `runs_per_policy` calls, the policies interleaved call by call
    so that clock drift affects them alike; p10, median and p90 per policy."""
    import numpy as np
    Ur = U.unsqueeze(0).expand(iters, *U.shape).contiguous()
    hr = h.unsqueeze(0).expand(iters, *h.shape).contiguous()
    tr = target.unsqueeze(0).expand(iters, *target.shape).contiguous()
    B = U.shape[0]
    tab = w["t_step"]
    res = {"workload": f"{iters} chained iterations of the benchmark batch (inputs repeated, anchors chained); "
                       f"{runs_per_policy} timed calls per policy, interleaved",
           "note": "on one GPU the delayed policy removes the dependence of the verify lengths on the current "
                   "draft but buys no overlap: the persistent draft kernel occupies every compute unit"}
    runs = [("global", "global", 0.0), ("global_delayed2", "global_delayed2", 0.0)]
    runs += [(f"threshold_{tau}", "threshold", tau) for tau in taus]
    fns = {}
    for label, policy, tau in runs:
        fns[label] = (lambda policy=policy, tau=tau: serve(anchor, Ur, hr, W1, W2, conf_w, w["conf_b"], sts_T, tr,
                                                           t_step, w["n_min"], policy=policy, tau=tau, mode=mode,
                                                           seed=seed))
        fns[label]()
    torch.cuda.synchronize()
    times = {label: [] for label, _, _ in runs}
    outs = {}
    for _ in range(runs_per_policy):
        for label, _, _ in runs:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            outs[label] = fns[label]()
            b.record()
            torch.cuda.synchronize()
            times[label].append(a.elapsed_time(b) * 1e3 / iters)
    for label, _, _ in runs:
        out = outs[label]
        m = out["m"].cpu().numpy().astype(float)
        acc = out["accepted"].cpu().numpy().astype(float)
        committed = acc.sum() + iters * B
        cost = float(sum(tab[B + int(x) - w["n_min"]] for x in m))
        t = np.asarray(times[label])
        res[label] = {"us_per_iteration_p10_p50_p90": [round(float(np.percentile(t, q)), 1) for q in (10, 50, 90)],
                      "verified_drafts_per_iteration": round(m.mean(), 1),
                      "accepted_per_iteration": round(acc.sum() / iters, 1),
                      "acceptance_rate": round(acc.sum() / max(m.sum(), 1.0), 4),
                      "committed_per_iteration": round(committed / iters, 1),
                      "committed_per_cost_unit": round(committed / cost, 3)}
    del Ur, hr, tr
    return res


def time_latency_case(torch, wl, dev, markov_draft, step, reps: int = 3, calls: int = 20):
    """The latency workload (one request, gamma = 8, V = 151936): the draft
    call and the whole step in one dspark_step call (events around `calls`
    back-to-back calls, best of `reps`), inputs resident in HBM."""
    c = wl.WORKLOADS[1]
    w = wl.make_workload(c)
    anchor, U, h, W1, W2 = dev(w["anchor"]), dev(w["U"]), dev(w["h"]), dev(w["W1"]), dev(w["W2"])
    conf_w, sts_T, target, t_step = dev(w["conf_w"]), dev(w["sts_T"]), dev(w["target"]), dev(w["t_step"])
    args = (anchor, U, h, W1, W2, conf_w, w["conf_b"], sts_T)

    def best(fn):
        t = []
        for _ in range(reps):
            for _ in range(3):
                fn()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            for _ in range(calls):
                fn()
            b.record()
            torch.cuda.synchronize()
            t.append(a.elapsed_time(b) * 1e3 / calls)
        return min(t)

    draft_us = best(lambda: markov_draft(*args, mode=c.sampling, seed=w["seed"]))
    step_us = best(lambda: step(*args, target, t_step, w["n_min"], mode=c.sampling, seed=w["seed"]))
    tok = step(*args, target, t_step, w["n_min"], mode=c.sampling, seed=w["seed"])[0].cpu().numpy()
    return {"workload": f"B={c.B} gamma={c.gamma} V={c.V} r={c.r} d={c.d} {c.dtype} {c.sampling}",
            "draft_us": round(draft_us, 2), "step_us": round(step_us, 2),
            "drafted_tokens_per_s": round(c.B * c.gamma / (step_us / 1e6), 1),
            "outputs_valid": bool(((tok >= 0) & (tok < c.V)).all()),
            "note": "batches of at most 16 requests synchronise the draft positions through the workgroups' "
                    "winner keys; the step is one dspark_step call (draft, then schedule and verify)"}


def time_w2_cold(torch, run, reps: int = 10, scratch_bytes: int = 512 << 20):
    """The draft call with W2 (and everything else) evicted from the on-chip
    and memory-side caches first: a 512 MB scratch buffer is streamed (read
    and written) before each timed call.  Median of `reps` calls (events
    around the call only)."""
    import numpy as np
    scratch = torch.empty(scratch_bytes // 4, dtype=torch.float32, device="cuda")
    scratch.fill_(1.0)
    ts = []
    for _ in range(reps):
        scratch.mul_(1.0000001)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    del scratch
    return float(np.median(ts))


def oracle_side_timings(w, single_thread_rows: int):
    """Host time of the oracle's scheduler and verify on the full batch (the
    oracle's own draft outputs as inputs), and, for the small configurations,
    the oracle's draft on one thread."""
    import numpy as np
    from oracle import dspark_oracle as orc
    cfg = w["cfg"]
    rows = np.arange(min(cfg.B, 8))
    tok, _, _, surv = orc.draft_workload(w, rows=rows)
    # a full-size survival / token array from the sample (the schedule and
    # verify costs depend on B * gamma only)
    reps_rows = (np.arange(cfg.B) % rows.size)
    surv_b, tok_b = surv[reps_rows], tok[reps_rows]
    res = {}
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < 0.5:
        lens, _, _ = orc.schedule(surv_b, w["t_step"], w["n_min"])
        n += 1
    res["schedule_ms"] = round((time.perf_counter() - t0) / n * 1e3, 3)
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < 0.5:
        orc.verify(tok_b, w["target"], lens)
        n += 1
    res["verify_ms"] = round((time.perf_counter() - t0) / n * 1e3, 3)
    if single_thread_rows:
        try:
            from threadpoolctl import threadpool_limits
        except Exception:  # pragma: no cover
            return res
        srows = np.arange(min(cfg.B, single_thread_rows))
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            orc.draft_workload(w, rows=srows)
            dt = time.perf_counter() - t0
        res["single_thread_drafted_tokens_per_s"] = round(srows.size * cfg.gamma / dt, 2)
        res["single_thread_sample"] = f"first {srows.size} of {cfg.B} requests, all {cfg.gamma} steps"
    return res


def graph_us(fn, calls: int = 50, reps: int = 5) -> float:
    """Device time per call of `fn` (a library call that allocates nothing):
    `calls` calls captured in one graph, replayed `reps` times, median."""
    import numpy as np
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for _ in range(calls):
            fn()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3 / calls)
    return float(np.median(ts))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, help="workload id (default: the B=256 configuration)")
    ap.add_argument("--cpu-rows", type=int, default=256, help="requests in the CPU-oracle sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum CPU-oracle time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sts", action="store_true", help="skip timing the temperature fit")
    ap.add_argument("--no-serve", action="store_true", help="skip the serving-loop policy comparison")
    ap.add_argument("--draft-launch", choices=("exclusive", "cooperative"), default="exclusive",
                    help="launch mode of the drafting kernel for the timed steps (the other is timed too)")
    ap.add_argument("--no-other-launch", action="store_true",
                    help="do not time the other launch mode (profiled runs use this: only plain launches)")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed step and its roofline (no ablation, RNN head, W2-cold, per-kernel legs)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (for HBM counter scaling) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU only (asked for --gpus {args.gpus}); "
              "see the design notes for how it would shard across GPUs.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from semi_ar_drafter_amd import (markov_draft, parallel_draft, rnn_draft, schedule, schedule_workspace_bytes,
                                     serve, set_draft_launch, sts_fit, verify)
    from semi_ar_drafter_amd import step as dspark_step
    from semi_ar_drafter_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        copy_calibration(args.calibrate_copy, 5)
        return
    cfg = wl.WORKLOADS[args.config]
    t_gen = time.perf_counter()
    w = wl.make_workload(cfg, progress=lambda b: print(f"[bench] generating {cfg.name}: request {b}/{cfg.B}",
                                                         file=sys.stderr, flush=True))
    print(f"[bench] generated {cfg.name} in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    anchor, U, h, W1, W2 = dev(w["anchor"]), dev(w["U"]), dev(w["h"]), dev(w["W1"]), dev(w["W2"])
    conf_w, sts_T, target, t_step = dev(w["conf_w"]), dev(w["sts_T"]), dev(w["target"]), dev(w["t_step"])
    B, g = cfg.B, cfg.gamma
    outs = (torch.empty((B, g), dtype=torch.int32, device="cuda"),
            torch.empty((B, g), dtype=torch.float32, device="cuda"),
            torch.empty((B, g), dtype=torch.float32, device="cuda"),
            torch.empty((B, g), dtype=torch.float32, device="cuda"))
    sched_out = (torch.empty(B, dtype=torch.int32, device="cuda"), torch.empty(1, dtype=torch.int32, device="cuda"),
                 torch.empty(1, dtype=torch.float64, device="cuda"))
    ver_out = (torch.empty(B, dtype=torch.int32, device="cuda"), torch.empty(B, dtype=torch.int32, device="cuda"))
    mode, seed = cfg.sampling, w["seed"]

    def step(ev0=None, ev1=None):
        if ev0 is not None:
            ev0.record()
        tok, logit, conf, surv = markov_draft(anchor, U, h, W1, W2, conf_w, w["conf_b"], sts_T, mode=mode,
                                              seed=seed, out=outs)
        if ev1 is not None:
            ev1.record()
        lens, m, obj = schedule(surv, t_step, w["n_min"], out=sched_out)
        verify(tok, target, lens, out=ver_out)

    # The benchmark is the only work on the device, which is the exclusive
    # launch mode's precondition; the default cooperative launch is timed too.
    set_draft_launch(args.draft_launch)
    # Untimed: run steps for SETTLE_S seconds first (the GPU's clocks ramp up
    # over the first tens of milliseconds of work), then the W warm-up steps.
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(K):
        step(*ev[i])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = start.elapsed_time(stop) / K
    draft_ms = [a.elapsed_time(b) for a, b in ev]
    draft_avg = sum(draft_ms) / K
    value = B * g / (ms_step / 1e3)
    # the timed outputs must be real drafts: a failed grid synchronisation
    # inside the kernel would have marked every token -1
    tok_chk = outs[0].cpu().numpy()
    outputs_valid = bool(((tok_chk >= 0) & (tok_chk < cfg.V)).all())
    if not outputs_valid:
        print("bench.py: the timed draft returned tokens outside [0, V) "
              "(a failed in-kernel synchronisation); the measurement is invalid", file=sys.stderr)
    other = "cooperative" if args.draft_launch == "exclusive" else "exclusive"
    other_ms = other_draft_us = None
    if not args.no_other_launch:
        set_draft_launch(other)
        for _ in range(2):
            step()
        oev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        o0, o1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        o0.record()
        for i in range(K):
            step(*oev[i])
        o1.record()
        torch.cuda.synchronize()
        other_ms = o0.elapsed_time(o1) / K
        other_draft_us = sum(a.elapsed_time(b) for a, b in oev) / K * 1e3
        set_draft_launch(args.draft_launch)

    # Latency of the scheduler and verify calls: events around each call as
    # the step issues it (includes the host-side launch of a small kernel),
    # and the device time per call with 50 calls captured in a graph and
    # replayed (launch overhead of the device alone; both kernels allocate
    # nothing, clear nothing with memset and leave their workspace as found).
    sv = []
    for _ in range(20):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        lens, m, obj = schedule(outs[3], t_step, w["n_min"], out=sched_out)
        e[1].record()
        verify(outs[0], target, lens, out=ver_out)
        e[2].record()
        sv.append(e)
    torch.cuda.synchronize()
    sched_call_us = float(np.median([a.elapsed_time(b) * 1e3 for a, b, _ in sv]))
    verify_call_us = float(np.median([b.elapsed_time(c) * 1e3 for _, b, c in sv]))
    sched_ws = torch.zeros(schedule_workspace_bytes(B, g), dtype=torch.uint8, device="cuda")
    sched_us = graph_us(lambda: schedule(outs[3], t_step, w["n_min"], out=sched_out, workspace=sched_ws))
    sched_1wg_us = graph_us(lambda: schedule(outs[3], t_step, w["n_min"], out=sched_out, one_workgroup=True))
    verify_us = graph_us(lambda: verify(outs[0], target, sched_out[0], out=ver_out))

    u_bytes = B * g * cfg.V * (2 if cfg.dtype == "bf16" else 4)
    par_us = rnn_us = w2_cold_us = None
    if not args.no_extras:
        # Ablation, outside the timed step: drafting with the parallel stage
        # alone (no sequential head) on the same U, to show what the Markov
        # head costs.
        p_out = (torch.empty((B, g), dtype=torch.int32, device="cuda"),
                 torch.empty((B, g), dtype=torch.float32, device="cuda"))
        for _ in range(2):
            parallel_draft(U, mode=mode, seed=seed, out=p_out)
        pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        for a, b in pev:
            a.record()
            parallel_draft(U, mode=mode, seed=seed, out=p_out)
            b.record()
        torch.cuda.synchronize()
        par_us = sum(a.elapsed_time(b) for a, b in pev) / len(pev) * 1e3

        # The RNN sequential head on the same inputs, outside the timed step
        # (the RNN head is built for bf16 storage).
        if cfg.dtype == "bf16":
            decay = dev(w["decay"])
            r_out = tuple(torch.empty((B, g), dtype=t, device="cuda")
                          for t in (torch.int32, torch.float32, torch.float32, torch.float32))
            for _ in range(2):
                rnn_draft(anchor, U, h, W1, W2, decay, conf_w, w["conf_b"], sts_T, mode=mode, seed=seed, out=r_out)
            rev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
            for a, b in rev:
                a.record()
                rnn_draft(anchor, U, h, W1, W2, decay, conf_w, w["conf_b"], sts_T, mode=mode, seed=seed, out=r_out)
                b.record()
            torch.cuda.synchronize()
            rnn_us = sum(a.elapsed_time(b) for a, b in rev) / len(rev) * 1e3

        # W2 cold: the draft call after a 512 MB stream has evicted W2 from the caches
        w2_cold_us = time_w2_cold(torch, lambda: markov_draft(anchor, U, h, W1, W2, conf_w, w["conf_b"], sts_T,
                                                              mode=mode, seed=seed, out=outs))

    abytes = algorithmic_bytes(cfg)
    achieved = abytes / (draft_avg / 1e3) / 1e9
    tflops = flops(cfg) / (draft_avg / 1e3) / 1e12
    print(f"[bench] step {ms_step * 1e3:.1f} us, draft {draft_avg * 1e3:.1f} us "
          f"(min {min(draft_ms) * 1e3:.1f}), {achieved:.0f} GB/s algorithmic, {tflops:.0f} TFLOP/s, "
          f"schedule {sched_us:.1f} us, verify {verify_us:.1f} us, wall {wall:.3f}s", file=sys.stderr, flush=True)

    launch_note = ("exclusive = a plain launch whose grid barrier relies on the caller's promise that nothing "
                   "else runs on the device (the benchmark is the only work on it); cooperative = the runtime's "
                   "co-residency guarantee, the library's default")
    sps = (f"64-point 4+0.02n+2e-5n^2, n in [{B}, {B + B * g}]" if args.config >= 3
           else f"1+0.01n, n in [{B}, {B + B * g}]")
    result = {
        "metric": f"drafted tokens/s at V={cfg.V} r={cfg.r} \u03b3={g} B={B}; % of HBM roofline",
        "value": round(value, 1),
        "unit": "drafted tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": "markov-draft+schedule+verify", "B": B, "gamma": g, "V": cfg.V, "r": cfg.r,
                   "d": cfg.d, "storage": cfg.dtype, "sampling": cfg.sampling, "sps_table": sps,
                   "draft_launch": args.draft_launch},
        "outputs_valid": outputs_valid,
        "draft_launch": {"mode": args.draft_launch, "note": launch_note},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic() if args.config == 3 else None,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-kernel scaled)",
                     "kernel": "markov_draft_kernel (one launch per dspark_markov_draft call)",
                     "algorithmic_bytes_per_launch": abytes, "launch_us": round(draft_avg * 1e3, 2),
                     "launch_us_p10_p50_p90": [round(float(np.percentile(draft_ms, q)) * 1e3, 2) for q in (10, 50, 90)],
                     "u_stream_gbs": round(u_bytes / (draft_avg / 1e3) / 1e9, 1)},
        "mfma": {"achieved_tflops": round(tflops, 1), "peak_tflops": BF16_PEAK_TFLOPS,
                 "frac": round(tflops / BF16_PEAK_TFLOPS, 4)},
        "schedule_us": round(sched_us, 2),
        "verify_us": round(verify_us, 2),
        "schedule_verify_timing": {
            "note": "schedule_us / verify_us: device time per call, 50 calls captured in a graph and replayed; "
                    "*_call_us: events around one call as the step issues it (adds the host-side launch)",
            "schedule_call_us": round(sched_call_us, 2), "verify_call_us": round(verify_call_us, 2),
            "schedule_one_workgroup_us": round(sched_1wg_us, 2)},
        "cpu_baseline": None,
    }
    if args.config == 4:
        valu = profiled_valu_fraction()
        if valu is not None:
            result["valu"] = valu
    if other_ms is not None:
        result["draft_launch"].update({f"{other}_ms_per_step": round(other_ms, 5),
                                       f"{other}_draft_us": round(other_draft_us, 2)})
    if par_us is not None:
        result["roofline"]["frac_of_measured_stream"] = round(achieved / (u_bytes / (par_us / 1e6) / 1e9), 4)
        result["roofline"]["measured_stream_note"] = ("the parallel-only draft kernel (a streaming read of U "
                                                      "with an argmax) on the same U, taken as the measured "
                                                      "streaming-read rate")
        result["ablation"] = {"parallel_only_us": round(par_us, 2),
                              "parallel_only_gbs": round(u_bytes / (par_us / 1e6) / 1e9, 1),
                              "markov_head_marginal_us": round(draft_avg * 1e3 - par_us, 2),
                              "note": "dspark_parallel_draft on the same U (no transition bias, no confidence), "
                                      "timed separately from the step"}
    if w2_cold_us is not None:
        result["w2_cold"] = {"draft_us": round(w2_cold_us, 2),
                             "hbm_frac": round(abytes / (w2_cold_us / 1e6) / 1e9 / HBM_PEAK_GBS, 4),
                             "note": "a 512 MB buffer streamed before each timed call (W2 evicted); "
                                     "W2 counted once per call in both; the headline is W2 warm (resident from "
                                     "the previous call, the serving steady state)"}
    if rnn_us is not None:
        # RNN head: the Markov head's bytes plus the recurrent state (read
        # and written once per step) and the decay vector
        rbytes = abytes + 2 * B * g * cfg.r * 2 + cfg.r * 4
        result["rnn_head"] = {"us_per_call": round(rnn_us, 2),
                              "drafted_tokens_per_s": round(B * g / (rnn_us / 1e6), 1),
                              "hbm_frac": round(rbytes / (rnn_us / 1e6) / 1e9 / HBM_PEAK_GBS, 4),
                              "marginal_us_vs_markov": round(rnn_us - draft_avg * 1e3, 2),
                              "note": "dspark_rnn_draft (per-channel decayed recurrent state) on the same inputs, "
                                      "timed separately from the step"}
    if not args.no_extras and args.config == 3:
        result["latency_case"] = time_latency_case(torch, wl, dev, markov_draft, dspark_step)
    if not args.no_sts:
        result["sts_fit"] = time_sts_fit(torch, wl, sts_fit)
    if not args.no_serve:
        result["serve"] = time_serve(torch, serve, w, anchor, U, h, W1, W2, conf_w, sts_T, target, t_step, mode, seed)
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, min(args.cpu_rows, B), args.cpu_seconds)
        result["cpu_baseline"] = {"value": round(cb["tokens"] / cb["seconds"], 2), "unit": "drafted tokens/s",
                                  "cores": cb["threads"], "kind": "oracle",
                                  "sample": f"{cb['reps']} x first {min(args.cpu_rows, B)} of {B} requests, all "
                                            f"{g} draft steps ({cb['seconds']:.1f}s; host reports "
                                            f"{os.cpu_count()} CPUs)"}
        result["cpu_baseline"].update(oracle_side_timings(w, single_thread_rows=4 if args.config <= 2 else 0))
    print(json.dumps(result), flush=True)
    if not outputs_valid:
        sys.exit(3)


if __name__ == "__main__":
    main()
