"""Parity helpers: device transfer of seeded workloads and the comparison
rule between the HIP path and the CPU oracle.

Rule: token ids, scheduled lengths, M* and verify outputs are bit-exact.
Logits agree within 1e-2 absolute, confidences and survivals within 1e-4
absolute.  Single exception: at a (request, position) where the oracle's
top-2 score gap is below 2e-2, a different GPU token is accepted if the
oracle's score of it is within 2e-2 of the maximum; the oracle then
continues its chain from the GPU's token ("replay").
"""
from __future__ import annotations

import dataclasses

import numpy as np

TIE_TOL = 2e-2
LOGIT_TOL = 1e-2
CONF_TOL = 1e-4


def to_device(w: dict, device="cuda:0") -> dict:
    import torch
    cfg = w["cfg"]

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    return dict(anchor=dev(w["anchor"]), U=dev(w["U"]), h=dev(w["h"]), W1=dev(w["W1"]), W2=dev(w["W2"]),
                conf_w=dev(w["conf_w"]), sts_T=dev(w["sts_T"]), target=dev(w["target"]),
                t_step=dev(w["t_step"]), conf_b=float(w["conf_b"]), n_min=int(w["n_min"]),
                seed=int(w["seed"]), mode=cfg.sampling, decay=dev(w["decay"]))


def gpu_draft(d: dict):
    import torch
    from semi_ar_drafter_amd import markov_draft
    out = markov_draft(d["anchor"], d["U"], d["h"], d["W1"], d["W2"], d["conf_w"], d["conf_b"], d["sts_T"],
                       mode=d["mode"], seed=d["seed"])
    torch.cuda.synchronize()
    return tuple(x.cpu().numpy() for x in out)


def gpu_rnn_draft(d: dict):
    import torch
    from semi_ar_drafter_amd import rnn_draft
    out = rnn_draft(d["anchor"], d["U"], d["h"], d["W1"], d["W2"], d["decay"], d["conf_w"], d["conf_b"], d["sts_T"],
                    mode=d["mode"], seed=d["seed"])
    torch.cuda.synchronize()
    return tuple(x.cpu().numpy() for x in out)


@dataclasses.dataclass
class DraftParity:
    replays: int = 0
    mismatches: int = 0
    max_dlogit: float = 0.0
    max_dconf: float = 0.0
    max_dsurv: float = 0.0
    first_mismatch: tuple | None = None

    def ok(self) -> bool:
        return (self.mismatches == 0 and self.max_dlogit <= LOGIT_TOL and self.max_dconf <= CONF_TOL
                and self.max_dsurv <= CONF_TOL)


def check_draft(w: dict, gpu_out, rows=None, head: str = "markov") -> DraftParity:
    """Runs the oracle (Markov or RNN head) on `rows` (default: all),
    replaying the GPU's token at near ties, and compares element by element."""
    from oracle import dspark_oracle as orc
    g_tok, g_logit, g_conf, g_surv = gpu_out
    B = g_tok.shape[0]
    rows = np.arange(B) if rows is None else np.asarray(rows)
    st = DraftParity()

    def choose(k, rws, s, x):
        x = x.copy()
        for i in range(len(rws)):
            g = int(g_tok[rws[i], k - 1])
            if g == int(x[i]):
                continue
            row = s[i]
            top = row[x[i]]
            if not (0 <= g < row.size):
                st.mismatches += 1
                st.first_mismatch = st.first_mismatch or (int(rws[i]), k, int(x[i]), g)
                continue
            part = np.partition(row, -2)[-2:]
            gap = float(part[1]) - float(part[0])
            if gap < TIE_TOL and float(row[g]) >= float(top) - TIE_TOL:
                st.replays += 1
                x[i] = g
            else:
                st.mismatches += 1
                st.first_mismatch = st.first_mismatch or (int(rws[i]), k, int(x[i]), g)
        return x

    o_tok, o_logit, o_conf, o_surv = orc.draft_workload(w, rows=rows, choose=choose, head=head)
    diff = o_tok != g_tok[rows]
    st.mismatches = max(st.mismatches, int(diff.sum()))
    st.max_dlogit = float(np.abs(o_logit - g_logit[rows]).max())
    st.max_dconf = float(np.abs(o_conf - g_conf[rows]).max())
    st.max_dsurv = float(np.abs(o_surv - g_surv[rows]).max())
    return st
