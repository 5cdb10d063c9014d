"""Comparison of GPU outputs with the fp64 oracle.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark sanity check).

Parity rule.  Greedy outputs must match bit for bit.  In sampling mode the
decisions of a sequence are compared in order; at the first difference the
mismatch is excused only when the oracle's own margin is below 1e-5: for an
acceptance test |u_k - threshold_k| < 1e-5, for the draw a distance below 1e-5
between u and the oracle's interval (normalised running sum) of the token the
GPU chose.  Excused mismatches must stay below 1e-4 of all decisions (accept
tests evaluated plus one draw per sequence).  Log normalisers must agree
within 1e-5 * max(1, |log Z|).
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .verify import Result, draw_interval

NEAR_TIE = 1e-5
BUDGET = 1e-4
LOGZ_TOL = 1e-5


@dataclasses.dataclass
class GpuOut:
    tokens: np.ndarray
    n: np.ndarray
    logz: np.ndarray | None     # None: not returned (then not compared)
    flags: np.ndarray | None


@dataclasses.dataclass
class Report:
    sequences: int
    decisions: int
    excused: int
    failures: list
    max_logz_err: float

    def check(self):
        assert not self.failures, f"{len(self.failures)} non-excused mismatches, first: {self.failures[:3]}"
        assert self.excused <= BUDGET * self.decisions, \
            f"{self.excused} excused mismatches over {self.decisions} decisions"
        assert self.max_logz_err <= LOGZ_TOL, f"log Z error {self.max_logz_err}"


def compare(batch, gpu: GpuOut, ref: Result, rows: np.ndarray | None = None) -> Report:
    """Compare GPU outputs for batch rows ``rows`` (default all) with the
    oracle's results for the same sequences, in the same order."""
    rows = np.arange(batch.B) if rows is None else np.asarray(rows)
    K = batch.K
    nd = getattr(batch, "num_drafts", None)
    kbs = np.full(batch.B, K) if nd is None else np.asarray(nd)
    failures, excused = [], 0
    greedy = batch.T == 0.0
    max_lz = 0.0
    for i, b in enumerate(rows):
        gt, gn = gpu.tokens[b], int(gpu.n[b])
        ot, on = ref.tokens[i], int(ref.n_accepted[i])
        kb = int(kbs[b])
        if not (0 <= gn <= kb) or np.any(gt[gn + 1:] != -1) or list(gt[:gn]) != list(batch.draft_tokens[b, :gn]):
            failures.append((int(b), "malformed output", gt.tolist(), gn))
            continue
        if gpu.flags is not None and gpu.flags[b] & 4 != ref.flags[i] & 4 and gn == on:
            failures.append((int(b), "bad-draft flag", int(gpu.flags[b]), int(ref.flags[i])))
        if greedy:
            if gn != on or not np.array_equal(gt, ot):
                failures.append((int(b), "greedy", gt.tolist(), ot.tolist()))
            continue
        if gpu.logz is not None:
            used = np.isfinite(ref.logz[i])  # rows the sequence uses (all of them unless K_b < K)
            lz = gpu.logz[b].astype(np.float64)[used]
            rz = ref.logz[i][used]
            max_lz = max(max_lz, float(np.max(np.abs(lz - rz) / np.maximum(1.0, np.abs(rz)))))
        if gn != on:
            k = min(gn, on)
            margin = abs(float(batch.u_accept[b, k]) - ref.thr[i, k])
            if margin < NEAR_TIE:
                excused += 1
            else:
                failures.append((int(b), f"accept test {k}", gn, on, margin))
            continue
        if gt[gn] != ot[on]:
            j = int(gt[gn])
            if not (0 <= j < batch.V):
                failures.append((int(b), "draw out of range", j))
                continue
            lo, hi = draw_interval(batch.logits_p[b][: kb + 1],
                                   None if batch.logits_q is None else batch.logits_q[b][:kb],
                                   gn, j, float(batch.u_resample[b]), batch.T, batch.dtype)
            u = float(batch.u_resample[b])
            dist = 0.0 if lo <= u < hi else min(abs(u - lo), abs(u - hi))
            if dist < NEAR_TIE:
                excused += 1
            else:
                failures.append((int(b), "draw", j, int(ot[on]), dist))
    decisions = int(np.sum(np.minimum(ref.n_accepted + 1, kbs[rows])) + len(rows))
    return Report(len(rows), decisions, excused, failures, max_lz)
