"""Device-side input validation (spec_debug_enable / spec_debug_counters /
spec_debug_reset): a clean batch counts nothing and draws the same outputs
as without validation; a small batch with planted contract breaks (draft ids
outside [0, V), uniforms outside (0, 1), a NaN and a +inf logit, a row with
no finite logit) gives exactly the counts the header defines, in sampling,
greedy and ragged calls.  The verify step runs on the broken inputs too: its
tokens are unspecified there, and it must only finish."""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


def _counts(sv, fn):
    """Counters added by fn() with validation on (restored afterwards)."""
    prev = sv.debug_enable(True)
    try:
        sv.debug_reset()
        fn()
        return sv.debug_counters()
    finally:
        sv.debug_enable(prev)


def test_clean_batch_counts_nothing_and_draws_the_same(gpu_lib):
    sv = gpu_lib
    b = workloads.make_batch(1, seqs=range(16))
    lp, lq, x, ua, ur = workloads.to_device(b)
    prev = sv.debug_enable(False)
    try:
        t0, n0, f0 = sv.verify(lp, lq, x, ua, ur, b.T, return_flags=True)
        torch.cuda.synchronize()
    finally:
        sv.debug_enable(prev)
    out = {}
    c = _counts(sv, lambda: out.update(r=sv.verify(lp, lq, x, ua, ur, b.T, return_flags=True)))
    t1, n1, f1 = out["r"]
    assert c == dict(calls=1, bad_draft_ids=0, bad_u_accept=0, bad_u_resample=0, nan_logits=0, inf_logits=0,
                     rows_no_finite=0), c
    np.testing.assert_array_equal(t1.cpu().numpy(), t0.cpu().numpy())
    np.testing.assert_array_equal(n1.cpu().numpy(), n0.cpu().numpy())
    np.testing.assert_array_equal(f1.cpu().numpy(), f0.cpu().numpy())


def _planted():
    """Four sequences of the tiny workload's recipe (K=4, V=1000, fp32) with
    contract breaks: sequence 0 draft ids V and -5 (positions 1, 3);
    sequence 1 accept uniforms 0 and NaN (positions 2, 3); sequence 2
    resample uniform 1; sequence 3 a NaN in target row 1, a +inf in draft
    row 0, and a bonus target row (row K) of -inf only."""
    b = workloads.make_batch(0, seqs=range(4))
    V = b.V
    x = b.draft_tokens.copy()
    x[0, 1], x[0, 3] = V, -5
    ua = b.u_accept.copy()
    ua[1, 2], ua[1, 3] = 0.0, np.nan
    ur = b.u_resample.copy()
    ur[2] = 1.0
    lp, lq = b.logits_p.copy(), b.logits_q.copy()
    lp[3, 1, 10] = np.nan
    lq[3, 0, 20] = np.inf
    lp[3, b.K, :] = -np.inf
    return workloads.custom_batch(lp, lq, x, ua, ur, b.T, b.dtype)


def test_planted_breaks_are_counted(gpu_lib):
    sv = gpu_lib
    b = _planted()
    lp, lq, x, ua, ur = workloads.to_device(b)
    c = _counts(sv, lambda: sv.verify(lp, lq, x, ua, ur, b.T))
    assert c == dict(calls=1, bad_draft_ids=2, bad_u_accept=2, bad_u_resample=1, nan_logits=1, inf_logits=1,
                     rows_no_finite=1), c
    # greedy reads target rows and draft ids only: no uniforms, no draft rows
    c = _counts(sv, lambda: sv.verify(lp, None, x, None, None, 0.0))
    assert c == dict(calls=1, bad_draft_ids=2, bad_u_accept=0, bad_u_resample=0, nan_logits=1, inf_logits=0,
                     rows_no_finite=1), c
    # per-sequence draft counts: only positions below K_b and the rows they
    # use are checked (sequence 0 keeps position 0, sequence 1 positions 0-1,
    # sequence 3 target rows 0-1 and draft row 0)
    kb = torch.tensor([1, 2, 4, 1], dtype=torch.int32, device=lp.device)
    c = _counts(sv, lambda: sv.verify(lp, lq, x, ua, ur, b.T, num_drafts=kb))
    assert c == dict(calls=1, bad_draft_ids=0, bad_u_accept=0, bad_u_resample=1, nan_logits=1, inf_logits=1,
                     rows_no_finite=0), c
    # two calls add up
    c = _counts(sv, lambda: (sv.verify(lp, lq, x, ua, ur, b.T), sv.verify(lp, lq, x, ua, ur, b.T)))
    assert c["calls"] == 2 and c["bad_draft_ids"] == 4 and c["nan_logits"] == 2, c
