"""Pins of the comparison machinery: ``oracle.draw_interval`` and
``oracle.parity.compare``.

Every sampling-mode GPU verdict goes through these two functions, so they are
pinned here on the CPU, independently of any GPU:

* ``draw_interval`` against a closed form worked by hand (the residual
  max(0, p - q) / Z of [B] "拒绝之后怎么办？——残差分布" on a four-token
  vocabulary), against the tiling of [0, 1) that any inverse CDF must give,
  and against the token the oracle itself draws for many uniforms (residual,
  bonus, per-sequence draft counts, and the zero-residual fallback).
* ``compare`` on synthetic "GPU outputs": an exact copy of the oracle passes,
  and each plausible wrong output (a shifted token, a wrong count, bad
  padding, a wrong accepted prefix, a dropped flag, a log Z error, a token out
  of range) fails, while a difference within the near-tie window is excused
  and counted against the budget of 1e-4 of decisions.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads
from oracle.parity import BUDGET, NEAR_TIE, GpuOut, Report, compare


# ------------------------------------------------------------ draw_interval --
def _ln(p):
    return np.log(np.asarray(p, np.float64)).astype(np.float32)


def test_draw_interval_closed_form_residual_and_bonus():
    """V = 4, T = 1, logits ln p and ln q.  Residual after a rejection at 0:
    max(0, p - q) = (0.3, 0, 0.2, 0), Z = 0.5, so the normalised intervals are
    token 0: [0, 0.6), token 1: empty at 0.6, token 2: [0.6, 1), token 3:
    empty at 1.  After one acceptance (K = 1) the bonus row p_1 is drawn from
    directly: its own cumulative sums."""
    p0, q0 = [0.4, 0.1, 0.3, 0.2], [0.1, 0.4, 0.1, 0.4]
    p1 = [0.125, 0.5, 0.25, 0.125]
    lp = np.stack([_ln(p0), _ln(p1)])       # [K+1, V] with K = 1
    lq = _ln(q0)[None, :]
    want_res = [(0.0, 0.6), (0.6, 0.6), (0.6, 1.0), (1.0, 1.0)]
    want_bonus = [(0.0, 0.125), (0.125, 0.625), (0.625, 0.875), (0.875, 1.0)]
    for j in range(4):
        lo, hi = oracle.draw_interval(lp, lq, 0, j, 0.5, 1.0, "fp32")
        np.testing.assert_allclose((lo, hi), want_res[j], rtol=0, atol=1e-6)
        lo, hi = oracle.draw_interval(lp, lq, 1, j, 0.5, 1.0, "fp32")
        np.testing.assert_allclose((lo, hi), want_bonus[j], rtol=0, atol=1e-6)


def test_draw_interval_zero_residual_falls_back_to_p():
    """p_n == q_n (identical logits): the residual is zero, and the draw uses
    p_n's own intervals, as the oracle's fallback does."""
    p = [0.5, 0.25, 0.125, 0.125]
    lp = np.stack([_ln(p), _ln(p)])
    lq = _ln(p)[None, :]
    cum = np.cumsum([0.0] + p)
    for j in range(4):
        lo, hi = oracle.draw_interval(lp, lq, 0, j, 0.3, 1.0, "fp32")
        np.testing.assert_allclose((lo, hi), (cum[j], cum[j + 1]), rtol=0, atol=1e-6)


def _intervals(lp, lq, n, T, dtype, V):
    return np.array([oracle.draw_interval(lp, lq, n, j, 0.5, T, dtype) for j in range(V)])


@pytest.mark.parametrize("dtype,T", [("fp32", 1.0), ("bf16", 0.7)])
def test_draw_interval_tiles_the_unit_interval(dtype, T):
    """Token intervals in ascending id order tile [0, 1): each starts where the
    previous one ends, the first at 0, the last ends at 1, none is reversed."""
    wl = workloads.Workload("t", 4, 3, 40, dtype, float(np.float32(T)), 2.0, 1.1, "noise", 0.8)
    b = workloads.make_batch(1, wl=wl, seed=5)
    for s in range(b.B):
        for n in range(b.K + 1):  # residual rows and the bonus row
            iv = _intervals(b.logits_p[s], b.logits_q[s], n, b.T, dtype, b.V)
            assert iv[0, 0] == 0.0
            assert abs(iv[-1, 1] - 1.0) < 1e-12
            assert np.all(iv[:, 1] >= iv[:, 0])
            np.testing.assert_array_equal(iv[1:, 0], iv[:-1, 1])


def _check_against_oracle_draws(batch, seqs_u=24):
    """For every sequence and many uniforms, the token the oracle draws is the
    one whose draw_interval holds u, and for the batch's own uniform the
    interval equals the (lo, hi) the oracle reports."""
    ref = oracle.verify_batch(batch)
    K = batch.K
    kbs = np.full(batch.B, K) if batch.num_drafts is None else batch.num_drafts
    for s in range(batch.B):
        kb = int(kbs[s])
        lp = batch.logits_p[s][: kb + 1]
        lq = batch.logits_q[s][:kb]
        n, j = int(ref.n_accepted[s]), int(ref.tokens[s, ref.n_accepted[s]])
        lo, hi = oracle.draw_interval(lp, lq, n, j, float(batch.u_resample[s]), batch.T, batch.dtype)
        assert (lo, hi) == (ref.draw_lo[s], ref.draw_hi[s])
        assert lo <= batch.u_resample[s] < hi
        # other uniforms: keep the accept uniforms (so n stays), vary the draw's
        iv = _intervals(lp, lq, n, batch.T, batch.dtype, batch.V)
        for u in np.linspace(0.0, 1.0, seqs_u, endpoint=False)[1:]:
            yp = oracle.widen(lp, batch.dtype) / batch.T
            yq = oracle.widen(lq, batch.dtype) / batch.T
            r = oracle.verify_sequence(yp, yq, batch.draft_tokens[s][:kb], batch.u_accept[s][:kb], float(u))
            assert r["n"] == n
            tok = int(r["tokens"][n])
            assert iv[tok, 0] <= u < iv[tok, 1], (s, u, tok, iv[tok])


def test_draw_interval_agrees_with_the_oracle_draw_residual_and_bonus():
    wl = workloads.Workload("t", 12, 3, 60, "bf16", float(np.float32(1.0)), 2.0, 1.1, "noise", 0.6)
    b = workloads.make_batch(1, wl=wl, seed=21)
    ref = oracle.verify_batch(b)
    assert np.any(ref.n_accepted < b.K) and np.any(ref.n_accepted == b.K), "both draw kinds covered"
    _check_against_oracle_draws(b)


def test_draw_interval_agrees_with_the_oracle_draw_ragged():
    wl = workloads.Workload("t", 12, 4, 50, "fp32", float(np.float32(0.8)), 2.0, 1.1, "noise", 0.5)
    b = workloads.make_batch(1, wl=wl, seed=22)
    b = dataclasses.replace(b, num_drafts=workloads.ragged_draft_counts(b.B, b.K, seed=22, low=0))
    assert np.any(b.num_drafts == 0)
    _check_against_oracle_draws(b)


def test_draw_interval_agrees_with_the_oracle_draw_small_residual():
    """q_0 is p_0 with one token's logit raised by 0.01: the test at that token
    rejects (u just below 1), and the residual max(0, p - q) is small but
    positive on every other token.  Its intervals still match the oracle's draws."""
    rng = np.random.default_rng(23)
    V = 30
    row = rng.normal(0, 2, V).astype(np.float32)
    lp = np.stack([row, row, rng.normal(0, 2, V).astype(np.float32)])[None]
    lq = np.stack([row, row])[None].copy()
    lq[0, 0, 3] += np.float32(0.01)
    b = workloads.custom_batch(lp, lq, [[3, 0]], [[np.nextafter(np.float32(1), np.float32(0)), 0.5]], [0.37],
                               1.0, "fp32")
    ref = oracle.verify_batch(b)
    assert ref.n_accepted[0] == 0 and ref.flags[0] == 0
    _check_against_oracle_draws(b)


def test_draw_interval_exact_zero_residual_flags_and_uses_p():
    """Identical rows and a draft id outside [0, V): the test fails (flag 4),
    the residual is exactly zero, so the draw falls back to p (flag 2) and
    draw_interval returns p's intervals."""
    rng = np.random.default_rng(24)
    V = 16
    row = rng.normal(0, 1, V).astype(np.float32)
    lp = np.stack([row, rng.normal(0, 1, V).astype(np.float32)])[None]
    lq = row[None, None, :]
    b = workloads.custom_batch(lp, lq, [[V + 2]], [[0.5]], [0.61], 1.0, "fp32")
    ref = oracle.verify_batch(b)
    assert ref.n_accepted[0] == 0
    assert ref.flags[0] == oracle.FLAG_ZW_ZERO | oracle.FLAG_BAD_DRAFT
    p = np.exp(row.astype(np.float64) - oracle.log_normalizer(row.astype(np.float64)))
    cum = np.concatenate([[0.0], np.cumsum(p)]) / np.sum(p)
    j = int(ref.tokens[0, 0])
    lo, hi = oracle.draw_interval(lp[0], lq[0], 0, j, 0.61, 1.0, "fp32")
    np.testing.assert_allclose((lo, hi), (cum[j], cum[j + 1]), rtol=0, atol=1e-14)
    assert lo <= 0.61 < hi


# ----------------------------------------------------------------- compare --
def _batch(seed=31, B=24, K=4, V=3000, dtype="bf16", T=0.9):
    wl = workloads.Workload("t", B, K, V, dtype, float(np.float32(T)), 2.0, 1.1, "noise", 1.0)
    return workloads.make_batch(1, wl=wl, seed=seed)


def _copy(ref):
    return GpuOut(ref.tokens.copy(), ref.n_accepted.copy(), ref.logz.astype(np.float32), ref.flags.copy())


def _pick(pred, n):
    idx = [i for i in range(n) if pred(i)]
    assert idx, "the fixture has no sequence of the kind this test needs"
    return idx[0]


def _fresh(b, **kw):
    """The batch with some host arrays replaced (copies, so fixtures stay intact)."""
    return dataclasses.replace(b, **{k: np.array(v) for k, v in kw.items()})


def test_compare_exact_copy_passes():
    b = _batch()
    ref = oracle.verify_batch(b)
    rep = compare(b, _copy(ref), ref)
    assert rep.failures == [] and rep.excused == 0
    assert rep.decisions == int(np.sum(np.minimum(ref.n_accepted + 1, b.K)) + b.B)
    rep.check()


def test_compare_fails_a_shifted_token_far_from_an_edge():
    b = _batch()
    ref = oracle.verify_batch(b)
    s = _pick(lambda i: min(b.u_resample[i] - ref.draw_lo[i], ref.draw_hi[i] - b.u_resample[i]) > 1e-3, b.B)
    g = _copy(ref)
    n = g.n[s]
    g.tokens[s, n] = (g.tokens[s, n] + 1) % b.V
    rep = compare(b, g, ref)
    assert [f[1] for f in rep.failures] == ["draw"]
    with pytest.raises(AssertionError):
        rep.check()


def test_compare_fails_a_token_out_of_range():
    b = _batch()
    ref = oracle.verify_batch(b)
    g = _copy(ref)
    g.tokens[2, g.n[2]] = b.V
    assert [f[1] for f in compare(b, g, ref).failures] == ["draw out of range"]


def _next_positive_token(b, s, n, j):
    iv = _intervals(b.logits_p[s], b.logits_q[s], n, b.T, b.dtype, b.V)
    for k in range(j + 1, b.V):
        if iv[k, 1] > iv[k, 0]:
            return k, iv
    return None, iv


@pytest.mark.parametrize("gap,excused", [(3e-6, True), (9e-6, True), (1.3e-5, False), (4e-5, False)])
def test_compare_near_edge_draw_window(gap, excused):
    """u placed `gap` below the end of the oracle token's interval; the GPU
    answers the next token (whose interval starts there).  Inside the 1e-5
    window the mismatch is excused and counted; outside it fails."""
    b = _batch()
    ref0 = oracle.verify_batch(b)
    s = _pick(lambda i: ref0.draw_hi[i] - ref0.draw_lo[i] > 1e-4 and ref0.draw_hi[i] < 0.99, b.B)
    u = np.float32(ref0.draw_hi[s] - gap)
    ur = b.u_resample.copy()
    ur[s] = u
    bb = _fresh(b, u_resample=ur)
    ref = oracle.verify_batch(bb)
    n, j = int(ref.n_accepted[s]), int(ref.tokens[s, ref.n_accepted[s]])
    assert j == ref0.tokens[s, ref0.n_accepted[s]]
    j1, _ = _next_positive_token(bb, s, n, j)
    g = _copy(ref)
    g.tokens[s, n] = j1
    rep = compare(bb, g, ref)
    if excused:
        assert rep.failures == [] and rep.excused == 1
        # one excused mismatch among ~100 decisions is over the 1e-4 budget
        assert rep.excused > BUDGET * rep.decisions
        with pytest.raises(AssertionError):
            rep.check()
    else:
        assert rep.excused == 0 and [f[1] for f in rep.failures] == ["draw"]


@pytest.mark.parametrize("later", [True, False])
def test_compare_accept_count_off_by_one(later):
    """GPU n differs from the oracle's at a test whose margin is large: a
    failure, whichever side rejected first."""
    b = _batch()
    ref = oracle.verify_batch(b)
    if later:
        s = _pick(lambda i: ref.n_accepted[i] < b.K - 1 and
                  abs(b.u_accept[i, ref.n_accepted[i]] - ref.thr[i, ref.n_accepted[i]]) > 1e-3, b.B)
    else:
        s = _pick(lambda i: ref.n_accepted[i] >= 1 and abs(b.u_accept[i, 0] - ref.thr[i, 0]) > 1e-3, b.B)
    g = _copy(ref)
    on = int(ref.n_accepted[s])
    gn = on + 1 if later else 0
    g.n[s] = gn
    row = np.full(b.K + 1, -1, np.int32)
    row[:gn] = b.draft_tokens[s, :gn]
    row[gn] = 0
    g.tokens[s] = row
    rep = compare(b, g, ref)
    assert [f[1] for f in rep.failures] == [f"accept test {min(gn, on)}"]


def _near_tie_accept_batch(b, ref, k_pos, gap, on_side):
    """A copy of the batch whose uniform at position k_pos of some sequence lies
    `gap` below (on_side 'accept') or above ('reject') its threshold."""
    s = _pick(lambda i: ref.n_accepted[i] > k_pos and ref.thr[i, k_pos] < 0.999, b.B)
    ua = b.u_accept.copy()
    thr = ref.thr[s, k_pos]
    ua[s, k_pos] = np.float32(thr - gap if on_side == "accept" else thr + gap)
    return s, _fresh(b, u_accept=ua)


@pytest.mark.parametrize("gpu_rejects_earlier", [True, False])
def test_compare_near_tie_accept_is_excused_at_the_first_difference(gpu_rejects_earlier):
    """The near-tie margin is read at the FIRST differing test (min of the two
    counts), not the later one."""
    b = _batch()
    ref0 = oracle.verify_batch(b)
    if gpu_rejects_earlier:
        # oracle accepts position 0 by 3e-6; the GPU rejects there
        s, bb = _near_tie_accept_batch(b, ref0, 0, 3e-6, "accept")
        ref = oracle.verify_batch(bb)
        assert ref.n_accepted[s] >= 1
        gn = 0
    else:
        # oracle rejects at its n by 3e-6; the GPU accepts there and rejects one later
        s = _pick(lambda i: ref0.n_accepted[i] < b.K - 1 and ref0.thr[i, ref0.n_accepted[i]] < 0.999, b.B)
        on = int(ref0.n_accepted[s])
        ua = b.u_accept.copy()
        ua[s, on] = np.float32(ref0.thr[s, on] + 3e-6)
        bb = _fresh(b, u_accept=ua)
        ref = oracle.verify_batch(bb)
        assert ref.n_accepted[s] == on
        gn = on + 1
        # the test after the oracle's rejection has a large margin: reading the
        # margin there (the max of the two counts) would fail this case
        assert abs(bb.u_accept[s, gn] - oracle.verify_batch(_fresh(bb, u_accept=np.where(
            np.arange(bb.B)[:, None] == s, np.float32(1e-7), bb.u_accept))).thr[s, gn]) > NEAR_TIE
    g = _copy(ref)
    g.n[s] = gn
    row = np.full(b.K + 1, -1, np.int32)
    row[:gn] = bb.draft_tokens[s, :gn]
    row[gn] = 1
    g.tokens[s] = row
    rep = compare(bb, g, ref)
    assert rep.failures == [] and rep.excused == 1
    # the decision count is the oracle's, not the GPU's
    assert rep.decisions == int(np.sum(np.minimum(ref.n_accepted + 1, bb.K)) + bb.B)


@pytest.mark.parametrize("mutation", ["padding", "prefix", "n_negative", "n_past_K"])
def test_compare_fails_malformed_outputs(mutation):
    b = _batch()
    ref = oracle.verify_batch(b)
    s = _pick(lambda i: 1 <= ref.n_accepted[i] < b.K, b.B)
    g = _copy(ref)
    n = int(g.n[s])
    if mutation == "padding":
        g.tokens[s, n + 1] = 7
    elif mutation == "prefix":
        g.tokens[s, 0] = (g.tokens[s, 0] + 1) % b.V
    elif mutation == "n_negative":
        g.n[s] = -1
    else:
        g.n[s] = b.K + 1
    assert [f[1] for f in compare(b, g, ref).failures] == ["malformed output"]


def test_compare_ragged_count_past_the_sequence_draft_count_is_malformed():
    b = _batch()
    b = dataclasses.replace(b, num_drafts=workloads.ragged_draft_counts(b.B, b.K, seed=32, low=0))
    ref = oracle.verify_batch(b)
    compare(b, _copy(ref), ref).check()
    s = _pick(lambda i: ref.n_accepted[i] == b.num_drafts[i] and b.num_drafts[i] < b.K, b.B)
    g = _copy(ref)
    kb = int(b.num_drafts[s])
    g.n[s] = kb + 1
    g.tokens[s, kb] = b.draft_tokens[s, kb]
    g.tokens[s, kb + 1] = 0
    assert [f[1] for f in compare(b, g, ref).failures] == ["malformed output"]


def test_compare_fails_a_dropped_bad_draft_flag():
    b = _batch()
    x = b.draft_tokens.copy()
    x[5, 0] = b.V + 11
    bb = _fresh(b, draft_tokens=x)
    ref = oracle.verify_batch(bb)
    assert ref.flags[5] & oracle.FLAG_BAD_DRAFT and ref.n_accepted[5] == 0
    compare(bb, _copy(ref), ref).check()
    g = _copy(ref)
    g.flags[5] = 0
    assert [f[1] for f in compare(bb, g, ref).failures] == ["bad-draft flag"]


@pytest.mark.parametrize("rel,ok", [(5e-6, True), (2e-5, False)])
def test_compare_log_normaliser_tolerance(rel, ok):
    """log Z within 1e-5 * max(1, |log Z|): every row of these workloads has
    |log Z| well above 1, so the check is relative there."""
    b = _batch()
    ref = oracle.verify_batch(b)
    assert np.all(np.abs(ref.logz) > 1.0)
    g = _copy(ref)
    g.logz = (ref.logz * (1.0 + rel)).astype(np.float32)
    rep = compare(b, g, ref)
    assert rep.failures == []
    assert abs(rep.max_logz_err - rel) < 2e-7
    if ok:
        rep.check()
    else:
        with pytest.raises(AssertionError):
            rep.check()


def test_compare_greedy_is_bit_exact():
    wl = workloads.Workload("t", 16, 4, 500, "bf16", 0.0, 2.0, 1.1, "greedy-mask")
    b = workloads.make_batch(4, wl=wl, seed=33)
    ref = oracle.verify_batch(b)
    g = GpuOut(ref.tokens.copy(), ref.n_accepted.copy(), None, ref.flags.copy())
    compare(b, g, ref).check()
    s = int(np.argmax(ref.n_accepted < b.K))
    g.tokens[s, ref.n_accepted[s]] += 1
    assert [f[1] for f in compare(b, g, ref).failures] == ["greedy"]


@pytest.mark.parametrize("excused,ok", [(0, True), (2, True), (3, False)])
def test_report_budget_trips_at_the_right_count(excused, ok):
    """20000 decisions allow at most 2 excused mismatches (1e-4 of them)."""
    rep = Report(sequences=4000, decisions=20000, excused=excused, failures=[], max_logz_err=0.0)
    if ok:
        rep.check()
    else:
        with pytest.raises(AssertionError):
            rep.check()
