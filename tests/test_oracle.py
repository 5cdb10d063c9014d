"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every pin here is independent of the oracle's own formulas: library routines
(scipy's logsumexp and softmax, numpy's argmax and searchsorted), closed
forms, the pages' identity and worked values, exact enumeration and
Monte-Carlo laws.  A plausible slip in the oracle (a dropped term, a flipped
comparison, an off-by-one index, p and q swapped) fails at least one of them.
"""
import json
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest
from scipy.special import logsumexp, softmax
from scipy.stats import chi2

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _seq(yp, yq, x, ua, ur):
    return oracle.verify_sequence(np.asarray(yp, float), np.asarray(yq, float), np.asarray(x),
                                  np.asarray(ua, float), float(ur))


# ----------------------------------------------------------------- log Z --
@pytest.mark.parametrize("V", [1, 2, 7, 1000, 32000])
@pytest.mark.parametrize("scale", [0.1, 3.0, 40.0])
def test_log_normalizer_matches_scipy(V, scale):
    rng = np.random.default_rng(V * 7 + int(scale * 10))
    y = rng.normal(0, scale, size=(3, V))
    y[0, 1::5] = -np.inf          # some -inf logits; element 0 stays finite
    np.testing.assert_allclose(oracle.log_normalizer(y), logsumexp(y, axis=-1), rtol=1e-14, atol=1e-13)


@pytest.mark.parametrize("V", [1, 3, 128256])
def test_log_normalizer_equal_logits_closed_form(V):
    c = 1.75
    y = np.full((2, V), c)
    np.testing.assert_allclose(oracle.log_normalizer(y), c + np.log(V), rtol=0, atol=1e-12)


def test_verify_reports_logz_at_temperature():
    # V equal logits x at temperature T: log Z = x/T + log V, for every row.
    K, V, x, T = 3, 50, 0.625, float(np.float32(0.7))
    lp = np.full((1, K + 1, V), x, np.float32)
    lq = np.full((1, K, V), x, np.float32)
    r = oracle.verify(lp, lq, np.zeros((1, K), np.int32), np.full((1, K), 0.5, np.float32),
                      np.full(1, 0.5, np.float32), T, "fp32")
    np.testing.assert_allclose(r.logz[0], x / T + np.log(V), rtol=0, atol=1e-12)


def test_widen_bf16_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F, 0xFF80], np.uint16)
    want = np.array([1.0, -1.0, 3.140625, 0.0, -0.0, 3.3895313892515355e38, -np.inf])
    np.testing.assert_array_equal(oracle.widen(bits, "bf16"), want)


# ------------------------------------------------------ identity and rates --
def _random_pq(rng, V, spread=2.0):
    return softmax(rng.normal(0, spread, V)), softmax(rng.normal(0, spread, V))


def test_residual_identity_per_token():
    """min(p,q) + max(0, p - q) = p for every token ([B] "拒绝之后怎么办？——残差分布",
    the two paths that produce a token)."""
    rng = np.random.default_rng(1)
    for V in (2, 8, 1000, 128256):
        p, q = _random_pq(rng, V)
        np.testing.assert_allclose(np.minimum(p, q) + oracle.residual(p, q), p, rtol=0, atol=1e-15)
        # the residual mass is what the acceptance path leaves over
        assert abs(oracle.residual(p, q).sum() - (1.0 - np.minimum(p, q).sum())) < 1e-14


def test_residual_never_negative_and_zero_where_q_dominates():
    rng = np.random.default_rng(2)
    p, q = _random_pq(rng, 64)
    w = oracle.residual(p, q)
    assert np.all(w >= 0)
    assert np.all(w[q >= p] == 0)
    assert np.all(w[p > q] > 0)


def test_acceptance_threshold_cases():
    """alpha(x) = min(1, p/q): 1 when p >= q, p/q otherwise ([B] "验收标准的精确数学", two cases)."""
    lp = np.log(np.array([0.5, 0.2, 0.1, 1e-300, 0.3]))
    lq = np.log(np.array([0.25, 0.2, 0.4, 0.5, 1e-310]))
    thr = oracle.acceptance_threshold(lp, lq)
    np.testing.assert_allclose(thr, [1.0, 1.0, 0.25, 2e-300, 1.0], rtol=1e-12, atol=0)


def test_acceptance_rate_is_sum_of_min():
    """P(accept at a position | x ~ q) = sum_x min(p, q) ([B] path 1 has mass min(q(x), p(x)))."""
    rng = np.random.default_rng(3)
    V, N = 8, 60000
    lp, lq = rng.normal(0, 1.5, (2, V)), rng.normal(0, 1.5, (1, V))
    p, q = softmax(lp[0]), softmax(lq[0])
    beta = np.minimum(p, q).sum()
    xs = rng.choice(V, size=N, p=q)
    us = rng.random(N)
    acc = sum(_seq(lp, lq, [x], [u], 0.5)["n"] == 1 for x, u in zip(xs, us))
    z = (acc / N - beta) / np.sqrt(beta * (1 - beta) / N)
    assert abs(z) < 5, (acc / N, beta)


# --------------------------------------------------------- exact enumeration --
def _segments(f, grid=2048):
    """Maximal intervals of (0,1) on which the piecewise-constant f is
    constant, found by a grid scan and bisection: [(lo, hi, value), ...]."""
    pts = (np.arange(grid) + 0.5) / grid
    vals = [f(x) for x in pts]
    cuts, seg_vals = [0.0], [vals[0]]
    for i in range(grid - 1):
        if vals[i + 1] != vals[i]:
            a, b = pts[i], pts[i + 1]
            for _ in range(64):
                m = 0.5 * (a + b)
                if f(m) == vals[i]:
                    a = m
                else:
                    b = m
            assert f(b) == vals[i + 1], "more than one change inside a grid cell"
            cuts.append(b)
            seg_vals.append(vals[i + 1])
    cuts.append(1.0)
    return [(cuts[i], cuts[i + 1], seg_vals[i]) for i in range(len(seg_vals))]


@pytest.mark.parametrize("T", [1.0, float(np.float32(0.7))])
def test_exact_outcome_law_V4_K2(T):
    """All outcomes at V=4, K=2, enumerated exactly.  The oracle is used as a
    black box: for each draft pair (weighted q1(x1) q2(x2)) the regions of
    u1, u2 and u_resample that give each output are located by bisection.
    The resulting law must equal the one the pages' two-path argument gives:
      (v)       : max(0, p1 - q1)(v)
      (v, w)    : min(p1, q1)(v) * max(0, p2 - q2)(w)
      (v, w, z) : min(p1, q1)(v) * min(p2, q2)(w) * p3(z)
    and the first token's marginal must be p1 exactly ([B] the identity
    min(q, p) + max(0, p - q) = p)."""
    V, K = 4, 2
    lp = np.array([[1.2, -0.3, 0.4, -1.0], [0.1, 0.9, -0.6, 0.3], [-0.2, 0.5, 0.0, 1.1]])
    lq = np.array([[0.2, 0.6, 0.9, -1.4], [1.0, -0.4, -0.2, 0.3]])
    yp, yq = lp / T, lq / T
    p = softmax(yp, axis=1)
    q = softmax(yq, axis=1)

    law = {}
    for x1 in range(V):
        for x2 in range(V):
            wx = q[0, x1] * q[1, x2]

            def out(u1, u2, ur):
                r = _seq(yp, yq, [x1, x2], [u1, u2], ur)
                return tuple(int(t) for t in r["tokens"] if t >= 0)

            # test 1 passes iff at least two tokens come out
            for a1, b1, acc1 in _segments(lambda u: len(out(u, 0.5, 0.5)) > 1):
                u1 = 0.5 * (a1 + b1)
                if not acc1:
                    for ar, br, toks in _segments(lambda ur: out(u1, 0.5, ur)):
                        law[toks] = law.get(toks, 0.0) + wx * (b1 - a1) * (br - ar)
                    continue
                for a2, b2, _acc2 in _segments(lambda u: len(out(u1, u, 0.5)) > 2):
                    u2 = 0.5 * (a2 + b2)
                    for ar, br, toks in _segments(lambda ur: out(u1, u2, ur)):
                        law[toks] = law.get(toks, 0.0) + wx * (b1 - a1) * (b2 - a2) * (br - ar)

    mn1, mn2 = np.minimum(p[0], q[0]), np.minimum(p[1], q[1])
    want = {}
    for v in range(V):
        want[(v,)] = max(0.0, p[0, v] - q[0, v])
        for w in range(V):
            want[(v, w)] = mn1[v] * max(0.0, p[1, w] - q[1, w])
            for z in range(V):
                want[(v, w, z)] = mn1[v] * mn2[w] * p[2, z]
    want = {k: v for k, v in want.items() if v > 0}
    assert set(law) == set(want)
    for k in want:
        assert abs(law[k] - want[k]) < 1e-12, (k, law[k], want[k])
    assert abs(sum(law.values()) - 1.0) < 1e-12
    first = np.zeros(V)
    for k, v in law.items():
        first[k[0]] += v
    np.testing.assert_allclose(first, p[0], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- chi-square --
def _first_tokens(args):
    seed, n, yp, yq = args
    rng = np.random.default_rng(seed)
    q0, q1 = softmax(yq[0]), softmax(yq[1])
    out = np.zeros(yp.shape[1], np.int64)
    x0s = rng.choice(len(q0), n, p=q0)
    x1s = rng.choice(len(q1), n, p=q1)
    us = rng.random((n, 3))
    for i in range(n):
        r = oracle.verify_sequence(yp, yq, np.array([x0s[i], x1s[i]]), us[i, :2], us[i, 2])
        out[r["tokens"][0]] += 1
    return out


def test_first_token_follows_p_chi_square():
    """10^6 verify steps at V=8, K=2 with x ~ q: the first emitted token must
    follow p_0 ([A] the output follows the target's distribution; [D]
    "Математическая гарантия").  chi-square with 7 degrees of freedom."""
    rng = np.random.default_rng(11)
    V = 8
    yp = rng.normal(0, 1.2, (3, V))
    yq = rng.normal(0, 1.2, (2, V))
    N, W = 10 ** 6, 8
    with ProcessPoolExecutor(W) as ex:
        counts = sum(ex.map(_first_tokens, [(100 + i, N // W, yp, yq) for i in range(W)]))
    p0 = softmax(yp[0])
    stat = np.sum((counts - N * p0) ** 2 / (N * p0))
    pval = chi2.sf(stat, V - 1)
    assert pval > 1e-3, (stat, pval, counts / N, p0)


# -------------------------------------------------------------------- E[N] --
def _mean_emitted(alpha_q0, K, N, seed):
    """Mean emitted tokens when every position has p = (1/2, 1/2) and
    q = (alpha_q0, 1 - alpha_q0), i.e. acceptance sum(min(p,q)) = 1.5 - alpha_q0."""
    rng = np.random.default_rng(seed)
    yp = np.zeros((K + 1, 2))
    yq = np.tile(np.log([alpha_q0, 1 - alpha_q0]), (K, 1))
    tot = 0
    for _ in range(N):
        x = (rng.random(K) >= alpha_q0).astype(np.int64)
        r = oracle.verify_sequence(yp, yq, x, rng.random(K), rng.random())
        tot += r["n"] + 1
    return tot / N


def test_expected_tokens_per_round_matches_pages():
    g = json.load(open(os.path.join(GOLDEN, "expected_tokens_per_round.json")))
    for case in g["cases"]:
        a, k = case["alpha"], case["k"]
        closed = (1 - a ** (k + 1)) / (1 - a)
        assert round(closed, case["printed_digits"]) == case["printed_E_N"]
        N = 20000
        mean = _mean_emitted(1.5 - a, k, N, seed=int(a * 100))
        assert abs(mean - closed) < 5 * 1.8 / np.sqrt(N), (a, mean, closed)
    for case in g["not_used"]:
        a, k = case["alpha"], case["k"]
        assert round((1 - a ** (k + 1)) / (1 - a), 1) != case["printed_E_N"]


def test_cycle_examples():
    """Token counts per round in the pages' worked cycles (accepted + 1)."""
    g = json.load(open(os.path.join(GOLDEN, "cycle_examples.json")))
    V = 16
    for case in g["cases"]:
        K, n_acc = case["K"], case["accepted"]
        rng = np.random.default_rng(K)
        yp = rng.normal(0, 1, (K + 1, V))
        yq = yp[:K] + rng.normal(0, 1, (K, V))
        x = np.argmax(yq, axis=1)
        ua = np.where(np.arange(K) < n_acc, 1e-12, 1.0 - 1e-12)  # accept, then reject unless thr == 1
        thr_ok = [oracle.acceptance_threshold(yp[k, x[k]] - logsumexp(yp[k]), yq[k, x[k]] - logsumexp(yq[k]))
                  for k in range(K)]
        if n_acc < K:
            assert thr_ok[n_acc] < 1.0 - 1e-12, "pick drafts whose test can fail"
        r = _seq(yp, yq, x, ua, 0.37)
        assert r["n"] == n_acc
        assert int(np.sum(r["tokens"] >= 0)) == case["emitted"]
        assert list(r["tokens"][:n_acc]) == list(x[:n_acc])


# ---------------------------------------------------------------- inverse CDF --
def test_inverse_cdf_matches_searchsorted_and_skips_zero_weights():
    rng = np.random.default_rng(5)
    w = rng.random(200)
    w[rng.random(200) < 0.4] = 0.0
    c = np.cumsum(w)
    for u in rng.random(500):
        v, lo, hi = oracle.inverse_cdf(w, u)
        assert v == np.searchsorted(c, u * c[-1], side="right")
        assert w[v] > 0
        assert lo <= u < hi
    # u at the very top of the range picks the last positive-weight token
    v, _, _ = oracle.inverse_cdf(np.array([0.2, 0.8, 0.0, 0.0]), np.nextafter(1.0, 0.0))
    assert v == 1


# ------------------------------------------------------------- special cases --
def test_identical_distributions_accept_everything():
    rng = np.random.default_rng(6)
    K, V = 5, 300
    y = rng.normal(0, 2, (K + 1, V))
    for _ in range(20):
        r = _seq(y, y[:K], rng.integers(0, V, K), rng.random(K), rng.random())
        assert r["n"] == K


def test_single_token_vocabulary():
    K = 4
    r = _seq(np.zeros((K + 1, 1)), np.ones((K, 1)), np.zeros(K, np.int64), [0.999] * K, 0.999)
    assert r["n"] == K and list(r["tokens"]) == [0] * (K + 1)


def test_tiny_uniform_accepts_wherever_threshold_exceeds_it():
    rng = np.random.default_rng(8)
    K, V = 6, 40
    yp, yq = rng.normal(0, 3, (K + 1, V)), rng.normal(0, 3, (K, V))
    x = np.argmin(yp[:K] - yq, axis=1)                    # drafts the target dislikes
    u = 2.0 ** -25
    r = _seq(yp, yq, x, [u] * K, 0.5)
    lzp, lzq = logsumexp(yp, axis=1), logsumexp(yq, axis=1)
    thr = [min(1.0, np.exp((yp[k, x[k]] - lzp[k]) - (yq[k, x[k]] - lzq[k]))) for k in range(K)]
    want = next((k for k in range(K) if not thr[k] > u), K)
    assert r["n"] == want


def test_temperature_scaling_invariance():
    """logits*2 at T*2 gives bit-identical outputs (x/T is unchanged exactly)."""
    rng = np.random.default_rng(9)
    B, K, V = 6, 4, 500
    lp = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
    lq = rng.normal(0, 2, (B, K, V)).astype(np.float32)
    x = rng.integers(0, V, (B, K)).astype(np.int32)
    ua = rng.random((B, K)).astype(np.float32)
    ur = rng.random(B).astype(np.float32)
    a = oracle.verify(lp, lq, x, ua, ur, 0.7, "fp32")
    b = oracle.verify(lp * 2, lq * 2, x, ua, ur, float(np.float32(0.7)) * 2, "fp32")
    np.testing.assert_array_equal(a.tokens, b.tokens)
    np.testing.assert_array_equal(a.n_accepted, b.n_accepted)


def test_bad_draft_id_is_rejected_and_flagged():
    rng = np.random.default_rng(10)
    K, V = 4, 30
    yp, yq = rng.normal(0, 1, (K + 1, V)), rng.normal(0, 1, (K, V))
    for bad in (-1, V, 1 << 30):
        x = np.array([0, bad, 1, 2])
        r = _seq(yp, yq, x, [1e-9] * K, 0.5)
        assert r["n"] == 1 and r["flags"] & oracle.FLAG_BAD_DRAFT


def test_greedy_matches_numpy_argmax_including_ties():
    rng = np.random.default_rng(12)
    K, V = 8, 1000
    for trial in range(30):
        lp = np.round(rng.normal(0, 2, (K + 1, V)), 1)
        for k in range(K + 1):                                # plant ties at the maximum
            i, j = rng.choice(V, 2, replace=False)
            lp[k, i] = lp[k, j] = lp[k].max() + 1
        a = np.argmax(lp, axis=1)
        other = np.array([np.flatnonzero(lp[k] == lp[k].max())[-1] for k in range(K)])
        take = rng.random(K) < 0.7
        x = np.where(take, a[:K], other)                      # "other" is the later tied index
        r = oracle.verify_greedy_sequence(lp, x)
        n = next((k for k in range(K) if x[k] != a[k]), K)
        assert r["n"] == n
        assert list(r["tokens"][: n + 1]) == list(x[:n]) + [a[n]]
        assert np.all(r["tokens"][n + 1:] == -1)


def test_batch_api_on_a_generated_workload():
    import workloads
    b = workloads.make_batch(1, seqs=range(6))
    r = oracle.verify_batch(b)
    assert r.tokens.shape == (6, b.K + 1)
    for i in range(6):
        n = r.n_accepted[i]
        assert 0 <= n <= b.K
        assert list(r.tokens[i, :n]) == list(b.draft_tokens[i, :n])
        assert 0 <= r.tokens[i, n] < b.V and np.all(r.tokens[i, n + 1:] == -1)
        assert r.draw_lo[i] <= b.u_resample[i] < r.draw_hi[i]
    assert r.decisions() == int(np.sum(np.minimum(r.n_accepted + 1, b.K)) + 6)


# ------------------------------------------------------- ragged draft counts --
def test_ragged_mean_emitted_follows_truncated_geometric():
    """Each sequence with its own draft count K_b ([B] "最优猜测长度 k"): with
    per-position acceptance a = sum(min(p, q)) = 0.8 the mean number of tokens
    per round of the sequences with K_b = k is (1 - a^(k+1)) / (1 - a) ([B]
    "加速比公式"), including k = 0 (one token, never a draft)."""
    rng = np.random.default_rng(5)
    K, V, N, a = 5, 2, 24000, 0.8
    q0 = 1.5 - a
    lp = np.zeros((N, K + 1, V), np.float32)
    lq = np.tile(np.log(np.array([q0, 1 - q0], np.float32)), (N, K, 1)).astype(np.float32)
    x = (rng.random((N, K)) >= q0).astype(np.int32)
    kb = rng.integers(0, K + 1, N)
    r = oracle.verify(lp, lq, x, rng.random((N, K), np.float32), rng.random(N, np.float32), 1.0, "fp32",
                      num_drafts=kb)
    assert np.all(r.n_accepted <= kb)
    for k in range(K + 1):
        sel = kb == k
        mean = float(np.mean(r.n_accepted[sel] + 1))
        closed = (1 - a ** (k + 1)) / (1 - a)
        assert abs(mean - closed) < 5 * 1.8 / np.sqrt(sel.sum()), (k, mean, closed)
    # nothing past a sequence's own drafts is emitted or tested
    for i in range(200):
        assert np.all(r.tokens[i, r.n_accepted[i] + 1:] == -1)
        assert np.all(np.isnan(r.thr[i, kb[i]:]))


def test_zero_drafts_draw_from_p0_by_searchsorted():
    """K_b = 0: no test, the token is p_0's inverse CDF (numpy's searchsorted
    on the cumulative sum, side="right")."""
    rng = np.random.default_rng(6)
    B, K, V = 64, 3, 50
    lp = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
    lq = rng.normal(0, 2, (B, K, V)).astype(np.float32)
    ur = rng.random(B, np.float32)
    r = oracle.verify(lp, lq, rng.integers(0, V, (B, K)).astype(np.int32), rng.random((B, K), np.float32), ur,
                      0.9, "fp32", num_drafts=np.zeros(B, np.int64))
    T = float(np.float32(0.9))
    for b in range(B):
        p = softmax(lp[b, 0].astype(np.float64) / T)
        c = np.cumsum(p)
        assert r.n_accepted[b] == 0
        assert r.tokens[b, 0] == min(int(np.searchsorted(c, float(ur[b]) * c[-1], side="right")), V - 1)
        assert np.all(r.tokens[b, 1:] == -1)


def test_position_stats_worked_example():
    """Three sequences, counted by hand.  (K_b, n): (3, 1) evaluates positions
    0, 1 and accepts 0; (2, 2) evaluates 0, 1 and accepts both; (0, 0)
    evaluates nothing."""
    s = oracle.position_stats(np.array([1, 2, 0]), np.array([3, 2, 0]), K=3)
    np.testing.assert_array_equal(s, [2, 2, 0, 2, 1, 0])


def test_position_acceptance_rates_follow_sum_of_min():
    """Per-position acceptance frequency accepted[k] / evaluated[k] against
    sum(min(p_k, q_k)) ([B] "验收标准的精确数学"), with a different rate at
    every position, ragged K_b; and evaluated[k+1] = accepted[k] minus the
    sequences that accepted all K_b = k+1 drafts."""
    rng = np.random.default_rng(8)
    K, V, N = 4, 2, 20000
    q0s = np.array([0.55, 0.75, 0.9, 0.65])      # rates 0.95, 0.75, 0.6, 0.85
    lp = np.zeros((N, K + 1, V), np.float32)
    lq = np.stack([np.tile(np.log(np.array([q, 1 - q], np.float32)), (N, 1)) for q in q0s], axis=1)
    x = (rng.random((N, K)) >= q0s[None, :]).astype(np.int32)
    kb = rng.integers(1, K + 1, N)
    r = oracle.verify(lp, lq.astype(np.float32), x, rng.random((N, K), np.float32), rng.random(N, np.float32),
                      1.0, "fp32", num_drafts=kb)
    s = oracle.position_stats(r.n_accepted, kb, K)
    ev, ac = s[:K], s[K:]
    for k in range(K):
        beta = 1.5 - q0s[k]
        assert abs(ac[k] / ev[k] - beta) < 5 * np.sqrt(beta * (1 - beta) / ev[k]), (k, ac[k] / ev[k], beta)
    for k in range(K - 1):
        full = np.sum((kb == k + 1) & (r.n_accepted == k + 1))
        assert ev[k + 1] == ac[k] - full


def test_threaded_batch_equals_one_pass():
    """verify_batch(..., workers=N) splits the sequences over threads; the result
    must be the one-pass result, field for field (also with draft counts)."""
    import dataclasses
    import workloads
    b = workloads.make_batch(1, seqs=range(20), V=3000, seed=77)
    for nd in (None, workloads.ragged_draft_counts(20, b.K, seed=77, low=0)):
        bb = dataclasses.replace(b, num_drafts=nd)
        one, many = oracle.verify_batch(bb), oracle.verify_batch(bb, workers=6)
        for f in dataclasses.fields(oracle.Result):
            np.testing.assert_array_equal(getattr(one, f.name), getattr(many, f.name), err_msg=f.name)
