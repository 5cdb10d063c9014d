"""The seeded input generator: determinism, rounding, uniforms and the
statistical shape the workloads are meant to have."""
import dataclasses

import numpy as np
import pytest
from scipy.special import softmax
from scipy.stats import chi2

import oracle
import workloads


def test_workload_table():
    shapes = [(w.B, w.K, w.V, w.dtype, w.greedy) for w in workloads.WORKLOADS]
    assert shapes == [(1, 4, 1000, "fp32", False), (64, 5, 32000, "bf16", False),
                      (256, 8, 128256, "bf16", False), (1024, 4, 256000, "fp32", False),
                      (512, 8, 152064, "bf16", True)]
    assert workloads.WORKLOADS[2].T == float(np.float32(0.7))


def test_sequences_are_deterministic_and_independent_of_batch_composition():
    a = workloads.make_batch(1, seqs=[3, 7])
    b = workloads.make_batch(1, seqs=[7, 3, 5])
    np.testing.assert_array_equal(a.logits_p[1], b.logits_p[0])
    np.testing.assert_array_equal(a.logits_q[0], b.logits_q[1])
    np.testing.assert_array_equal(a.draft_tokens[1], b.draft_tokens[0])
    np.testing.assert_array_equal(a.u_resample[0], b.u_resample[1])
    c = workloads.make_batch(1, seqs=[3, 7], seed=7)
    assert not np.array_equal(a.logits_p, c.logits_p)


def test_parallel_generation_matches_serial():
    a = workloads.make_batch(0, seqs=[0])
    b = workloads.make_batch(1, seqs=range(5), workers=2)
    c = workloads.make_batch(1, seqs=range(5), workers=1)
    np.testing.assert_array_equal(b.logits_p, c.logits_p)
    np.testing.assert_array_equal(b.draft_tokens, c.draft_tokens)
    assert a.logits_p.dtype == np.float32 and b.logits_p.dtype == np.uint16


def test_bf16_rounding_is_round_to_nearest_even():
    import torch
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 3, 100000), rng.normal(0, 1e-3, 1000),
                        [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0]]).astype(np.float32)
    ours = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    # exact ties go to the even neighbour
    assert workloads.f32_to_bf16_bits(np.array([1.0 + 2 ** -8], np.float32))[0] == 0x3F80
    assert workloads.f32_to_bf16_bits(np.array([1.0 + 3 * 2 ** -8], np.float32))[0] == 0x3F82


def test_uniforms_are_exact_and_inside_the_open_interval():
    b = workloads.make_batch(1, seqs=range(16))
    for u in (b.u_accept.ravel(), b.u_resample):
        assert u.dtype == np.float32
        assert np.all(u > 0) and np.all(u < 1)
        i = u.astype(np.float64) * 2 ** 23 - 0.5
        np.testing.assert_array_equal(i, np.round(i))


def test_greedy_workload_has_no_draft_logits_and_half_argmax_drafts():
    b = workloads.make_batch(4, seqs=range(24), V=4096)
    assert b.logits_q is None
    lp = oracle.widen(b.logits_p, "bf16")
    hits = np.mean([b.draft_tokens[s, k] == np.argmax(lp[s, k]) for s in range(24) for k in range(b.K)])
    assert 0.35 < hits < 0.65


def test_small_workload_acceptance_in_stated_range():
    """The small bf16 workload is meant to accept roughly 0.6-0.7 per position."""
    b = workloads.make_batch(1, seqs=range(12))
    beta = []
    for s in range(12):
        yp = oracle.widen(b.logits_p[s], "bf16") / b.T
        yq = oracle.widen(b.logits_q[s], "bf16") / b.T
        beta += [np.minimum(softmax(yp[k]), softmax(yq[k])).sum() for k in range(b.K)]
    assert 0.6 <= np.mean(beta) <= 0.7, np.mean(beta)


def test_draft_tokens_follow_q():
    """Gumbel-max drafts are distributed as softmax(draft logits / T)."""
    wl = dataclasses.replace(workloads.WORKLOADS[0], V=6, K=1, B=1)
    N = 20000
    b = workloads.make_batch(0, seqs=range(N), wl=wl)
    # rows differ per sequence, so bucket each draw by the rank of the chosen
    # token in its own row: the expected count at rank r is the sum over
    # sequences of q at that rank
    yq = oracle.widen(b.logits_q[:, 0], "fp32") / b.T
    q = softmax(yq, axis=1)
    x = b.draft_tokens[:, 0]
    ranks = np.argsort(np.argsort(-q, axis=1), axis=1)
    got = np.bincount(ranks[np.arange(N), x], minlength=6)
    want = np.array([np.sum(q[ranks == r]) for r in range(6)])
    stat = np.sum((got - want) ** 2 / want)
    assert chi2.sf(stat, 5) > 1e-3, (got, want)


@pytest.mark.parametrize("cfg", [0, 1, 3])
def test_generated_shapes(cfg):
    b = workloads.make_batch(cfg, seqs=range(2), V=2048)
    assert b.logits_p.shape == (2, b.K + 1, 2048)
    assert b.logits_q.shape == (2, b.K, 2048)
    assert b.draft_tokens.shape == (2, b.K) and b.draft_tokens.dtype == np.int32
    assert np.all((b.draft_tokens >= 0) & (b.draft_tokens < 2048))


def test_tree_batches_are_valid_and_deterministic():
    a = workloads.make_tree_batch(6, 20, 500, "bf16", seed=3, workers=3)
    b = workloads.make_tree_batch(6, 20, 500, "bf16", seed=3)
    np.testing.assert_array_equal(a.logits, b.logits)
    np.testing.assert_array_equal(a.parents, b.parents)
    np.testing.assert_array_equal(a.tokens, b.tokens)
    assert np.all(a.parents[:, 0] == -1)
    v = np.arange(1, 20)
    assert np.all((a.parents[:, 1:] >= 0) & (a.parents[:, 1:] < v))
    assert a.logits.dtype == np.uint16 and a.logits.shape == (6, 20, 500)


def test_histories_are_deterministic_and_self_similar():
    h1, n1 = workloads.make_histories(8, 2000, 32000, seed=4, workers=4)
    h2, n2 = workloads.make_histories(8, 2000, 32000, seed=4)
    np.testing.assert_array_equal(h1, h2)
    np.testing.assert_array_equal(n1, n2)
    assert np.all((n1 >= 1000) & (n1 <= 2000))
    for b in range(8):
        assert np.all(h1[b, n1[b]:] == -1) and np.all((h1[b, : n1[b]] >= 0) & (h1[b, : n1[b]] < 32000))
    # copies make repeated 4-grams common
    h = h1[0, : n1[0]]
    grams = {tuple(h[i:i + 4]) for i in range(len(h) - 3)}
    assert len(grams) < 0.9 * (len(h) - 3)
