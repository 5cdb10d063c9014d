"""GPU parity of spec_verify_ragged: per-sequence draft counts K_b and the
per-position acceptance counters, against the fp64 oracle."""
import dataclasses
import sys

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import run_gpu
from oracle.parity import compare

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _ragged(cfg, B=None, low=0, seed=11, V=None):
    wl = workloads.WORKLOADS[cfg]
    if B is not None:
        wl = dataclasses.replace(wl, B=B)
    if V is not None:
        wl = dataclasses.replace(wl, V=V)
    b = workloads.make_batch(cfg, wl=wl, seed=seed, workers=workloads.default_workers())
    return dataclasses.replace(b, num_drafts=workloads.ragged_draft_counts(b.B, b.K, seed=seed, low=low))


def _stats_tensor(K):
    import torch
    return torch.zeros(2 * K, dtype=torch.int64, device="cuda")


@pytest.mark.parametrize("cfg,B,V", [(1, None, None), (2, 64, None), (0, None, None)])
def test_ragged_sampling_matches_oracle(gpu_lib, cfg, B, V):
    b = _ragged(cfg, B=B, V=V)
    say(f"[ragged] workload {cfg} B={b.B} K={b.K} V={b.V} K_b from {b.num_drafts.min()} to {b.num_drafts.max()}")
    st = _stats_tensor(b.K)
    g = run_gpu(gpu_lib, b, position_stats=st)
    ref = oracle.verify_batch(b)
    rep = compare(b, g, ref)
    say(f"[ragged] decisions={rep.decisions} excused={rep.excused}")
    rep.check()
    assert np.all(g.n <= b.num_drafts)
    # the counters are exactly the counts of the GPU's own outcomes
    np.testing.assert_array_equal(st.cpu().numpy(), oracle.position_stats(g.n, b.num_drafts, b.K))


@pytest.mark.parametrize("low", [0, 1])
def test_ragged_headline_full_size(gpu_lib, low):
    """The headline shape at full size (B=256, K=8, V=128256 bf16, T=0.7) with
    K_b uniform on [low, 8]: the ragged sweep's large shape (21760 workgroups)
    and the unsplit fast draw, log Z of the used rows included."""
    b = _ragged(2, low=low, seed=41 + low)
    say(f"[ragged] headline B={b.B} K_b from {b.num_drafts.min()} to {b.num_drafts.max()}")
    st = _stats_tensor(b.K)
    g = run_gpu(gpu_lib, b, position_stats=st)
    ref = oracle.verify_batch(b, workers=workloads.default_workers())
    rep = compare(b, g, ref)
    say(f"[ragged] headline: decisions={rep.decisions} excused={rep.excused} max_logz_err={rep.max_logz_err:.2e}")
    rep.check()
    np.testing.assert_array_equal(st.cpu().numpy(), oracle.position_stats(g.n, b.num_drafts, b.K))


def test_ragged_greedy_full_size(gpu_lib):
    """The greedy workload at full size (B=512, K=8, V=152064 bf16) with K_b
    uniform on [0, 8]: the ragged arg-max sweep's large shape (23040
    workgroups), bit-exact."""
    b = _ragged(4, seed=43)
    say(f"[ragged] greedy B={b.B} K_b from {b.num_drafts.min()} to {b.num_drafts.max()}")
    st = _stats_tensor(b.K)
    g = run_gpu(gpu_lib, b, position_stats=st)
    ref = oracle.verify_batch(b, workers=workloads.default_workers())
    np.testing.assert_array_equal(g.n, ref.n_accepted)
    np.testing.assert_array_equal(g.tokens, ref.tokens)
    np.testing.assert_array_equal(st.cpu().numpy(), oracle.position_stats(ref.n_accepted, b.num_drafts, b.K))


def test_ragged_greedy_matches_oracle(gpu_lib):
    b = _ragged(4, B=96, V=30000, seed=12)
    st = _stats_tensor(b.K)
    g = run_gpu(gpu_lib, b, position_stats=st)
    ref = oracle.verify_batch(b)
    np.testing.assert_array_equal(g.n, ref.n_accepted)
    np.testing.assert_array_equal(g.tokens, ref.tokens)
    np.testing.assert_array_equal(st.cpu().numpy(), oracle.position_stats(ref.n_accepted, b.num_drafts, b.K))


def test_full_counts_equal_the_fixed_entry_point(gpu_lib):
    """K_b = K everywhere: spec_verify_ragged gives what spec_verify gives."""
    b = workloads.make_batch(1, seed=13, workers=workloads.default_workers())
    fixed = run_gpu(gpu_lib, b)
    rag = run_gpu(gpu_lib, dataclasses.replace(b, num_drafts=np.full(b.B, b.K, np.int32)))
    np.testing.assert_array_equal(fixed.tokens, rag.tokens)
    np.testing.assert_array_equal(fixed.n, rag.n)


def test_counts_outside_the_range_are_clamped_and_counters_accumulate(gpu_lib):
    b = workloads.make_batch(1, seed=14, workers=workloads.default_workers())
    kb = workloads.ragged_draft_counts(b.B, b.K, seed=14, low=0)
    wild = kb.copy()
    wild[::4] = -3
    wild[1::4] = b.K + 5
    clamped = np.clip(wild, 0, b.K)
    st = _stats_tensor(b.K)
    g1 = run_gpu(gpu_lib, dataclasses.replace(b, num_drafts=wild), position_stats=st)
    g2 = run_gpu(gpu_lib, dataclasses.replace(b, num_drafts=clamped), position_stats=st)
    np.testing.assert_array_equal(g1.tokens, g2.tokens)
    np.testing.assert_array_equal(g1.n, g2.n)
    ref = oracle.verify_batch(dataclasses.replace(b, num_drafts=clamped))
    compare(dataclasses.replace(b, num_drafts=clamped), g2, ref).check()
    np.testing.assert_array_equal(st.cpu().numpy(), 2 * oracle.position_stats(g2.n, clamped, b.K))
