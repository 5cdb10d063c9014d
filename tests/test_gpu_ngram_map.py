"""GPU parity of the n-gram map (spec_ngram_map_update) against oracle.ngram:
a table built from a history and then fed the tokens each step adds must
propose, after every call, exactly what the oracle's scan of the history so
far proposes (bit-exact drafts and counts)."""
import sys

import numpy as np
import pytest

import workloads
from oracle import ngram

pytestmark = pytest.mark.gpu


def _cap(L, n_min, n_max):
    """Slots for a history of L tokens: twice the most distinct n-grams it can hold."""
    need = 2 * (n_max - n_min + 1) * max(L, 1)
    return max(64, 1 << (need - 1).bit_length())


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _update(sv, tables, cap, h, old, new, n_min, n_max, hits, K):
    import torch
    d, c, s = sv.ngram_map_update(tables, cap, h, _dev(old), _dev(new), n_min, n_max, hits, K)
    torch.cuda.synchronize()
    return d.cpu().numpy(), c.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("B,L,vocab,n_min,n_max,hits,K", [(32, 3000, 50, 1, 4, 1, 5), (16, 2000, 32000, 2, 8, 2, 8),
                                                          (8, 1500, 3, 1, 16, 3, 32), (24, 4000, 500, 3, 3, 1, 1)],
                         ids=lambda x: str(x))
def test_map_follows_the_oracle_as_histories_grow(gpu_lib, B, L, vocab, n_min, n_max, hits, K):
    import torch
    hist, lens = workloads.make_histories(B, L, vocab, seed=3 * L + vocab, workers=workloads.default_workers())
    rng = np.random.default_rng(L + vocab)
    steps = 8
    m = rng.integers(1, K + 2, (steps, B)).astype(np.int32)  # tokens each step adds
    start = np.maximum(lens - m.sum(0), 0).astype(np.int32)
    cap = _cap(L, n_min, n_max)
    tables = torch.empty(gpu_lib.ngram_map_bytes(B, cap), dtype=torch.uint8, device="cuda")  # cleared by the build
    h = _dev(hist)
    print(f"[ngram-map] B={B} L={L} vocab={vocab} n={n_min}..{n_max} hits={hits} K={K} capacity={cap}",
          file=sys.stderr, flush=True)
    old, new = np.zeros(B, np.int32), start
    for step in range(steps + 1):
        d, c, st = _update(gpu_lib, tables, cap, h, old, new, n_min, n_max, hits, K)
        rd, rc = ngram.propose(hist, new, n_min, n_max, hits, K)
        assert not st.any(), f"step {step}: a table overflowed"
        np.testing.assert_array_equal(c, rc, err_msg=f"step {step}: counts")
        np.testing.assert_array_equal(d, rd, err_msg=f"step {step}: drafts")
        if step < steps:
            old, new = new, np.minimum(new + m[step], lens).astype(np.int32)


def test_map_at_edge_lengths(gpu_lib):
    """Builds at lengths 0..19, random and full lengths, and past L_max
    (clamped); then one update that adds nothing (len_old == len_new) and one
    whose len_old exceeds len_new (clamped to it: nothing added)."""
    import torch
    rng = np.random.default_rng(7)
    B, L = 40, 64
    hist = rng.integers(0, 3, (B, L)).astype(np.int32)
    lens = np.concatenate([np.arange(0, 20), rng.integers(0, L + 1, 18), [L, L + 50]]).astype(np.int32)
    cap = _cap(L, 1, 5)
    tables = torch.empty(gpu_lib.ngram_map_bytes(B, cap), dtype=torch.uint8, device="cuda")
    h = _dev(hist)
    clamped = np.minimum(lens, L)
    rd, rc = ngram.propose(hist, clamped, 1, 5, 1, 6)
    for old in (np.zeros(B, np.int32), lens, lens + 7):
        d, c, st = _update(gpu_lib, tables, cap, h, old, lens, 1, 5, 1, 6)
        assert not st.any()
        np.testing.assert_array_equal(c, rc)
        np.testing.assert_array_equal(d, rd)


def test_full_table_reports_and_rebuild_recovers(gpu_lib):
    """A table of 64 slots cannot hold the n-grams of 200-400 varied tokens: the
    call reports SPECV_NGRAM_MAP_FULL and proposes nothing, and so do later
    updates, until a call with len_old == 0 rebuilds it from a history that
    fits."""
    import torch
    B, L, cap = 4, 400, 64
    hist, lens = workloads.make_histories(B, L, 32000, seed=5, p_copy=0.0)  # 200 to 400 tokens
    tables = torch.empty(gpu_lib.ngram_map_bytes(B, cap), dtype=torch.uint8, device="cuda")
    h = _dev(hist)
    d, c, st = _update(gpu_lib, tables, cap, h, np.zeros(B, np.int32), lens - 10, 1, 4, 1, 5)
    assert np.all(st == gpu_lib.NGRAM_MAP_FULL) and not c.any() and np.all(d == -1)
    d, c, st = _update(gpu_lib, tables, cap, h, lens - 10, lens, 1, 4, 1, 5)
    assert np.all(st == gpu_lib.NGRAM_MAP_FULL) and not c.any()
    short = np.full(B, 8, np.int32)  # at most 4 * 8 n-grams
    d, c, st = _update(gpu_lib, tables, cap, h, np.zeros(B, np.int32), short, 1, 4, 1, 5)
    rd, rc = ngram.propose(hist, short, 1, 4, 1, 5)
    assert not st.any()
    np.testing.assert_array_equal(c, rc)
    np.testing.assert_array_equal(d, rd)


def test_long_histories_match_the_scan(gpu_lib):
    """Histories of up to 40000 tokens: after the build and after each of four
    updates the map proposes what the scan kernel (spec_ngram_propose)
    proposes for the same lengths; the oracle checks the last step."""
    import torch
    B, L, vocab, n_min, n_max, hits, K = 8, 40000, 1000, 1, 4, 1, 5
    hist, lens = workloads.make_histories(B, L, vocab, seed=41, workers=workloads.default_workers())
    cap = _cap(L, n_min, n_max)
    tables = torch.empty(gpu_lib.ngram_map_bytes(B, cap), dtype=torch.uint8, device="cuda")
    h = _dev(hist)
    old, new = np.zeros(B, np.int32), (lens - 24).astype(np.int32)
    for step in range(5):
        d, c, st = _update(gpu_lib, tables, cap, h, old, new, n_min, n_max, hits, K)
        sd, sc = gpu_lib.ngram_propose(h, _dev(new), n_min, n_max, hits, K)
        torch.cuda.synchronize()
        assert not st.any()
        np.testing.assert_array_equal(c, sc.cpu().numpy(), err_msg=f"step {step}")
        np.testing.assert_array_equal(d, sd.cpu().numpy(), err_msg=f"step {step}")
        old, new = new, (new + 6).astype(np.int32)
    rd, rc = ngram.propose(hist, old, n_min, n_max, hits, K)
    np.testing.assert_array_equal(c, rc)
    np.testing.assert_array_equal(d, rd)


N_RANDOM_MAP = int(__import__("os").environ.get("SPECV_RANDOM_MAP_CASES", "8"))


@pytest.mark.parametrize("case", range(N_RANDOM_MAP))
def test_random_map_schedules_match_oracle(gpu_lib, case):
    """Random histories, sizes, hits, K and growth schedules (one to K + 1
    tokens per step, some steps adding none, some sequences rebuilt midway
    with previous length 0) against the oracle after every call."""
    import torch
    rng = np.random.default_rng(6000 + case)
    B = int(rng.integers(1, 24))
    L = int(rng.choice([40, 300, 2000, 5000]))
    vocab = int(rng.choice([2, 7, 300, 32000]))
    n_max = int(rng.integers(1, 17))
    n_min = int(rng.integers(1, n_max + 1))
    hits = int(rng.integers(1, 4))
    K = int(rng.integers(1, 9))
    hist, lens = workloads.make_histories(B, L, vocab, seed=case)
    steps = 6
    m = rng.integers(0, K + 2, (steps, B)).astype(np.int32)
    start = np.maximum(lens - m.sum(0), 0).astype(np.int32)
    cap = _cap(L, n_min, n_max)
    tables = torch.empty(gpu_lib.ngram_map_bytes(B, cap), dtype=torch.uint8, device="cuda")
    h = _dev(hist)
    print(f"[ngram-map] random case {case}: B={B} L={L} vocab={vocab} n={n_min}..{n_max} hits={hits} K={K}",
          file=sys.stderr, flush=True)
    old, new = np.zeros(B, np.int32), start
    for step in range(steps + 1):
        d, c, st = _update(gpu_lib, tables, cap, h, old, new, n_min, n_max, hits, K)
        rd, rc = ngram.propose(hist, new, n_min, n_max, hits, K)
        assert not st.any()
        np.testing.assert_array_equal(c, rc, err_msg=f"step {step}")
        np.testing.assert_array_equal(d, rd, err_msg=f"step {step}")
        if step < steps:
            nxt = np.minimum(new + m[step], lens).astype(np.int32)
            rebuild = rng.random(B) < 0.15  # these sequences are rebuilt from scratch next call
            old = np.where(rebuild, 0, new).astype(np.int32)
            new = nxt
