"""GPU parity of the n-gram (prompt-lookup) proposer against oracle.ngram:
bit-exact drafts and counts."""
import os
import sys

import numpy as np
import pytest

import workloads
from oracle import ngram

pytestmark = pytest.mark.gpu


def _run(gpu_lib, hist, lens, n_min, n_max, hits, K):
    import torch
    d, c = gpu_lib.ngram_propose(torch.from_numpy(np.ascontiguousarray(hist)).cuda(),
                                 torch.from_numpy(np.ascontiguousarray(lens)).cuda(), n_min, n_max, hits, K)
    torch.cuda.synchronize()
    return d.cpu().numpy(), c.cpu().numpy()


@pytest.mark.parametrize("B,L,vocab,n_min,n_max,hits,K", [(64, 4096, 32000, 1, 4, 1, 5), (32, 20000, 500, 2, 8, 2, 8),
                                                          (16, 300, 3, 1, 16, 3, 32), (128, 2048, 50000, 3, 3, 1, 1),
                                                          (8, 40000, 1000, 1, 4, 1, 5)],
                         ids=lambda x: str(x))
def test_proposals_match_oracle(gpu_lib, B, L, vocab, n_min, n_max, hits, K):
    hist, lens = workloads.make_histories(B, L, vocab, seed=L + vocab, workers=workloads.default_workers())
    print(f"[ngram] B={B} L={L} vocab={vocab} n={n_min}..{n_max} hits={hits} K={K}", file=sys.stderr, flush=True)
    d, c = _run(gpu_lib, hist, lens, n_min, n_max, hits, K)
    rd, rc = ngram.propose(hist, lens, n_min, n_max, hits, K)
    np.testing.assert_array_equal(c, rc)
    np.testing.assert_array_equal(d, rd)


def test_edge_lengths(gpu_lib):
    rng = np.random.default_rng(7)
    B, L = 40, 64
    hist = rng.integers(0, 3, (B, L)).astype(np.int32)
    lens = np.concatenate([np.arange(0, 20), rng.integers(0, L + 1, 18), [L, L + 50]]).astype(np.int32)
    d, c = _run(gpu_lib, hist, lens, 1, 5, 1, 6)
    rd, rc = ngram.propose(hist, np.minimum(lens, L), 1, 5, 1, 6)
    np.testing.assert_array_equal(c, rc)
    np.testing.assert_array_equal(d, rd)


N_RANDOM = int(os.environ.get("SPECV_RANDOM_NGRAM_CASES", "12"))


@pytest.mark.parametrize("case", range(N_RANDOM))
def test_random_proposals_match_oracle(gpu_lib, case):
    # shapes on both sides of the four preloaded rounds (16385 tokens), all n
    # ranges, small and large vocabularies, padded rows with short histories
    rng = np.random.default_rng(7000 + case)
    B = int(rng.integers(1, 17))
    L = int(rng.choice([5, 100, 4097, 8193, 16385, 16386, 24000]))
    vocab = int(rng.choice([2, 7, 300, 32000]))
    n_max = int(rng.integers(1, 17))
    n_min = int(rng.integers(1, n_max + 1))
    hits = int(rng.integers(1, 4))
    K = int(rng.integers(1, 33))
    hist, lens = workloads.make_histories(B, L, vocab, seed=case, workers=workloads.default_workers())
    lens = np.minimum(lens, rng.integers(0, L + 1, B)).astype(np.int32) if rng.random() < 0.3 else lens
    print(f"[ngram-random] case {case}: B={B} L={L} vocab={vocab} n={n_min}..{n_max} hits={hits} K={K}",
          file=sys.stderr, flush=True)
    d, c = _run(gpu_lib, hist, lens, n_min, n_max, hits, K)
    rd, rc = ngram.propose(hist, lens, n_min, n_max, hits, K)
    np.testing.assert_array_equal(c, rc)
    np.testing.assert_array_equal(d, rd)


def test_vector_and_element_loads_agree(gpu_lib):
    # rows of L_max % 4 == 0 in a 16-byte aligned history are read as 16-byte
    # vectors; the same rows one int32 off that alignment are read token by
    # token: both must give the oracle's proposals
    import torch
    B, L = 48, 12288
    hist, lens = workloads.make_histories(B, L, 50, seed=99, workers=workloads.default_workers())
    h16 = torch.from_numpy(hist).cuda()
    buf = torch.empty(B * L + 1, dtype=torch.int32, device="cuda")
    buf[1:] = h16.view(-1)
    h4 = buf[1:].view(B, L)
    assert h16.data_ptr() % 16 == 0 and h4.data_ptr() % 16 == 4
    ln = torch.from_numpy(lens).cuda()
    d1, c1 = gpu_lib.ngram_propose(h16, ln, 1, 8, 1, 6)
    d2, c2 = gpu_lib.ngram_propose(h4, ln, 1, 8, 1, 6)
    torch.cuda.synchronize()
    rd, rc = ngram.propose(hist, lens, 1, 8, 1, 6)
    for d, c in ((d1, c1), (d2, c2)):
        np.testing.assert_array_equal(c.cpu().numpy(), rc)
        np.testing.assert_array_equal(d.cpu().numpy(), rd)
