"""Many small random workloads against the oracle.

Each case draws its shape (B, K, V), logit dtype, temperature (greedy a quarter
of the time), logit recipe and, for about a third of the cases, per-sequence
draft counts from its own seeded generator; the HIP path must meet the parity
rule of oracle.parity on every one.  Small vocabularies (1, 2, 7 tokens) and
sizes that are and are not whole 16-byte vectors are among the choices.  A
second set draws large vocabularies with small batches, which take the split
fast draw.
"""
import dataclasses
import os
import sys

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import run_gpu
from oracle.parity import compare

pytestmark = pytest.mark.gpu

N_CASES = int(os.environ.get("SPECV_RANDOM_CASES", "64"))  # more on demand
VOCABS = [1, 2, 7, 8, 63, 64, 257, 1000, 4096, 5003, 20000]


def random_batch(case: int):
    rng = np.random.default_rng(5000 + case)
    B = int(rng.integers(1, 40))
    K = int(rng.integers(1, 13))
    V = int(rng.choice(VOCABS))
    dt = str(rng.choice(["fp32", "bf16"]))
    greedy = bool(rng.random() < 0.25)
    T = 0.0 if greedy else float(np.float32(rng.choice([0.3, 0.7, 1.0, 1.7])))
    wl = workloads.Workload(f"random-{case}", B, K, V, dt, T, float(rng.choice([0.5, 2.0, 4.0])),
                            float(rng.choice([0.0, 1.1, 3.3])), "greedy-mask" if greedy else "noise",
                            float(rng.choice([0.1, 0.8, 2.0])))
    b = workloads.make_batch(1, wl=wl, seed=case)
    if rng.random() < 0.3:
        b = dataclasses.replace(b, num_drafts=workloads.ragged_draft_counts(B, K, seed=case, low=0))
    return b


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_workload_matches_oracle(gpu_lib, case):
    """Every third case runs with the one-launch path for short rows turned
    off (spec_short_max_seqs(0)), so that rows of at most 2048 tokens also
    take the general path."""
    b = random_batch(case)
    ragged = getattr(b, "num_drafts", None) is not None
    general = case % 3 == 0
    print(f"[random] case {case}: {b.wl.describe()}{' ragged' if ragged else ''}"
          f"{' general path' if general else ''}", file=sys.stderr, flush=True)
    old = gpu_lib.short_max_seqs(0) if general else None
    try:
        out = run_gpu(gpu_lib, b)
    finally:
        if general:
            gpu_lib.short_max_seqs(old)
    compare(b, out, oracle.verify_batch(b)).check()


# Large vocabularies with small batches: the fast draw is split over several
# workgroups per sequence (rows of at least 3 blocks of 16 segments), on the
# vector and (odd V with bf16) the scalar path.
N_SPLIT_CASES = int(os.environ.get("SPECV_RANDOM_SPLIT_CASES", "32"))
SPLIT_VOCABS = [49152, 50257, 65536, 100003, 128256, 152064]


def random_split_batch(case: int):
    rng = np.random.default_rng(9000 + case)
    B = int(rng.integers(1, 25))
    K = int(rng.integers(1, 9))
    V = int(rng.choice(SPLIT_VOCABS))
    dt = str(rng.choice(["fp32", "bf16"]))
    T = float(np.float32(rng.choice([0.5, 0.7, 1.0, 1.3])))
    wl = workloads.Workload(f"random-split-{case}", B, K, V, dt, T, float(rng.choice([1.0, 2.0])),
                            float(rng.choice([0.0, 1.1])), "noise", float(rng.choice([0.3, 0.7, 1.5])))
    b = workloads.make_batch(1, wl=wl, seed=case, workers=workloads.default_workers())
    if rng.random() < 0.3:
        b = dataclasses.replace(b, num_drafts=workloads.ragged_draft_counts(B, K, seed=case, low=0))
    return b


@pytest.mark.parametrize("case", range(N_SPLIT_CASES))
def test_random_split_workload_matches_oracle(gpu_lib, case):
    b = random_split_batch(case)
    ragged = getattr(b, "num_drafts", None) is not None
    print(f"[random-split] case {case}: {b.wl.describe()}{' ragged' if ragged else ''}", file=sys.stderr,
          flush=True)
    compare(b, run_gpu(gpu_lib, b), oracle.verify_batch(b)).check()


# Large batches of short rows (at most 2048 tokens): the one-launch path at
# any batch size, on both capacities (rows of at most 1024 tokens, and up to
# 2048), against the oracle on every sequence.
N_SHORT_CASES = int(os.environ.get("SPECV_RANDOM_SHORT_CASES", "6"))
SHORT_VOCABS = [2, 63, 257, 1000, 1023, 1024, 1025, 1500, 2047, 2048]


def random_short_batch(case: int):
    rng = np.random.default_rng(13000 + case)
    B = int(rng.integers(300, 4000))
    K = int(rng.integers(1, 9))
    V = int(rng.choice(SHORT_VOCABS))
    dt = str(rng.choice(["fp32", "bf16"]))
    T = float(np.float32(rng.choice([0.3, 0.7, 1.0, 1.7])))
    wl = workloads.Workload(f"random-short-{case}", B, K, V, dt, T, float(rng.choice([0.5, 2.0])),
                            float(rng.choice([0.0, 1.1, 3.3])), "noise", float(rng.choice([0.1, 0.8, 2.0])))
    b = workloads.make_batch(1, wl=wl, seed=case, workers=workloads.default_workers())
    if rng.random() < 0.3:
        b = dataclasses.replace(b, num_drafts=workloads.ragged_draft_counts(B, K, seed=case, low=0))
    return b


@pytest.mark.parametrize("case", range(N_SHORT_CASES))
def test_random_large_batch_of_short_rows_matches_oracle(gpu_lib, case):
    b = random_short_batch(case)
    ragged = getattr(b, "num_drafts", None) is not None
    print(f"[random-short] case {case}: {b.wl.describe()}{' ragged' if ragged else ''}", file=sys.stderr,
          flush=True)
    out = run_gpu(gpu_lib, b)
    assert np.all(out.flags & gpu_lib.FLAG_FP64), "short rows: every draw is an fp64 draw (one-launch path)"
    compare(b, out, oracle.verify_batch(b, workers=workloads.default_workers())).check()
