"""The fast draw split over several workgroups per sequence.

A batch of at most 128 sequences leaves CUs idle when each sequence's
decisive rows are streamed by one workgroup, so the library gives a sequence
up to 16 workgroups (one per idle CU, at most one per block of 16 segments,
and none for rows of fewer than 3 blocks); the last of them to finish makes
the draw.  These cases run that path
against the oracle (the parity rule of oracle.parity), on the vector and the
scalar path, with per-sequence draft counts, and check that sequences get the
same outputs whether they run split (in a small batch) or not (in a batch of
more than 128).
"""
import dataclasses
import sys

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import run_gpu
from oracle.parity import compare

pytestmark = pytest.mark.gpu

MAX_SPLIT, SPLIT_MAX_SEQS, WAVES, MIN_BLOCKS = 16, 128, 16, 3


def expected_split(B: int, V: int, dtype: str, vec: bool) -> int:
    """Workgroups per sequence that the split rule gives on this device (for the log and to
    make sure a case meant to split does)."""
    import torch
    if B > SPLIT_MAX_SEQS:
        return 1
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    per_vec = (8 if dtype == "bf16" else 4) if vec else 1
    units = V // per_vec if vec else V
    total = max(1, -(-units // (64 * (2 if vec else 8))))
    iters = -(-total // 1024)
    nseg = -(-total // iters)
    blocks = -(-nseg // WAVES)
    return 1 if blocks < MIN_BLOCKS else max(1, min(cus // B, blocks, MAX_SPLIT))


def sv_flag_fp64() -> int:
    import speculative_sampling_verify_spec_amd as sv
    return sv.FLAG_FP64


def scalar_workload() -> workloads.Workload:
    # bf16 with an odd V: rows are not whole 16-byte vectors, so the scalar path runs
    return workloads.Workload("odd-V", 4, 6, 100003, "bf16", float(np.float32(0.8)), 2.0, 1.1, "noise", 0.8)


CASES = {
    "headline-1": lambda: workloads.make_batch(2, seqs=range(1)),
    "headline-16": lambda: workloads.make_batch(2, seqs=range(16), workers=workloads.default_workers()),
    "headline-100": lambda: workloads.make_batch(2, seqs=range(100), workers=workloads.default_workers()),
    # both sides of the switch: the largest split batch (two workgroups per sequence on 256
    # CUs) and the smallest batch that no longer splits
    "headline-128": lambda: workloads.make_batch(2, seqs=range(128), workers=workloads.default_workers()),
    "headline-129": lambda: workloads.make_batch(2, seqs=range(129), workers=workloads.default_workers()),
    "sharp-fp32-8": lambda: workloads.make_batch(3, seqs=range(8), workers=workloads.default_workers()),
    "scalar-odd-V-4": lambda: workloads.make_batch(1, wl=scalar_workload(), workers=workloads.default_workers()),
    "k32-4": lambda: workloads.make_batch(1, wl=workloads.Workload("k32", 4, 32, 65536, "bf16", float(np.float32(0.9)),
                                                                    2.0, 1.1, "noise", 0.6)),
    "headline-32-ragged": lambda: dataclasses.replace(
        workloads.make_batch(2, seqs=range(32), workers=workloads.default_workers()),
        num_drafts=workloads.ragged_draft_counts(32, 8, seed=7, low=0)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_split_draw_matches_oracle(gpu_lib, name):
    b = CASES[name]()
    vec = (b.V * (2 if b.dtype == "bf16" else 4)) % 16 == 0
    split = expected_split(b.B, b.V, b.dtype, vec)
    print(f"[split] {name}: {b.wl.describe()} split={split}", file=sys.stderr, flush=True)
    assert split == 1 if b.B > SPLIT_MAX_SEQS else split > 1
    compare(b, run_gpu(gpu_lib, b), oracle.verify_batch(b)).check()


def test_split_and_unsplit_give_the_same_outputs(gpu_lib):
    # 192 sequences (config 1's recipe at V = 49152) run unsplit; their first
    # 64, on their own, split in three.  At this V both batches take the
    # sweep's small shape, so their normalisers agree to the bit.
    big = workloads.make_batch(1, seqs=range(192), V=49152, workers=workloads.default_workers())
    small = dataclasses.replace(big, wl=dataclasses.replace(big.wl, B=64), seqs=big.seqs[:64],
                                logits_p=big.logits_p[:64], logits_q=big.logits_q[:64],
                                draft_tokens=big.draft_tokens[:64], u_accept=big.u_accept[:64],
                                u_resample=big.u_resample[:64])
    assert expected_split(192, big.V, big.dtype, True) == 1
    assert expected_split(64, big.V, big.dtype, True) > 1
    print(f"[split] {big.wl.describe()}: 192 unsplit against 64 split {expected_split(64, big.V, big.dtype, True)}",
          file=sys.stderr, flush=True)
    g_big, g_small = run_gpu(gpu_lib, big), run_gpu(gpu_lib, small)
    np.testing.assert_array_equal(g_small.n, g_big.n[:64])
    np.testing.assert_array_equal(g_small.tokens, g_big.tokens[:64])
    # a split draw may also go to the fp64 path when a published value is not
    # yet visible to the last workgroup; its token is the same
    fp64 = int(sv_flag_fp64())
    extra = int(np.count_nonzero((g_small.flags & fp64) & ~(g_big.flags[:64] & fp64)))
    print(f"[split] draws sent to the fp64 path by the split alone: {extra}", file=sys.stderr, flush=True)
    np.testing.assert_array_equal(g_small.flags & ~fp64, g_big.flags[:64] & ~fp64)
    np.testing.assert_array_equal(g_small.logz, g_big.logz[:64])
    compare(small, g_small, oracle.verify_batch(small)).check()
