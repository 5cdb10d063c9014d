"""Draws placed right next to an interval edge.

The fp32 draw certifies a token only when t = u Z lies further from both ends
of the token's interval than its error bound, which is of the order of 1e-6
of the mass.  Uniforms chosen so that t lies between 1e-11 and 1e-7 of the mass
above the lower end of the oracle's token therefore must all go to the fp64
draw (SPECV_FLAG_FP64).  The fp64 draw is good to ~1e-12, so it must return the
oracle's token exactly; no near-tie excuse applies at these margins.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import speculative_sampling_verify_spec_amd as sv
import workloads
from gpu_helpers import run_gpu
from oracle.parity import compare

pytestmark = pytest.mark.gpu


def edge_uniforms(b, ref, lo_min=1e-3, margin_lo=1e-11, margin_hi=1e-7):
    """Replace u_resample of every sequence whose oracle token interval
    [lo, hi) allows it by the smallest float32 above lo (kept when its margin
    u - lo lies in (margin_lo, margin_hi)).  Returns the new uniforms, the
    chosen sequences and their tokens."""
    ur = b.u_resample.copy()
    chosen, tokens = [], []
    for s in range(b.B):
        n = int(ref.n_accepted[s])
        j = int(ref.tokens[s, n])
        lo, hi = oracle.draw_interval(b.logits_p[s], b.logits_q[s], n, j, 0.5, b.T, b.dtype)
        if lo < lo_min:
            continue
        u = np.float32(lo)
        if float(u) <= lo:
            u = np.nextafter(u, np.float32(1.0))
        margin = float(u) - lo
        if not (margin_lo < margin < margin_hi) or hi - float(u) < 1e-6:
            continue
        ur[s] = u
        chosen.append(s)
        tokens.append(j)
    return ur, np.array(chosen, dtype=np.int64), np.array(tokens, dtype=np.int64)


# V = 999, 1000 and 2000: rows of one and two fp64 chunks; batches of at most
# one sequence per CU take the one-launch path for short rows, which draws
# every token in fp64 (V = 999: element loads, not 16-byte vectors)
@pytest.mark.parametrize("cfg,nseq,V", [(1, None, None), (2, 32, None), (3, 16, None), (1, 48, 1000), (0, 40, 2000),
                                        (1, 24, 999)],
                         ids=["small-bf16", "headline-bf16", "sharp-fp32", "V1000-bf16", "V2000-fp32",
                              "V999-bf16-scalar"])
def test_draws_at_an_edge_go_to_fp64_and_match(gpu_lib, cfg, nseq, V):
    seqs = None if nseq is None else range(nseq)
    b = workloads.make_batch(cfg, seqs=seqs, workers=workloads.default_workers(), V=V)
    ref = oracle.verify_batch(b)
    ur, chosen, tokens = edge_uniforms(b, ref)
    print(f"cfg {cfg}: {len(chosen)} of {b.B} sequences get an edge uniform", flush=True)
    assert len(chosen) >= b.B // 4
    b2 = dataclasses.replace(b, u_resample=ur)
    g = run_gpu(gpu_lib, b2)
    ref2 = oracle.verify_batch(b2)
    # the accept decisions do not change; the oracle keeps its token
    np.testing.assert_array_equal(ref2.n_accepted, ref.n_accepted)
    np.testing.assert_array_equal(ref2.tokens[chosen, ref.n_accepted[chosen]], tokens)
    assert np.all(g.flags[chosen] & sv.FLAG_FP64), "an edge draw was certified by the fp32 path"
    same = chosen[g.n[chosen] == ref2.n_accepted[chosen]]
    np.testing.assert_array_equal(g.tokens[same], ref2.tokens[same])
    compare(b2, g, ref2).check()


def _head(b, m):
    """The first m sequences of a batch."""
    return dataclasses.replace(b, wl=dataclasses.replace(b.wl, B=m), seqs=b.seqs[:m], logits_p=b.logits_p[:m],
                               logits_q=None if b.logits_q is None else b.logits_q[:m],
                               draft_tokens=b.draft_tokens[:m], u_accept=b.u_accept[:m],
                               u_resample=b.u_resample[:m])


@pytest.mark.parametrize("cfg,V", [(1, None), (1, 4001), (0, 6000)],
                         ids=["small-bf16", "V4001-bf16-scalar", "V6000-fp32"])
def test_sums_ahead_match_the_queued_path(gpu_lib, cfg, V):
    """Batches of at most half as many sequences as CUs compute every
    sequence's fp64 chunk sums in k_verify's spare workgroups, and the fp64
    draw runs its select alone; larger batches queue the uncertain draws and
    run both fp64 kernels.  The same 64 sequences, with edge uniforms that
    send many of them to the fp64 draw, drawn both ways (alone, and among
    320) give the same tokens, counts and flags bit for bit, and the
    oracle's.  Nearly all of the 320 are queued, more than the fp64 grids
    cover in one pass (80), so the kernels also walk the queue in passes."""
    b = workloads.make_batch(cfg, seqs=range(320), workers=workloads.default_workers(), V=V)
    ref = oracle.verify_batch(b, workers=workloads.default_workers())
    ur, chosen, _ = edge_uniforms(b, ref)
    b2 = dataclasses.replace(b, u_resample=ur)
    print(f"cfg {cfg} V={b.V}: 320 sequences, {len(chosen)} edge uniforms", flush=True)
    big = run_gpu(gpu_lib, b2)
    small = _head(b2, 64)
    g = run_gpu(gpu_lib, small)
    c64 = chosen[chosen < 64]
    assert len(c64) >= 16
    assert np.all(g.flags[c64] & sv.FLAG_FP64), "an edge draw was certified by the fp32 path"
    np.testing.assert_array_equal(g.tokens, big.tokens[:64])
    np.testing.assert_array_equal(g.n, big.n[:64])
    np.testing.assert_array_equal(g.flags, big.flags[:64])
    compare(small, g, oracle.verify_batch(small)).check()


def _cus():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("cfg,V", [(1, 1000), (0, 2000), (1, 999)], ids=["V1000-bf16", "V2000-fp32", "V999-bf16-scalar"])
def test_short_rows_both_paths(gpu_lib, cfg, V):
    """Short rows (at most two fp64 chunks) are drawn by the one-launch kernel
    at any batch size, and, with spec_short_max_seqs(0), by the sweep,
    k_verify and the one-workgroup fp64 kernel.  The same batch of 2 CUs + 64
    sequences with edge uniforms through both: both meet the oracle's parity
    rule, every edge draw is an fp64 draw on both paths, and the two agree
    wherever their counts do."""
    B = 2 * _cus() + 64
    b = workloads.make_batch(cfg, seqs=range(B), workers=workloads.default_workers(), V=V)
    ref = oracle.verify_batch(b, workers=workloads.default_workers())
    ur, chosen, _ = edge_uniforms(b, ref)
    b2 = dataclasses.replace(b, u_resample=ur)
    ref2 = oracle.verify_batch(b2, workers=workloads.default_workers())
    print(f"cfg {cfg} V={b.V}: {B} sequences, {len(chosen)} edge uniforms", flush=True)
    g = run_gpu(gpu_lib, b2)
    old = gpu_lib.short_max_seqs(0)
    try:
        big = run_gpu(gpu_lib, b2)
    finally:
        gpu_lib.short_max_seqs(old)
    compare(b2, g, ref2).check()
    compare(b2, big, ref2).check()
    assert len(chosen) >= 16
    assert np.all(g.flags & sv.FLAG_FP64), "the one-launch path draws every token in fp64"
    assert np.all(big.flags[chosen] & sv.FLAG_FP64), "an edge draw was certified by the fp32 path"
    same = g.n == big.n
    assert same.sum() >= B - B // 16
    np.testing.assert_array_equal(g.tokens[same], big.tokens[same])
    np.testing.assert_array_equal(g.flags & ~sv.FLAG_FP64, big.flags & ~sv.FLAG_FP64)
