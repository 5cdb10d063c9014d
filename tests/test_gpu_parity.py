"""GPU parity: the HIP path against the fp64 oracle, through the C ABI.

Sizes: the five workloads at full size (every sequence of each, the large
sharp fp32 one generated in blocks), small odd shapes that
exercise ragged tails and the scalar path, and special cases.
"""
import dataclasses
import sys
import types

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import run_gpu
from oracle.parity import compare
from workloads import to_device

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


_BATCHES = {}


def full_batch(cfg):
    if cfg not in _BATCHES:
        _BATCHES[cfg] = workloads.make_batch(cfg, workers=workloads.default_workers())
    return _BATCHES[cfg]


@pytest.mark.parametrize("cfg", [0, 1, 2, 4])
def test_workload_full_size(gpu_lib, cfg):
    b = full_batch(cfg)
    say(f"[parity] workload {cfg} {b.wl.describe()}")
    g = run_gpu(gpu_lib, b)
    ref = oracle.verify_batch(b)
    rep = compare(b, g, ref)
    say(f"[parity] workload {cfg}: decisions={rep.decisions} excused={rep.excused} "
        f"max_logz_err={rep.max_logz_err:.2e}")
    rep.check()


_SHARP = {}


def sharp_blocks(step=64):
    """The sharp workload (B=1024, K=4, V=256000, fp32: 9.4 GB of logits) as
    host blocks of `step` sequences, generated once per session."""
    if "blocks" not in _SHARP:
        wl = workloads.WORKLOADS[3]
        blocks = []
        for s0 in range(0, wl.B, step):
            blocks.append(workloads.make_batch(3, seqs=range(s0, s0 + step), workers=workloads.default_workers()))
            say(f"[parity] workload 3: generated {s0 + step}/{wl.B}")
        _SHARP["blocks"] = blocks
    return _SHARP["blocks"]


def sharp_on_device(blocks):
    """Copy the blocks into one set of device tensors [B, ...]."""
    import torch
    wl = workloads.WORKLOADS[3]
    B, K, V = wl.B, wl.K, wl.V
    lp = torch.empty((B, K + 1, V), dtype=torch.float32, device="cuda")
    lq = torch.empty((B, K, V), dtype=torch.float32, device="cuda")
    x = torch.empty((B, K), dtype=torch.int32, device="cuda")
    ua = torch.empty((B, K), dtype=torch.float32, device="cuda")
    ur = torch.empty((B,), dtype=torch.float32, device="cuda")
    s0 = 0
    for blk in blocks:
        s1 = s0 + blk.B
        lp[s0:s1], lq[s0:s1], x[s0:s1], ua[s0:s1], ur[s0:s1] = to_device(blk)
        s0 = s1
    return lp, lq, x, ua, ur


def compare_blocks(blocks, g, num_drafts=None):
    """Every sequence of every block against the oracle (threads per block)."""
    fails, exc, dec, lz, s0 = [], 0, 0, 0.0, 0
    for blk in blocks:
        s1 = s0 + blk.B
        if num_drafts is not None:
            blk = dataclasses.replace(blk, num_drafts=num_drafts[s0:s1])
        gs = dataclasses.replace(g, tokens=g.tokens[s0:s1], n=g.n[s0:s1], logz=g.logz[s0:s1], flags=g.flags[s0:s1])
        rep = compare(blk, gs, oracle.verify_batch(blk, workers=workloads.default_workers()))
        fails += [(f[0] + s0,) + tuple(f[1:]) for f in rep.failures]
        exc += rep.excused
        dec += rep.decisions
        lz = max(lz, rep.max_logz_err)
        s0 = s1
    return fails, exc, dec, lz


def test_sharp_fp32_workload_full_size(gpu_lib):
    """B=1024, K=4, V=256000 fp32: every one of the 1024 sequences against the
    oracle (tokens, counts, log Z of all 9 rows)."""
    blocks = sharp_blocks()
    say("[parity] workload 3: copying to the device")
    dev = sharp_on_device(blocks)
    g = run_gpu(gpu_lib, workloads.WORKLOADS[3], dev_inputs=dev)
    del dev
    fails, exc, dec, lz = compare_blocks(blocks, g)
    say(f"[parity] workload 3, all {len(g.n)} sequences: decisions={dec} excused={exc} max_logz_err={lz:.2e}")
    assert not fails, fails[:3]
    assert exc <= 1e-4 * dec
    assert lz <= 1e-5


def test_sharp_fp32_workload_full_size_ragged(gpu_lib):
    """The same 1024 sequences with per-sequence draft counts K_b uniform on
    [0, 4] through spec_verify_ragged_ex (its large sweep shape, the unsplit
    fast draw), log Z of the rows each sequence uses included."""
    import torch
    blocks = sharp_blocks()
    wl = workloads.WORKLOADS[3]
    kb = workloads.ragged_draft_counts(wl.B, wl.K, seed=31, low=0)
    say(f"[parity] workload 3 ragged: K_b from {kb.min()} to {kb.max()}")
    dev = sharp_on_device(blocks)
    st = torch.zeros(2 * wl.K, dtype=torch.int64, device="cuda")
    g = run_gpu(gpu_lib, types.SimpleNamespace(T=wl.T, num_drafts=kb), dev_inputs=dev, position_stats=st)
    del dev
    fails, exc, dec, lz = compare_blocks(blocks, g, num_drafts=kb)
    say(f"[parity] workload 3 ragged: decisions={dec} excused={exc} max_logz_err={lz:.2e}")
    assert not fails, fails[:3]
    assert exc <= 1e-4 * dec
    assert lz <= 1e-5
    np.testing.assert_array_equal(st.cpu().numpy(), oracle.position_stats(g.n, kb, wl.K))


@pytest.mark.parametrize("cfg", [1, 2])
def test_draw_matches_oracle_exactly(gpu_lib, cfg):
    """The draw is computed in fp64: every drawn token must equal the oracle's
    whenever the acceptance decisions agree, with no excuse needed (the oracle
    margin of every draw on these batches is far above the fp64 error)."""
    b = full_batch(cfg)
    g = run_gpu(gpu_lib, b)
    ref = oracle.verify_batch(b)
    same_n = g.n == ref.n_accepted
    rows = np.flatnonzero(same_n)
    assert len(rows) >= b.B - 1
    np.testing.assert_array_equal(g.tokens[rows], ref.tokens[rows])


SMALL = [
    # (B, K, V, dtype, T)
    (1, 1, 1, "fp32", 1.0), (3, 2, 1, "bf16", 0.5), (2, 1, 7, "fp32", 0.9), (3, 4, 7, "bf16", 1.3),
    (3, 2, 1001, "bf16", 0.7), (3, 2, 1001, "fp32", 1.0), (2, 5, 4096, "bf16", 1.0), (2, 3, 8192, "fp32", 0.6),
    (1, 32, 999, "bf16", 1.0), (2, 32, 2048, "fp32", 2.0), (5, 3, 70001, "bf16", 0.8), (3, 7, 262400, "bf16", 1.0),
    (2, 2, 300000, "fp32", 1.0),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}K{}V{}{}T{}".format(*s))
def test_small_and_ragged_shapes(gpu_lib, shape):
    B, K, V, dt, T = shape
    wl = workloads.Workload("small", B, K, V, dt, float(np.float32(T)), 2.0, 1.1, "noise", 0.8)
    b = workloads.make_batch(1, wl=wl, seed=100 + V + K)
    say(f"[parity] small {wl.describe()}")
    rep = compare(b, run_gpu(gpu_lib, b), oracle.verify_batch(b))
    rep.check()


@pytest.mark.parametrize("shape", [(3, 2, 1001), (4, 8, 4096), (2, 32, 777), (6, 4, 50000)])
def test_greedy_small_shapes_with_ties(gpu_lib, shape):
    B, K, V = shape
    rng = np.random.default_rng(V)
    lp32 = np.round(rng.normal(0, 2, (B, K + 1, V)), 1).astype(np.float32)
    for s in range(B):
        for k in range(K + 1):
            i, j = sorted(rng.choice(V, 2, replace=False)) if V > 1 else (0, 0)
            lp32[s, k, i] = lp32[s, k, j] = lp32[s, k].max() + 0.5
    a = np.argmax(lp32, axis=2)
    later = np.array([[np.flatnonzero(lp32[s, k] == lp32[s, k].max())[-1] for k in range(K)] for s in range(B)])
    x = np.where(rng.random((B, K)) < 0.75, a[:, :K], later).astype(np.int32)
    for dt in ("fp32", "bf16"):
        lp = lp32 if dt == "fp32" else workloads.f32_to_bf16_bits(lp32)
        b = workloads.custom_batch(lp, None, x, None, None, 0.0, dt)
        rep = compare(b, run_gpu(gpu_lib, b), oracle.verify_batch(b))
        rep.check()


@pytest.mark.parametrize("B,K,V,T", [(192, 8, 65536, 0.0), (192, 4, 65536, 0.9)], ids=["greedy", "sampling"])
def test_fp32_launches_large_enough_for_the_large_sweep_shape(gpu_lib, B, K, V, T):
    """fp32 rows in launches of at least 6144 sweep workgroups (the large
    shape: 16-byte units, 4096 of them per chunk), compared in full."""
    rows = B * (K + 1 if T == 0.0 else 2 * K + 1)
    assert rows * -(-(V // 4) // 4096) >= 6144
    draft = "greedy-mask" if T == 0.0 else "noise"
    wl = workloads.Workload("fp32-large", B, K, V, "fp32", float(np.float32(T)), 2.0, 1.1, draft, 0.8)
    b = workloads.make_batch(1, wl=wl, seed=7, workers=workloads.default_workers())
    say(f"[parity] {wl.describe()}")
    compare(b, run_gpu(gpu_lib, b), oracle.verify_batch(b)).check()


def test_identical_rows_accept_everything(gpu_lib):
    rng = np.random.default_rng(3)
    B, K, V = 16, 6, 3000
    lp = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
    lq = lp[:, :K].copy()
    x = rng.integers(0, V, (B, K)).astype(np.int32)
    ua = rng.random((B, K)).astype(np.float32)
    ur = rng.random(B).astype(np.float32)
    b = workloads.custom_batch(lp, lq, x, ua, ur, 0.8, "fp32")
    g = run_gpu(gpu_lib, b)
    assert np.all(g.n == K)
    compare(b, g, oracle.verify_batch(b)).check()


def test_bad_draft_ids_reject_and_flag(gpu_lib):
    rng = np.random.default_rng(4)
    B, K, V = 6, 4, 500
    lp = rng.normal(0, 1, (B, K + 1, V)).astype(np.float32)
    lq = rng.normal(0, 1, (B, K, V)).astype(np.float32)
    x = rng.integers(0, V, (B, K)).astype(np.int32)
    x[:, 1] = [-1, V, V + 5, -(1 << 30), 1 << 30, -7]
    ua = np.full((B, K), 1e-7, np.float32)
    b = workloads.custom_batch(lp, lq, x, ua, rng.random(B).astype(np.float32), 1.0, "fp32")
    g = run_gpu(gpu_lib, b)
    ref = oracle.verify_batch(b)
    assert np.all(g.flags & 4)
    compare(b, g, ref).check()
    bg = workloads.custom_batch(lp, None, x, None, None, 0.0, "fp32")
    compare(bg, run_gpu(gpu_lib, bg), oracle.verify_batch(bg)).check()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_zero_residual_draws_from_the_target_row(gpu_lib, dtype):
    """A rejection where the draft row equals the target row leaves max(0, p - q) = 0
    everywhere; the draw then follows p_n (flag 2).  Reached here by an invalid draft id
    (flag 4) at a position whose rows are identical."""
    rng = np.random.default_rng(5)
    B, K, V = 8, 5, 2048
    lp = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
    if dtype == "bf16":
        lp = workloads.f32_to_bf16_bits(lp)
    lq = lp[:, :K].copy()
    x = rng.integers(0, V, (B, K)).astype(np.int32)
    x[:, 2] = -1
    ua = rng.random((B, K)).astype(np.float32)
    ur = rng.random(B).astype(np.float32)
    b = workloads.custom_batch(lp, lq, x, ua, ur, 0.8, dtype)
    g = run_gpu(gpu_lib, b)
    assert np.all(g.n == 2)
    assert np.all(g.flags & 2) and np.all(g.flags & 4)
    compare(b, g, oracle.verify_batch(b)).check()


def masked_batch(B, K, V, dtype, seed):
    """Rows as after vocabulary masking, the rest -inf: every target row keeps 64 random
    tokens; the draft row at the same position keeps 40 of them (its logits the target's
    plus noise) and 8 tokens outside them, so the supports overlap in part.  Draft tokens
    come from the draft row's support, except at position 1 of every other sequence, where
    they are drawn from the whole vocabulary."""
    rng = np.random.default_rng(seed)
    lp = np.full((B, K + 1, V), -np.inf, np.float32)
    lq = np.full((B, K, V), -np.inf, np.float32)
    x = np.empty((B, K), np.int32)
    for b in range(B):
        for k in range(K + 1):
            keep_p = rng.choice(V, 64, replace=False)
            lp[b, k, keep_p] = rng.normal(0, 2, 64)
            if k == K:
                break
            shared = rng.choice(keep_p, 40, replace=False)
            lq[b, k, shared] = lp[b, k, shared] + rng.normal(0, 0.5, 40)
            others = np.setdiff1d(rng.choice(V, 16, replace=False), keep_p)[:8]
            lq[b, k, others] = rng.normal(0, 2, others.size)
            keep_q = np.concatenate([shared, others])
            x[b, k] = rng.choice(keep_q) if (k != 1 or b % 2 == 0) else rng.integers(0, V)
    if dtype == "bf16":
        lp, lq = workloads.f32_to_bf16_bits(lp), workloads.f32_to_bf16_bits(lq)
    ua = rng.random((B, K)).astype(np.float32)
    ur = rng.random(B).astype(np.float32)
    return workloads.custom_batch(lp, lq, x, ua, ur, 0.9, dtype)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("shape", [(16, 6, 4096), (4, 4, 50001)], ids=["vector", "odd-V"])
def test_masked_vocabulary(gpu_lib, dtype, shape):
    """-inf logits weigh exactly 0 in the normalisers, the acceptance test and the draw."""
    B, K, V = shape
    b = masked_batch(B, K, V, dtype, seed=21)
    say(f"[parity] masked {dtype} B={B} K={K} V={V}")
    compare(b, run_gpu(gpu_lib, b), oracle.verify_batch(b)).check()
    # greedy: sequence i copies the target's arg-max for its first i mod (K + 1) positions
    xg = b.draft_tokens.copy()
    for i in range(B):
        for k in range(i % (K + 1)):
            xg[i, k] = int(np.argmax(workloads.bf16_bits_to_f32(b.logits_p[i, k]) if dtype == "bf16"
                                     else b.logits_p[i, k]))
    greedy = workloads.custom_batch(b.logits_p, None, xg, None, None, 0.0, dtype)
    compare(greedy, run_gpu(gpu_lib, greedy), oracle.verify_batch(greedy)).check()


def test_determinism_and_temperature_scaling(gpu_lib):
    b = full_batch(1)
    g1 = run_gpu(gpu_lib, b)
    g2 = run_gpu(gpu_lib, b)
    np.testing.assert_array_equal(g1.tokens, g2.tokens)
    np.testing.assert_array_equal(g1.logz, g2.logz)
    # fp32 copy scaled by 2 at twice the temperature: every fp32 step is scaled by a power of two
    lp = oracle.widen(b.logits_p, "bf16").astype(np.float32)
    lq = oracle.widen(b.logits_q, "bf16").astype(np.float32)
    b1 = workloads.custom_batch(lp, lq, b.draft_tokens, b.u_accept, b.u_resample, b.T, "fp32")
    b2 = workloads.custom_batch(lp * 2, lq * 2, b.draft_tokens, b.u_accept, b.u_resample, b.T * 2, "fp32")
    h1, h2 = run_gpu(gpu_lib, b1), run_gpu(gpu_lib, b2)
    np.testing.assert_array_equal(h1.tokens, h2.tokens)
    np.testing.assert_array_equal(h1.n, h2.n)


def test_first_token_follows_p_on_gpu(gpu_lib):
    """10^6 sequences at V=8, K=2 sharing one (p, q) pair, drafts x ~ q: the
    first emitted token must follow p_0 (chi-square, 7 degrees of freedom)."""
    import torch
    from scipy.special import softmax
    from scipy.stats import chi2
    rng = np.random.default_rng(21)
    B, K, V = 10 ** 6, 2, 8
    yp = rng.normal(0, 1.2, (K + 1, V)).astype(np.float32)
    yq = rng.normal(0, 1.2, (K, V)).astype(np.float32)
    p0, q = softmax(yp[0].astype(np.float64)), softmax(yq.astype(np.float64), axis=1)
    x = np.stack([rng.choice(V, B, p=q[k]) for k in range(K)], axis=1).astype(np.int32)
    lp = torch.from_numpy(yp).cuda().expand(B, K + 1, V).contiguous()
    lq = torch.from_numpy(yq).cuda().expand(B, K, V).contiguous()
    ua = torch.from_numpy(rng.random((B, K), dtype=np.float32)).cuda()
    ur = torch.from_numpy(rng.random(B, dtype=np.float32)).cuda()
    tok, n = gpu_lib.verify(lp, lq, torch.from_numpy(x).cuda(), ua, ur, 1.0)
    first = tok[:, 0].cpu().numpy()
    counts = np.bincount(first, minlength=V)
    stat = np.sum((counts - B * p0) ** 2 / (B * p0))
    say(f"[parity] chi2 first token: stat={stat:.2f} p={chi2.sf(stat, V - 1):.3g}")
    assert chi2.sf(stat, V - 1) > 1e-3
    # acceptance at position 0 happens with probability sum(min(p0, q0))
    beta = np.minimum(p0, q[0]).sum()
    acc = float((n.cpu().numpy() >= 1).mean())
    assert abs(acc - beta) < 5 * np.sqrt(beta * (1 - beta) / B)


def test_excused_budget_over_many_seeds(gpu_lib):
    """The small bf16 workload over 24 seeds (1536 sequences)."""
    dec = exc = 0
    for seed in range(24):
        b = workloads.make_batch(1, seed=1000 + seed, workers=workloads.default_workers())
        rep = compare(b, run_gpu(gpu_lib, b), oracle.verify_batch(b))
        assert not rep.failures, rep.failures[:3]
        dec += rep.decisions
        exc += rep.excused
    say(f"[parity] many seeds: decisions={dec} excused={exc}")
    assert exc <= 1e-4 * dec


def test_fp64_queue_longer_than_one_pass(gpu_lib):
    """512 sequences of the small bf16 recipe: about a fifth of their draws
    are not certified by the fast path (its distributions are flat), far more
    than the 32 sequences the fp64 kernels take per pass, so their grids loop."""
    wl = dataclasses.replace(workloads.WORKLOADS[1], B=512)
    b = workloads.make_batch(1, wl=wl, seed=77, workers=workloads.default_workers())
    say(f"[parity] long fp64 queue {wl.describe()}")
    g = run_gpu(gpu_lib, b)
    ref = oracle.verify_batch(b)
    compare(b, g, ref).check()
    same = np.flatnonzero(g.n == ref.n_accepted)
    np.testing.assert_array_equal(g.tokens[same], ref.tokens[same])


@pytest.mark.parametrize("shape", [(1, 1, 2_200_000, "bf16", 1.0), (2, 1, 600_001, "fp32", 0.9)],
                         ids=lambda s: "B{}K{}V{}{}T{}".format(*s))
def test_rows_longer_than_the_segment_table(gpu_lib, shape):
    """Rows so long that a draw segment spans several wave iterations (the
    segment table holds 1024 entries), on the vector and on the scalar path."""
    B, K, V, dt, T = shape
    wl = workloads.Workload("long", B, K, V, dt, float(np.float32(T)), 2.0, 1.1, "noise", 0.8)
    b = workloads.make_batch(1, wl=wl, seed=9)
    say(f"[parity] long rows {wl.describe()}")
    compare(b, run_gpu(gpu_lib, b), oracle.verify_batch(b)).check()


def test_resample_uniform_at_the_ends_of_its_grid(gpu_lib):
    """The smallest and the largest uniform of the grid: the draw's first
    token with weight, and the end of the row where rounding can leave the
    running sum short of u * Z."""
    b = workloads.make_batch(1, seed=5, workers=workloads.default_workers())
    ur = b.u_resample.copy()
    ur[: b.B // 2] = np.float32(0.5 * 2.0 ** -23)
    ur[b.B // 2:] = np.float32(1.0 - 0.5 * 2.0 ** -23)
    b2 = dataclasses.replace(b, u_resample=ur)
    g = run_gpu(gpu_lib, b2)
    ref = oracle.verify_batch(b2)
    compare(b2, g, ref).check()
    same = np.flatnonzero(g.n == ref.n_accepted)
    np.testing.assert_array_equal(g.tokens[same], ref.tokens[same])


@pytest.mark.parametrize("nseq,V,ragged", [(320, None, False), (300, 31999, False), (288, None, True)],
                         ids=["bf16-vector", "bf16-element-loads", "bf16-vector-ragged"])
def test_more_sequences_than_cus(gpu_lib, nseq, V, ragged):
    """Batches of more sequences than the MI355X's 256 CUs take k_verify's
    512-thread shape (two sequences per CU): the small workload's recipe at
    B = 288-320, with 16-byte vector loads and, at V = 31999, element loads,
    and once with per-sequence draft counts; every sequence against the
    oracle."""
    b = workloads.make_batch(1, seqs=range(nseq), workers=workloads.default_workers(), V=V)
    if ragged:
        b = dataclasses.replace(b, num_drafts=workloads.ragged_draft_counts(b.B, b.K, seed=5, low=0))
    say(f"[parity] {nseq} sequences, V={b.V}, ragged={ragged}")
    g = run_gpu(gpu_lib, b)
    rep = compare(b, g, oracle.verify_batch(b, workers=workloads.default_workers()))
    say(f"[parity] {nseq} sequences: decisions={rep.decisions} excused={rep.excused} "
        f"max_logz_err={rep.max_logz_err:.2e}")
    rep.check()


def test_bound_calls_match(gpu_lib):
    """bind_spec_verify / bind_spec_verify_ragged (arguments marshalled once,
    as bench.py times them) enqueue the same calls: the same outputs as
    spec_verify / spec_verify_ragged, on every repeat."""
    import torch
    sv = gpu_lib
    b = workloads.make_batch(1, seqs=range(48), workers=workloads.default_workers())
    lp, lq, x, ua, ur = to_device(b)
    B, K, V, T = b.B, b.K, b.V, b.T
    ws = torch.empty(sv.workspace_size(B, K, V, sv.SPECV_BF16, T), dtype=torch.uint8, device="cuda")
    kb = torch.from_numpy(workloads.ragged_draft_counts(B, K, seed=9, low=0)).cuda()
    outs = {}
    for name in ("plain", "bound", "ragged", "ragged-bound"):
        tok = torch.full((B, K + 1), -7, dtype=torch.int32, device="cuda")
        n = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        fl = torch.zeros((B,), dtype=torch.int32, device="cuda")
        if name == "plain":
            rcs = [sv.spec_verify(lp, lq, x, ua, ur, T, tok, n, ws, out_flags=fl, extended=True)]
        elif name == "bound":
            call = sv.bind_spec_verify(lp, lq, x, ua, ur, T, tok, n, ws, out_flags=fl, extended=True)
            rcs = [call() for _ in range(3)]
        elif name == "ragged":
            rcs = [sv.spec_verify_ragged(lp, lq, x, kb, ua, ur, T, tok, n, ws, out_flags=fl)]
        else:
            call = sv.bind_spec_verify_ragged(lp, lq, x, kb, ua, ur, T, tok, n, ws, out_flags=fl)
            rcs = [call() for _ in range(3)]
        torch.cuda.synchronize()
        assert rcs == [0] * len(rcs), rcs
        outs[name] = (tok.cpu().numpy(), n.cpu().numpy(), fl.cpu().numpy() & ~sv.FLAG_FP64)
    for a, c in (("plain", "bound"), ("ragged", "ragged-bound")):
        for u, v in zip(outs[a], outs[c]):
            np.testing.assert_array_equal(u, v, err_msg=f"{a} vs {c}")
