"""GPU parity of token-tree verification (greedy) and of the tree attention
mask / depth position ids, against the CPU oracle in oracle.tree."""
import sys

import numpy as np
import pytest

import workloads
from oracle import tree

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _logits_dev(tb):
    import torch
    if tb.dtype == "bf16":
        return _dev(tb.logits.view(np.int16)).view(torch.bfloat16)
    return _dev(tb.logits)


@pytest.mark.parametrize("B,N,V,dt,pb", [(8, 1, 1000, "bf16", 0.5), (16, 5, 777, "fp32", 0.5),
                                         (32, 32, 32000, "bf16", 0.5), (8, 64, 5001, "fp32", 0.3),
                                         (12, 64, 128256, "bf16", 0.7), (6, 17, 999, "bf16", 1.0)],
                         ids=lambda x: str(x))
def test_tree_verification_matches_oracle(gpu_lib, B, N, V, dt, pb):
    import torch
    tb = workloads.make_tree_batch(B, N, V, dt, seed=N + V, p_branch=pb, workers=workloads.default_workers())
    say(f"[tree] B={B} N={N} V={V} {dt} p_branch={pb}")
    tok, path, n = gpu_lib.verify_tree_greedy(_logits_dev(tb), _dev(tb.tokens), _dev(tb.parents))
    torch.cuda.synchronize()
    rt, rp, rn = tree.verify_tree_greedy(tb.logits, tb.tokens, tb.parents, tb.dtype)
    np.testing.assert_array_equal(n.cpu().numpy(), rn)
    np.testing.assert_array_equal(tok.cpu().numpy(), rt)
    np.testing.assert_array_equal(path.cpu().numpy(), rp)


def _run_tree(sv, tb):
    import torch
    tok, path, n = sv.verify_tree_greedy(_logits_dev(tb), _dev(tb.tokens), _dev(tb.parents))
    torch.cuda.synchronize()
    return tok.cpu().numpy(), path.cpu().numpy(), n.cpu().numpy()


@pytest.mark.parametrize("B,N,V,dt,pb,all_match", [(8, 2, 3000, "bf16", 0.5, False), (8, 3, 3000, "fp32", 0.0, False),
                                                   (8, 4, 3000, "bf16", 0.0, True), (16, 64, 4096, "bf16", 0.0, False),
                                                   (16, 64, 4096, "fp32", 0.0, True), (32, 48, 2048, "bf16", 1.0, True),
                                                   (24, 32, 5001, "fp32", 0.5, False)],
                         ids=lambda x: str(x))
def test_tree_rounds_and_full_sweep_agree(gpu_lib, B, N, V, dt, pb, all_match):
    """Token trees read in rounds by depth (the roots, depths 1-2, the rest,
    with k_tree_round marking the rows each round needs) and with every row
    swept at once give the oracle's outputs.  Chains (p_branch 0), bushy
    trees (p_branch 1), the round boundaries (N = 2, 3, 4) and trees whose
    every token is its parent's arg-max (every row needed)."""
    tb = workloads.make_tree_batch(B, N, V, dt, seed=3 * N + V, p_branch=pb, workers=workloads.default_workers())
    if all_match:  # every node's token is its parent's first arg-max: every node is accepted
        amax = np.argmax(workloads.storage_to_f64(tb.logits, dt), axis=2)
        for b in range(B):
            for v in range(1, N):
                tb.tokens[b, v] = amax[b, tb.parents[b, v]]
    say(f"[tree] rounds vs full: B={B} N={N} V={V} {dt} p_branch={pb} all_match={all_match}")
    rt, rp, rn = tree.verify_tree_greedy(tb.logits, tb.tokens, tb.parents, tb.dtype)
    old = gpu_lib.rounds_min_bytes(0.0)
    try:
        got_rounds = _run_tree(gpu_lib, tb)
        gpu_lib.rounds_min_bytes(1e18)
        got_full = _run_tree(gpu_lib, tb)
    finally:
        gpu_lib.rounds_min_bytes(old)
    for got, name in ((got_rounds, "rounds"), (got_full, "full")):
        np.testing.assert_array_equal(got[2], rn, err_msg=name)
        np.testing.assert_array_equal(got[0], rt, err_msg=name)
        np.testing.assert_array_equal(got[1], rp, err_msg=name)
    if all_match:
        assert np.all(rn == np.array([max(tree.tree_mask(tb.parents[b])[1]) for b in range(B)]))


@pytest.mark.parametrize("N", [1, 2, 5, 33, 64])
def test_tree_mask_matches_oracle(gpu_lib, N):
    import torch
    rng = np.random.default_rng(N)
    B = 20
    parents = np.stack([np.concatenate([[-1], [rng.integers(0, v) if rng.random() < 0.5 else v - 1
                                               for v in range(1, N)]]) for _ in range(B)]).astype(np.int32)
    parents[3, N // 2] = N + 7 if N > 2 else parents[3, N // 2]      # invalid parents: see only themselves
    parents[4, N - 1] = -5 if N > 1 else parents[4, N - 1]
    mask, depth = gpu_lib.tree_mask(_dev(parents))
    torch.cuda.synchronize()
    mask, depth = mask.cpu().numpy(), depth.cpu().numpy()
    for b in range(B):
        m, d = tree.tree_mask(parents[b])
        np.testing.assert_array_equal(mask[b], m)
        np.testing.assert_array_equal(depth[b], d)


def test_tree_with_invalid_parents_matches_oracle(gpu_lib):
    import torch
    tb = workloads.make_tree_batch(16, 24, 3000, "fp32", seed=5, workers=workloads.default_workers())
    parents = tb.parents.copy()
    parents[::3, 7] = 30
    parents[1::3, 11] = -2
    tok, path, n = gpu_lib.verify_tree_greedy(_logits_dev(tb), _dev(tb.tokens), _dev(parents))
    torch.cuda.synchronize()
    rt, rp, rn = tree.verify_tree_greedy(tb.logits, tb.tokens, parents, tb.dtype)
    np.testing.assert_array_equal(n.cpu().numpy(), rn)
    np.testing.assert_array_equal(tok.cpu().numpy(), rt)
    np.testing.assert_array_equal(path.cpu().numpy(), rp)


def test_chain_tree_equals_the_linear_greedy_entry_point(gpu_lib):
    """A chain tree of K+1 nodes is linear greedy verification: the same
    accepted counts and tokens as spec_verify at T = 0."""
    import torch
    b = workloads.make_batch(4, seqs=range(48), workers=workloads.default_workers())
    lp, _, x, _, _ = workloads.to_device(b)
    tok_lin, n_lin = gpu_lib.verify(lp, None, x, None, None, 0.0)
    K = b.K
    tokens = torch.cat([torch.zeros((b.B, 1), dtype=torch.int32, device="cuda"), x], dim=1).contiguous()
    parents = torch.arange(-1, K, dtype=torch.int32, device="cuda").expand(b.B, K + 1).contiguous()
    tok_t, path, n_t = gpu_lib.verify_tree_greedy(lp, tokens, parents)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(n_t.cpu().numpy(), n_lin.cpu().numpy())
    np.testing.assert_array_equal(tok_t.cpu().numpy(), tok_lin.cpu().numpy())


N_RANDOM_TREES = int(__import__("os").environ.get("SPECV_RANDOM_TREE_CASES", "16"))


@pytest.mark.parametrize("case", range(N_RANDOM_TREES))
def test_random_trees_match_oracle(gpu_lib, case):
    """Random tree batches (size, depth structure, vocabulary, dtype, share of
    tokens that match their parent's arg-max) in rounds by depth (the tests'
    threshold) against the oracle."""
    rng = np.random.default_rng(8000 + case)
    B = int(rng.integers(1, 40))
    N = int(rng.integers(1, 65))
    V = int(rng.choice([1, 2, 7, 64, 1000, 4097, 32000]))
    dt = str(rng.choice(["fp32", "bf16"]))
    pb = float(rng.choice([0.0, 0.3, 0.7, 1.0]))
    tb = workloads.make_tree_batch(B, N, V, dt, seed=case, p_branch=pb)
    match = float(rng.choice([0.0, 0.5, 0.9, 1.0]))
    amax = np.argmax(workloads.storage_to_f64(tb.logits, dt), axis=2)
    for b in range(B):
        for v in range(1, N):
            if rng.random() < match:
                tb.tokens[b, v] = amax[b, tb.parents[b, v]]
    say(f"[tree] random case {case}: B={B} N={N} V={V} {dt} p_branch={pb} match={match}")
    rt, rp, rn = tree.verify_tree_greedy(tb.logits, tb.tokens, tb.parents, tb.dtype)
    tok, path, n = _run_tree(gpu_lib, tb)
    np.testing.assert_array_equal(n, rn)
    np.testing.assert_array_equal(tok, rt)
    np.testing.assert_array_equal(path, rp)
