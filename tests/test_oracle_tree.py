"""Pins of the token-tree oracle (greedy verification, attention mask and
depth position ids) against the pages' worked examples and independent
formulations."""
import json
import os

import numpy as np

import oracle
from oracle import tree

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tree_examples.json")


def random_tree(rng, n, p_branch=0.5):
    """parents with parents[v] < v: a chain that branches with probability p_branch."""
    parents = [-1]
    for v in range(1, n):
        parents.append(int(rng.integers(0, v)) if rng.random() < p_branch else v - 1)
    return np.array(parents, np.int32)


def test_mask_and_depth_match_the_pages_example():
    g = json.load(open(GOLDEN))["mask_example"]
    mask, depth = tree.tree_mask(g["parents"])
    assert mask[4].tolist() == g["mask_row_4"]
    a, b = g["equal_depth"]
    assert depth[a] == depth[b] == 1


def test_mask_is_the_transitive_closure_of_the_parent_relation():
    """Visibility = reflexive-transitive closure of child -> parent, computed
    here by boolean matrix powers; depth = visible nodes - 1; never more than
    the causal (lower-triangular) mask."""
    rng = np.random.default_rng(1)
    for _ in range(50):
        n = int(rng.integers(1, 40))
        parents = random_tree(rng, n)
        A = np.zeros((n, n), np.int64)
        for v in range(1, n):
            A[v, parents[v]] = 1
        closure = np.eye(n, dtype=np.int64)
        step = np.eye(n, dtype=np.int64)
        for _ in range(n):
            step = np.minimum(step @ A, 1)
            closure = np.minimum(closure + step, 1)
        mask, depth = tree.tree_mask(parents)
        np.testing.assert_array_equal(mask, closure)
        np.testing.assert_array_equal(depth, mask.sum(axis=1) - 1)
        assert np.all(np.triu(mask, 1) == 0)


def test_chain_tree_reduces_to_linear_greedy_matching():
    """A chain (every node's parent is the previous node) is the pages' linear
    greedy verification ([C] 9.1): same accepted count and emitted tokens."""
    rng = np.random.default_rng(2)
    for _ in range(40):
        K, V = int(rng.integers(1, 9)), int(rng.integers(2, 30))
        lp = np.round(rng.normal(0, 1, (K + 1, V)), 1).astype(np.float32)
        a = np.argmax(lp, axis=1)
        x = np.where(rng.random(K) < 0.7, a[:K], rng.integers(0, V, K)).astype(np.int32)
        lin = oracle.verify_greedy_sequence(lp.astype(np.float64), x)
        tokens = np.concatenate([[0], x]).astype(np.int32)      # node v >= 1 carries x_{v-1}
        r = tree.verify_tree_greedy_sequence(lp, tokens, np.arange(-1, K, dtype=np.int32))
        assert r["n"] == lin["n"]
        np.testing.assert_array_equal(r["tokens"][: K + 1], lin["tokens"])
        np.testing.assert_array_equal(r["path"][: r["n"] + 1], np.arange(r["n"] + 1))


def test_deepest_accepted_node_by_path_enumeration():
    """Brute force: a node is reachable when every node on its root path
    carries its parent's first arg-max; the answer is the deepest reachable
    node (lowest index among equals), its path and the arg-max after it."""
    rng = np.random.default_rng(3)
    for _ in range(200):
        n, V = int(rng.integers(1, 20)), int(rng.integers(2, 6))
        parents = random_tree(rng, n, 0.6)
        lg = rng.integers(-3, 3, (n, V)).astype(np.float32)    # small integers: many ties
        amax = np.argmax(lg, axis=1)
        tok = np.where(rng.random(n) < 0.6, amax[np.maximum(parents, 0)], rng.integers(0, V, n)).astype(np.int32)
        paths = []
        for v in range(n):
            p, u = [v], v
            while u != 0:
                u = int(parents[u])
                p.append(u)
            paths.append(p[::-1])
        ok = [all(tok[c] == amax[pp] for pp, c in zip(p[:-1], p[1:])) for p in paths]
        best = max((len(paths[v]), -v) for v in range(n) if ok[v])
        d = -best[1]
        r = tree.verify_tree_greedy_sequence(lg, tok, parents)
        assert r["n"] == len(paths[d]) - 1
        np.testing.assert_array_equal(r["path"][: r["n"] + 1], paths[d])
        np.testing.assert_array_equal(r["tokens"][: r["n"]], tok[paths[d][1:]])
        assert r["tokens"][r["n"]] == amax[d]
        assert np.all(r["tokens"][r["n"] + 1:] == -1)


def test_the_pages_flowchart_tree():
    """[A]'s tree: the target prefers the, then cat, then sat; the accepted
    branch is the -> cat -> sat (three drafts) and the bonus is what follows sat."""
    g = json.load(open(GOLDEN))["flowchart_example"]
    words, parents = g["words"], np.array(g["parents"], np.int32)
    V = len(words)
    idx = {w: i for i, w in enumerate(words)}
    rng = np.random.default_rng(4)
    lg = rng.normal(0, 0.1, (V, V)).astype(np.float32)        # node v's row: next-word scores
    prefer = {"<root>": "the", "the": "cat", "cat": "sat", "sat": "<root>", "a": "big", "dog": "ran"}
    for v, w in enumerate(words):
        if w in prefer:
            lg[v, idx[prefer[w]]] = 5.0
    tokens = np.array([idx[w] for w in words], np.int32)
    r = tree.verify_tree_greedy_sequence(lg, tokens, parents)
    assert [words[t] for t in r["tokens"][: r["n"]]] == g["accepted_branch"]
    assert r["n"] == 3 and words[r["tokens"][3]] == "<root>"


def test_invalid_parent_is_never_accepted():
    lg = np.zeros((4, 3), np.float32)
    lg[:, 1] = 1.0                                             # every arg-max is token 1
    r = tree.verify_tree_greedy_sequence(lg, np.array([0, 1, 1, 1], np.int32), np.array([-1, 0, 5, 2], np.int32))
    assert r["n"] == 1 and r["path"][:2].tolist() == [0, 1]
    mask, depth = tree.tree_mask([-1, 0, 5, 2])
    assert mask[2].tolist() == [0, 0, 1, 0] and depth[2] == 0 and depth[3] == 1
