"""Plain CPU oracle for token-tree verification in greedy mode and for the
tree attention mask with depth position ids.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

Sources (cited by title and section):
  [A] "Speculative Decoding: Cách LLM Sinh Văn Bản Nhanh Gấp 2–3 Lần"
      (anhtu.dev), "Token tree: kiểm nhiều nhánh đoán cùng lúc".
  [C] "5.3 Medusa, EAGLE và MTP" (infra-guide-du8.pages.dev), sections 3.1,
      3.2, 8 and 9.1.

A draft tree of N nodes is given by ``parents`` (node 0 is the root, whose
parent is -1; every other node's parent comes before it) and a token per
node.  The root holds the last committed token; node v != 0 proposes its
token as the continuation of its parent.  The target model has produced
logits at every node: row v is the distribution of the token after node v.

* Mask and positions ([C] 3.1, 3.2, 8): node v sees itself and its
  ancestors, nothing else; its position id is its depth (root 0).
* Greedy verification ([C] 9.1, greedy matching; [A]: the deepest accepted
  branch is the round's output): the root is accepted; node v is accepted
  when its parent is accepted and its token is the first arg-max of its
  parent's row.  The output is the path from the root to the deepest
  accepted node d (its tokens, root excluded) followed by the first arg-max
  of row d, the bonus token.

Readings where the pages say nothing: among accepted nodes of equal depth
the lowest index wins (possible only when siblings repeat a token); a node
whose parent index is not in [0, v) is never accepted, sees only itself in
the mask and has depth 0; outputs are padded with -1 to N entries.
"""
from __future__ import annotations

import numpy as np

from .verify import first_argmax, widen


def tree_mask(parents) -> tuple[np.ndarray, np.ndarray]:
    """Visibility mask [N, N] (uint8, 1 = node i may attend to node j) and
    depth position ids [N] for one tree."""
    parents = [int(p) for p in parents]
    n = len(parents)
    mask = np.zeros((n, n), np.uint8)
    depth = np.zeros(n, np.int32)
    for v in range(n):
        p = parents[v]
        ok = v > 0 and 0 <= p < v
        depth[v] = depth[p] + 1 if ok else 0
        mask[v, v] = 1
        u = p if ok else -1
        while u != -1:  # climb the ancestor chain (parents come first, so it ends)
            mask[v, u] = 1
            pu = parents[u]
            u = pu if (u > 0 and 0 <= pu < u) else -1
    return mask, depth


def verify_tree_greedy_sequence(logits, tokens, parents, dtype: str = "fp32"):
    """One tree.  logits [N, V] (fp32 or bf16 bits), tokens [N], parents [N].
    Returns dict(tokens [N], path [N], n) with n the number of accepted drafts."""
    lg = widen(np.asarray(logits), dtype)
    n_nodes = lg.shape[0]
    amax = [first_argmax(lg[v]) for v in range(n_nodes)]
    parents = [int(p) for p in parents]
    accepted = [False] * n_nodes
    depth = [0] * n_nodes
    accepted[0] = True
    for v in range(1, n_nodes):
        p = parents[v]
        if 0 <= p < v:
            depth[v] = depth[p] + 1
            accepted[v] = accepted[p] and int(tokens[v]) == amax[p]
    best = 0
    for v in range(n_nodes):
        if accepted[v] and depth[v] > depth[best]:
            best = v
    path = []
    u = best
    while True:
        path.append(u)
        if u == 0:
            break
        u = parents[u]
    path.reverse()
    out_tokens = np.full(n_nodes, -1, np.int32)
    out_path = np.full(n_nodes, -1, np.int32)
    d = len(path) - 1
    for i, v in enumerate(path[1:]):
        out_tokens[i] = int(tokens[v])
    out_tokens[d] = amax[best]
    out_path[: d + 1] = path
    return dict(tokens=out_tokens, path=out_path, n=d)


def verify_tree_greedy(logits, tokens, parents, dtype: str = "fp32"):
    """Every tree of a batch: logits [B, N, V], tokens [B, N], parents [B, N].
    Returns (tokens [B, N], path [B, N], n [B])."""
    B, N = np.shape(tokens)
    out_t = np.full((B, N), -1, np.int32)
    out_p = np.full((B, N), -1, np.int32)
    out_n = np.zeros(B, np.int32)
    for b in range(B):
        r = verify_tree_greedy_sequence(logits[b], tokens[b], parents[b], dtype)
        out_t[b], out_p[b], out_n[b] = r["tokens"], r["path"], r["n"]
    return out_t, out_p, out_n
