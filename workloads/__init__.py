"""Seeded synthetic inputs for the speculative-sampling verify step.

This module only *makes inputs*: target logits, draft logits, draft tokens and
the uniforms the verify step consumes.  It holds none of the verify step's
arithmetic (no normaliser, no acceptance test, no residual, no inverse CDF), so
that the fp64 oracle and the HIP path can both be fed from it without sharing
any of the computation they are compared on.

Workload recipe (one reading of the pages' setting, stated here in full):

* Every target row is Zipf-biased Gaussian noise: a seeded permutation ``perm``
  of the vocabulary gives each token a rank, ``bias[perm[r]] = -a * ln(r + 1)``,
  and ``logit = N(0, sigma^2) + bias``.  ``a`` is 1.1 (3.3 for the sharp
  workload).
* Draft rows are the target row plus Gaussian noise, or, for the sharp
  workload, the target row with the values at its 50 best-ranked tokens
  shuffled by an independent permutation.
* Logits are generated in float64 and rounded to float32 (round to nearest
  even); bf16 workloads round that float32 once more to bf16 (round to nearest
  even).  Consumers see only the rounded values.
* Draft tokens are sampled from the draft distribution at temperature T with
  the Gumbel-max construction ``argmax(y / T + G)``, G standard Gumbel, on the
  *rounded* draft logits.  (This is the draft model's job, which the verify
  step takes as given.)  For the greedy workload, each position holds the
  target row's first arg-max with probability 1/2 and a uniform random token
  otherwise.
* Uniforms are float32 values ``(i + 0.5) * 2**-23`` with ``i`` uniform in
  ``[0, 2**23)``: odd multiples of 2**-24, so exactly representable in float32
  (24 significant bits) and strictly inside (0, 1).
* Seeds: sequence ``b`` of workload ``c`` draws from
  ``SeedSequence(entropy=[seed, c], spawn_key=(b,))`` in a fixed order, so any
  subset of sequences can be regenerated alone, in any order, in parallel
  (threads).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Iterable, Optional, Sequence

import numpy as np

DEFAULT_SEED = 2026
U_BITS = 23


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic verify workload (batch shape, dtype, temperature, recipe)."""

    name: str
    B: int
    K: int
    V: int
    dtype: str          # "fp32" or "bf16"
    T: float            # the float32 value handed to the library; 0.0 = greedy
    sigma: float        # std of the Gaussian part of the target logits
    zipf: float         # a in bias = -a * ln(rank + 1)
    draft: str          # "noise" | "top50-shuffle" | "greedy-mask"
    draft_sigma: float = 0.0

    @property
    def greedy(self) -> bool:
        return self.T == 0.0

    def describe(self) -> str:
        mode = "greedy" if self.greedy else f"T={self.T:.6g}"
        return f"B={self.B} K={self.K} V={self.V} {self.dtype} {mode}"


def _f32(x: float) -> float:
    return float(np.float32(x))


# The five workloads: a tiny fp32 case, a small bf16 case, the headline bf16
# case, a large sharp fp32 case that rejects almost always, and a greedy case.
WORKLOADS: tuple[Workload, ...] = (
    Workload("tiny-fp32", 1, 4, 1000, "fp32", _f32(1.0), 1.0, 1.1, "noise", 0.5),
    Workload("small-bf16", 64, 5, 32000, "bf16", _f32(1.0), 2.0, 1.1, "noise", 1.0),
    Workload("headline-bf16", 256, 8, 128256, "bf16", _f32(0.7), 2.0, 1.1, "noise", 0.7),
    Workload("sharp-fp32", 1024, 4, 256000, "fp32", _f32(1.0), 1.0, 3.3, "top50-shuffle"),
    Workload("greedy-bf16", 512, 8, 152064, "bf16", 0.0, 2.0, 1.1, "greedy-mask"),
)


def workload(i: int) -> Workload:
    return WORKLOADS[i]


# ---------------------------------------------------------------- rounding --
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the bf16 bit patterns as uint16.  Finite inputs only (the
    generator never makes NaN or inf)."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = bits + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_logits(x64: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> storage array: float32 for "fp32", uint16 bf16 bits for "bf16"."""
    x32 = x64.astype(np.float32)
    if dtype == "fp32":
        return x32
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored logits to float64 (used to sample draft tokens)."""
    if dtype == "fp32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    return bf16_bits_to_f32(a).astype(np.float64)


def uniforms(rng: np.random.Generator, n: int) -> np.ndarray:
    i = rng.integers(0, 1 << U_BITS, size=n, dtype=np.int64)
    return ((i.astype(np.float64) + 0.5) * 2.0 ** -U_BITS).astype(np.float32)


# ------------------------------------------------------------- one sequence --
def _rng(seed: int, cfg_id: int, b: int) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=[seed, cfg_id], spawn_key=(b,))
    return np.random.Generator(np.random.PCG64(ss))


def _zipf_row(rng: np.random.Generator, V: int, sigma: float, a: float):
    perm = rng.permutation(V)
    bias = np.empty(V, dtype=np.float64)
    bias[perm] = -a * np.log(np.arange(1, V + 1, dtype=np.float64))
    return rng.normal(0.0, sigma, size=V) + bias, perm


def make_sequence(wl: Workload, cfg_id: int, b: int, seed: int = DEFAULT_SEED,
                  V: Optional[int] = None, K: Optional[int] = None) -> dict:
    """Inputs of sequence ``b``: logits_p [K+1,V], logits_q [K,V] (None if
    greedy), draft_tokens [K] int32, u_accept [K] f32, u_resample [1] f32."""
    V = wl.V if V is None else V
    K = wl.K if K is None else K
    rng = _rng(seed, cfg_id, b)
    p64 = np.empty((K + 1, V))
    perms = []
    for k in range(K + 1):
        p64[k], perm = _zipf_row(rng, V, wl.sigma, wl.zipf)
        perms.append(perm)
    lp = round_logits(p64, wl.dtype)
    lq = None
    if wl.draft == "noise":
        q64 = p64[:K] + rng.normal(0.0, wl.draft_sigma, size=(K, V))
        lq = round_logits(q64, wl.dtype)
    elif wl.draft == "top50-shuffle":
        q64 = p64[:K].copy()
        top = min(50, V)
        for k in range(K):
            idx = perms[k][:top]
            q64[k, idx] = p64[k, idx[rng.permutation(top)]]
        lq = round_logits(q64, wl.dtype)
    if wl.greedy:
        take_argmax = rng.random(K) < 0.5
        rand_tok = rng.integers(0, V, size=K)
        p_rounded = storage_to_f64(lp, wl.dtype)
        x = np.where(take_argmax, np.argmax(p_rounded[:K], axis=1), rand_tok)
    else:
        yq = storage_to_f64(lq, wl.dtype) / wl.T
        x = np.argmax(yq + rng.gumbel(size=(K, V)), axis=1)
    ua = uniforms(rng, K)
    ur = uniforms(rng, 1)
    return dict(logits_p=lp, logits_q=lq, draft_tokens=x.astype(np.int32),
                u_accept=ua, u_resample=ur)


# ------------------------------------------------------------------- batches --
@dataclasses.dataclass
class Batch:
    """A host-side batch in the library's layout (row-major, V innermost)."""

    wl: Workload
    cfg_id: int
    seqs: np.ndarray                 # which sequence ids of the workload these are
    logits_p: np.ndarray             # [B,K+1,V] float32 or uint16 (bf16 bits)
    logits_q: Optional[np.ndarray]   # [B,K,V] or None (greedy)
    draft_tokens: np.ndarray         # [B,K] int32
    u_accept: np.ndarray             # [B,K] float32
    u_resample: np.ndarray           # [B] float32
    num_drafts: Optional[np.ndarray] = None  # [B] int32 per-sequence draft counts K_b, or None (all K)

    @property
    def B(self) -> int:
        return int(self.draft_tokens.shape[0])

    @property
    def K(self) -> int:
        return int(self.draft_tokens.shape[1])

    @property
    def V(self) -> int:
        return int(self.logits_p.shape[2])

    @property
    def T(self) -> float:
        return self.wl.T

    @property
    def dtype(self) -> str:
        return self.wl.dtype


def _gen_block(args):
    wl, cfg_id, seqs, seed, V, K = args
    return [make_sequence(wl, cfg_id, int(b), seed, V, K) for b in seqs]


def make_batch(cfg_id: int, seqs: Optional[Iterable[int]] = None, seed: int = DEFAULT_SEED,
               workers: int = 1, wl: Optional[Workload] = None,
               V: Optional[int] = None, K: Optional[int] = None) -> Batch:
    """Generate sequences ``seqs`` (default: all B) of workload ``cfg_id``.

    ``wl`` overrides the workload (for custom shapes in tests); ``V``/``K``
    override its vocabulary size and draft length."""
    wl = WORKLOADS[cfg_id] if wl is None else wl
    seqs = np.arange(wl.B) if seqs is None else np.asarray(list(seqs), dtype=np.int64)
    Vv = wl.V if V is None else V
    Kk = wl.K if K is None else K
    if workers > 1 and len(seqs) > 1:
        parts = np.array_split(seqs, min(workers * 4, len(seqs)))
        # threads, not processes: numpy's bulk generators release the GIL, and no
        # child process is ever forked from a process that may hold a GPU context
        with ThreadPoolExecutor(workers) as ex:
            out = [s for blk in ex.map(_gen_block, [(wl, cfg_id, p, seed, Vv, Kk) for p in parts]) for s in blk]
    else:
        out = _gen_block((wl, cfg_id, seqs, seed, Vv, Kk))
    lp = np.stack([s["logits_p"] for s in out])
    lq = None if wl.greedy else np.stack([s["logits_q"] for s in out])
    return Batch(wl=dataclasses.replace(wl, B=len(seqs), V=Vv, K=Kk), cfg_id=cfg_id, seqs=seqs,
                 logits_p=lp, logits_q=lq,
                 draft_tokens=np.stack([s["draft_tokens"] for s in out]),
                 u_accept=np.stack([s["u_accept"] for s in out]),
                 u_resample=np.concatenate([s["u_resample"] for s in out]))


def default_workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def custom_batch(logits_p, logits_q, draft_tokens, u_accept, u_resample, T: float, dtype: str) -> Batch:
    """Wrap hand-made arrays (edge-case tests) in a Batch."""
    lp = np.asarray(logits_p)
    B, K1, V = lp.shape
    wl = Workload("custom", B, K1 - 1, V, dtype, _f32(T), 0.0, 0.0, "custom")
    return Batch(wl=wl, cfg_id=-1, seqs=np.arange(B), logits_p=lp,
                 logits_q=None if logits_q is None else np.asarray(logits_q),
                 draft_tokens=np.asarray(draft_tokens, dtype=np.int32).reshape(B, K1 - 1),
                 u_accept=None if u_accept is None else np.asarray(u_accept, dtype=np.float32).reshape(B, K1 - 1),
                 u_resample=None if u_resample is None else np.asarray(u_resample, dtype=np.float32).reshape(B))


# ------------------------------------------------------------------- trees --
TREE_STREAM = 100  # seed stream of the token-tree inputs


@dataclasses.dataclass
class TreeBatch:
    """Token trees in the library's layout: logits [B,N,V] (row v: the
    target's scores after node v), tokens [B,N] (node 0: the committed root
    token), parents [B,N] (parents[:, 0] == -1, parents[v] < v)."""

    logits: np.ndarray
    tokens: np.ndarray
    parents: np.ndarray
    dtype: str

    @property
    def B(self) -> int:
        return int(self.tokens.shape[0])

    @property
    def N(self) -> int:
        return int(self.tokens.shape[1])

    @property
    def V(self) -> int:
        return int(self.logits.shape[2])


def make_tree(b: int, N: int, V: int, dtype: str, seed: int = DEFAULT_SEED, p_branch: float = 0.5,
              sigma: float = 2.0, zipf: float = 1.1) -> dict:
    """Tree ``b``: a chain that branches (node v hangs under a uniformly drawn
    earlier node with probability p_branch, else under v - 1); every node's
    row is a Zipf-biased Gaussian row as in the other workloads; node v's
    token is its parent's first arg-max with probability 1/2, else uniform."""
    rng = _rng(seed, TREE_STREAM, b)
    parents = np.empty(N, np.int32)
    parents[0] = -1
    for v in range(1, N):
        parents[v] = rng.integers(0, v) if rng.random() < p_branch else v - 1
    rows = np.empty((N, V))
    for v in range(N):
        rows[v], _ = _zipf_row(rng, V, sigma, zipf)
    lg = round_logits(rows, dtype)
    amax = np.argmax(storage_to_f64(lg, dtype), axis=1)
    tokens = np.empty(N, np.int32)
    tokens[0] = rng.integers(0, V)
    take = rng.random(N) < 0.5
    rand_tok = rng.integers(0, V, size=N)
    tokens[1:] = np.where(take[1:], amax[parents[1:]], rand_tok[1:])
    return dict(logits=lg, tokens=tokens, parents=parents)


def make_tree_batch(B: int, N: int, V: int, dtype: str, seed: int = DEFAULT_SEED, p_branch: float = 0.5,
                    workers: int = 1) -> TreeBatch:
    """B trees of N nodes (see make_tree), generated in threads."""
    def one(b):
        return make_tree(b, N, V, dtype, seed, p_branch)
    if workers > 1 and B > 1:
        with ThreadPoolExecutor(workers) as ex:
            trees = list(ex.map(one, range(B)))
    else:
        trees = [one(b) for b in range(B)]
    return TreeBatch(logits=np.stack([t["logits"] for t in trees]), tokens=np.stack([t["tokens"] for t in trees]),
                     parents=np.stack([t["parents"] for t in trees]), dtype=dtype)


# --------------------------------------------------------------- histories --
HISTORY_STREAM = 200  # seed stream of the token histories


def make_history(b: int, L: int, vocab: int, seed: int = DEFAULT_SEED, p_copy: float = 0.5) -> np.ndarray:
    """Token history ``b`` of length uniform in [L/2, L]: alternating spans of
    fresh tokens (Zipf-distributed ranks over a seeded vocabulary permutation,
    mean span 8) and, with probability p_copy, copies of an earlier span (mean
    length 16), the self-similarity of edited code and templates that n-gram
    proposers feed on."""
    rng = _rng(seed, HISTORY_STREAM, b)
    n = int(rng.integers(max(1, L // 2), L + 1))
    perm = rng.permutation(vocab)
    out = np.empty(n, np.int64)
    m = 0
    while m < n:
        if m > 16 and rng.random() < p_copy:
            start = int(rng.integers(0, m - 1))
            span = min(int(rng.geometric(1 / 16)), m - start, n - m)
            out[m:m + span] = out[start:start + span]
        else:
            span = min(int(rng.geometric(1 / 8)), n - m)
            ranks = np.minimum(rng.zipf(1.2, size=span) - 1, vocab - 1)
            out[m:m + span] = perm[ranks]
        m += span
    return out.astype(np.int32)


def make_histories(B: int, L: int, vocab: int, seed: int = DEFAULT_SEED, p_copy: float = 0.5,
                   workers: int = 1):
    """B histories padded with -1 to [B, L] int32, and their lengths [B]."""
    def one(b):
        return make_history(b, L, vocab, seed, p_copy)
    if workers > 1 and B > 1:
        with ThreadPoolExecutor(workers) as ex:
            hs = list(ex.map(one, range(B)))
    else:
        hs = [one(b) for b in range(B)]
    out = np.full((B, L), -1, np.int32)
    for b, h in enumerate(hs):
        out[b, : len(h)] = h
    return out, np.array([len(h) for h in hs], np.int32)


def ragged_draft_counts(B: int, K: int, seed: int = DEFAULT_SEED, low: int = 1) -> np.ndarray:
    """Per-sequence draft counts K_b, uniform on [low, K], seeded: the
    stand-in for a proposer that adapts its draft length per sequence."""
    rng = np.random.default_rng(np.random.SeedSequence(entropy=[seed, 9001]))
    return rng.integers(low, K + 1, B).astype(np.int32)


def to_device(batch: Batch, device="cuda"):
    """Copy a batch to torch device tensors (bf16 bit patterns become bfloat16)."""
    import torch

    def t(a, dt=None):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if dt is not None:
            a = a.view(dt)
        return torch.from_numpy(a).to(device)

    if batch.dtype == "bf16":
        lp = t(batch.logits_p, np.int16).view(torch.bfloat16)
        lq = None if batch.logits_q is None else t(batch.logits_q, np.int16).view(torch.bfloat16)
    else:
        lp, lq = t(batch.logits_p), t(batch.logits_q)
    return lp, lq, t(batch.draft_tokens.astype(np.int32)), t(batch.u_accept), t(batch.u_resample)
