"""Plain fp64 CPU oracle for the speculative-sampling verify step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this module: only the tests, the smoke check and the benchmark's CPU
baseline leg do.  It shares no code with the HIP library; the two meet only
through the seeded inputs in ``workloads``.

Sources (the pages, cited by title and section):
  [A] "Speculative Decoding: Cách LLM Sinh Văn Bản Nhanh Gấp 2–3 Lần" (anhtu.dev)
  [B] "投机解码：让大模型「猜」着跑的数学魔术" (blog.oscine.io)
  [C] "5.3 Medusa, EAGLE và MTP" (infra-guide-du8.pages.dev)
  [D] "Спекулятивное декодирование: ускорение инференса LLM на 20–50%" (glukhov.org)

What it computes, per sequence (all arithmetic in float64; inputs are widened
exactly; T is the float32 value the library receives):

1. Distributions at temperature T.  ``y = logits / T``; the target rows give
   p_k = softmax(y_p,k) for k = 0..K, the draft rows give q_k = softmax(y_q,k)
   for k = 0..K-1.  p is the target's and q the draft's probability of a
   token ([A] "Toán học của sự miễn phí"; [B] "拒绝采样"; [D] "Математическая
   гарантия").  The same T is applied to both.
2. Acceptance test, left to right.  Draft token x_k is accepted iff
   ``u_accept[k] < min(1, p_k(x_k) / q_k(x_k))`` (strict).  The ratio is taken
   in the log domain so a vanishing q does not divide by zero.  The scan stops
   at the first rejection; n is its index, or K if every test passes.
   ([B] "验收标准的精确数学", the equation for alpha(x) and its two cases;
   [B] "多 Token 验证：左到右，遇错即停".)
3. The replacement token.  After a rejection at n < K the token is drawn from
   the residual ``max(0, p_n - q_n) / Z``, Z its sum ([B] "拒绝之后怎么办？——
   残差分布", the equations for p_resid and Z; [D] "Математическая гарантия",
   the equation for r(x)).  If all K are accepted, the bonus token is drawn
   from p_K, the target's distribution one position past the last draft ([A]
   "Toán học của sự miễn phí", third rule; [B] "多 Token 验证", fourth step).
4. The draw is an inverse CDF with the supplied uniform: with C the running
   sum of the weights in ascending token order, the token is the smallest v
   with ``C(v) > u_resample * Z``.  (The pages only say "sample"; this is the
   plainest deterministic reading that consumes one supplied uniform.)
5. Output: ``tokens = [x_0, .., x_{n-1}, j, -1, ..]`` (K+1 entries) and n
   ([B] "多 Token 验证": at least one and at most k+1 tokens per round).
6. Greedy mode (T == 0): a_k is the first index of the maximum of target row
   k.  Accept while a_k == x_k; emit a_n (a_K is the bonus).  No draft logits
   and no uniforms are read.  ([C] section 9.1, greedy matching versus exact
   sampling; [D] "Механизм «черновик — проверка»", longest matching prefix.)

Readings where the pages say nothing (kept identical on the HIP side):

* A draft id outside [0, V) fails its test (threshold 0) and sets flag bit 2.
* If rounding makes Z == 0 after a rejection (exactly, Z == 0 means p == q,
  which always accepts), the draw falls back to p_n and sets flag bit 1.
* If rounding puts u * Z at or beyond the last running sum, the draw takes the
  last token with positive weight.
* Positions after the emitted token hold -1.

Pins (tests/test_oracle.py): scipy's logsumexp and the equal-logits closed
form for log Z; the per-token identity min(p,q) + max(0, p-q) = p; the
acceptance rate sum(min(p,q)); an exact enumeration of every outcome at V=4,
K=2 against the law that the pages' two paths give; a chi-square test that the
first emitted token follows p; the truncated-geometric mean of emitted tokens;
numpy's argmax for greedy; special cases (p == q, V == 1, T-scaling).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

FLAG_ZW_ZERO = 2       # residual mass rounded to zero; drew from p_n instead
FLAG_BAD_DRAFT = 4     # a draft id outside [0, V) was rejected


# ------------------------------------------------------------------ inputs --
def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored logits -> float64, exactly.  bf16 arrives as uint16 bit patterns."""
    if dtype == "fp32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ------------------------------------------------------------- the method --
def log_normalizer(y: np.ndarray) -> np.ndarray:
    """log sum_v exp(y[..., v]) with the maximum taken out first."""
    m = np.max(y, axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(y - m), axis=-1, keepdims=True)))[..., 0]


def softmax_from(y: np.ndarray, logz: np.ndarray) -> np.ndarray:
    return np.exp(y - logz[..., None])


def acceptance_threshold(log_p_x: np.ndarray, log_q_x: np.ndarray) -> np.ndarray:
    """min(1, p(x)/q(x)) evaluated as min(1, exp(log p(x) - log q(x))).  Where both are
    -inf the difference is NaN, and NaN >= 0 and u < NaN are false: the draft is rejected."""
    with np.errstate(invalid="ignore", over="ignore"):
        lr = log_p_x - log_q_x
        return np.where(lr >= 0.0, 1.0, np.exp(lr))


def residual(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """max(0, p - q), unnormalised."""
    return np.maximum(p - q, 0.0)


def inverse_cdf(w: np.ndarray, u: float):
    """Smallest v with C(v) > u * C(V-1), C the running sum of w.

    Returns (v, lo, hi): the token and the interval [lo, hi) of u (in units of
    the normalised running sum) that selects it."""
    c = np.cumsum(w)
    z = c[-1]
    t = u * z
    v = int(np.searchsorted(c, t, side="right"))
    if v >= len(w):
        v = int(np.flatnonzero(w > 0.0)[-1])
    lo = (c[v - 1] if v > 0 else 0.0) / z
    hi = c[v] / z
    return v, lo, hi


def first_argmax(row: np.ndarray) -> int:
    """First index attaining the maximum of the row."""
    return int(np.flatnonzero(row == np.max(row))[0])


# --------------------------------------------------------------- results --
@dataclasses.dataclass
class Result:
    tokens: np.ndarray        # [B, K+1] int32, -1 padded
    n_accepted: np.ndarray    # [B] int32
    logz: np.ndarray          # [B, 2K+1] natural-log normalisers: K+1 target rows then K draft rows
    thr: np.ndarray           # [B, K] acceptance thresholds (NaN where not evaluated)
    draw_lo: np.ndarray       # [B] normalised running-sum interval of the drawn token
    draw_hi: np.ndarray
    bonus: np.ndarray         # [B] bool: the draw came from p_K
    flags: np.ndarray         # [B] int32: FLAG_* bits

    def decisions(self) -> int:
        """Accept tests evaluated plus one draw per sequence."""
        K = self.thr.shape[1]
        return int(np.sum(np.minimum(self.n_accepted + 1, K)) + len(self.n_accepted))


def verify_sequence(yp: np.ndarray, yq: np.ndarray, x: np.ndarray, ua: np.ndarray, ur: float):
    """One sequence, sampling mode.  yp [K+1,V] and yq [K,V] are logits / T."""
    K, V = yq.shape
    lzp = log_normalizer(yp)
    lzq = log_normalizer(yq)
    thr = np.full(K, np.nan)
    flags = 0
    n = K
    for k in range(K):
        xk = int(x[k])
        if 0 <= xk < V:
            thr[k] = acceptance_threshold(yp[k, xk] - lzp[k], yq[k, xk] - lzq[k])
        else:
            thr[k] = 0.0
            flags |= FLAG_BAD_DRAFT
        if not (ua[k] < thr[k]):
            n = k
            break
    if n < K:
        p = softmax_from(yp[n], lzp[n])
        w = residual(p, softmax_from(yq[n], lzq[n]))
        if not np.sum(w) > 0.0:
            w = p
            flags |= FLAG_ZW_ZERO
    else:
        w = softmax_from(yp[K], lzp[K])
    j, lo, hi = inverse_cdf(w, float(ur))
    tokens = np.full(K + 1, -1, dtype=np.int32)
    tokens[:n] = x[:n]
    tokens[n] = j
    return dict(tokens=tokens, n=n, logz=np.concatenate([lzp, lzq]), thr=thr,
                lo=lo, hi=hi, bonus=(n == K), flags=flags)


def verify_greedy_sequence(lp: np.ndarray, x: np.ndarray):
    """One sequence, greedy mode.  lp [K+1,V] raw target logits."""
    K = lp.shape[0] - 1
    a = np.array([first_argmax(lp[k]) for k in range(K + 1)])
    n = K
    for k in range(K):
        if a[k] != int(x[k]):
            n = k
            break
    tokens = np.full(K + 1, -1, dtype=np.int32)
    tokens[:n] = x[:n]
    tokens[n] = a[n]
    flags = FLAG_BAD_DRAFT if np.any((x[: min(n + 1, K)] < 0) | (x[: min(n + 1, K)] >= lp.shape[1])) else 0
    return dict(tokens=tokens, n=n, flags=flags)


def verify(logits_p, logits_q, draft_tokens, u_accept, u_resample, T: float, dtype: str,
           seqs: Optional[np.ndarray] = None, num_drafts: Optional[np.ndarray] = None) -> Result:
    """Verify every sequence (or the subset ``seqs``) of a batch.

    logits_p [B,K+1,V], logits_q [B,K,V] (ignored when T == 0), draft_tokens
    [B,K], u_accept [B,K], u_resample [B]; logits as float32 or bf16 bits.

    ``num_drafts`` [B] (optional) gives sequence b its own draft count
    0 <= K_b <= K, as when the draft length is adapted per sequence ([B]
    "最优猜测长度 k：贪心还是保守？"): only its first K_b + 1 target rows, first
    K_b draft rows, drafts and accept uniforms take part, the bonus row is
    p_{K_b}, and outputs past the emitted token are -1 up to K + 1 entries.
    Rows a sequence does not use have NaN log normalisers."""
    B, K1, V = np.shape(logits_p)
    K = K1 - 1
    idx = np.arange(B) if seqs is None else np.asarray(seqs)
    S = len(idx)
    out = Result(tokens=np.full((S, K + 1), -1, np.int32), n_accepted=np.zeros(S, np.int32),
                 logz=np.full((S, 2 * K + 1), np.nan), thr=np.full((S, K), np.nan),
                 draw_lo=np.full(S, np.nan), draw_hi=np.full(S, np.nan),
                 bonus=np.zeros(S, bool), flags=np.zeros(S, np.int32))
    T = float(np.float32(T))
    for i, b in enumerate(idx):
        kb = K if num_drafts is None else int(num_drafts[b])
        x = np.asarray(draft_tokens[b])[:kb]
        if T == 0.0:
            r = verify_greedy_sequence(widen(logits_p[b][: kb + 1], dtype), x)
        else:
            yp = widen(logits_p[b][: kb + 1], dtype) / T
            yq = widen(logits_q[b][:kb], dtype) / T
            r = verify_sequence(yp, yq, x, np.asarray(u_accept[b])[:kb], float(u_resample[b]))
            out.logz[i, : kb + 1] = r["logz"][: kb + 1]
            out.logz[i, K + 1: K + 1 + kb] = r["logz"][kb + 1:]
            out.thr[i, :kb] = r["thr"]
            out.draw_lo[i] = r["lo"]
            out.draw_hi[i] = r["hi"]
            out.bonus[i] = r["bonus"]
        out.tokens[i, : kb + 1] = r["tokens"]
        out.n_accepted[i] = r["n"]
        out.flags[i] = r["flags"]
    return out


def position_stats(n_accepted: np.ndarray, num_drafts: np.ndarray, K: int) -> np.ndarray:
    """Per-position acceptance counters ([D] "Когда процент принятия падает":
    acceptance changes with the position in the draft; [D] "Мониторинг в
    производстве": it is the quantity to watch).  Returns [2K] integers:
    evaluated[k], then accepted[k].  Position k of a sequence is evaluated
    when all earlier drafts were accepted (k <= n) and it exists (k < K_b); it
    is accepted when k < n."""
    n = np.asarray(n_accepted)[:, None]
    kb = np.asarray(num_drafts)[:, None]
    k = np.arange(K)[None, :]
    evaluated = np.sum((k <= n) & (k < kb), axis=0)
    accepted = np.sum(k < n, axis=0)
    return np.concatenate([evaluated, accepted]).astype(np.int64)


def verify_batch(batch, seqs: Optional[np.ndarray] = None, workers: int = 1) -> Result:
    """Convenience wrapper for a ``workloads.Batch``-like object.  With
    workers > 1 the sequences are split into that many contiguous parts run in
    threads (numpy's array operations release the interpreter lock); the
    result is the same as one pass."""
    idx = np.arange(batch.B) if seqs is None else np.asarray(seqs)
    args = (batch.logits_p, batch.logits_q, batch.draft_tokens, batch.u_accept, batch.u_resample, batch.T,
            batch.dtype)
    nd = getattr(batch, "num_drafts", None)
    if workers <= 1 or len(idx) < 2:
        return verify(*args, idx, nd)
    from concurrent.futures import ThreadPoolExecutor
    parts = [p for p in np.array_split(idx, min(workers, len(idx))) if len(p)]
    with ThreadPoolExecutor(len(parts)) as ex:
        res = list(ex.map(lambda p: verify(*args, p, nd), parts))
    return Result(**{f.name: np.concatenate([getattr(r, f.name) for r in res])
                     for f in dataclasses.fields(Result)})


def draw_interval(logits_p_seq, logits_q_seq, n: int, j: int, u: float, T: float, dtype: str):
    """Normalised running-sum interval [lo, hi) that selects token j at the
    draw after n acceptances (residual if n < K, bonus row otherwise)."""
    T = float(np.float32(T))
    yp = widen(logits_p_seq, dtype) / T
    K = yp.shape[0] - 1
    p = softmax_from(yp[n], log_normalizer(yp[n]))
    if n < K:
        yq = widen(logits_q_seq, dtype)[n] / T
        w = residual(p, softmax_from(yq, log_normalizer(yq)))
        if not np.sum(w) > 0.0:
            w = p
    else:
        w = p
    c = np.cumsum(w)
    z = c[-1]
    lo = (c[j - 1] if j > 0 else 0.0) / z
    return lo, c[j] / z
