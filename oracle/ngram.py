"""Plain CPU oracle of the n-gram (prompt-lookup) draft proposer.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

Sources (cited by title and section):
  [A] "Speculative Decoding: Cách LLM Sinh Văn Bản Nhanh Gấp 2–3 Lần"
      (anhtu.dev): Prompt Lookup proposes phrases already in the context; the
      vLLM "ngram" configuration with a maximum n-gram window.
  [D] "Спекулятивное декодирование: ускорение инференса LLM на 20–50%"
      (glukhov.org), "Спекулятивное декодирование на n-граммах": when the
      last tokens match an earlier n-gram, propose what followed it; n-gram
      size, a minimum number of hits, a few tokens per match.

Reading (the pages give the idea, not the exact rule): for a history
h[0..L) and sizes n_max down to n_min, an occurrence of the n-gram ending at
e (1 <= e <= L - 1, so at least one token follows it) is a position where
h[e-n..e) == h[L-n..L).  The proposer takes the largest n with at least
min_hits occurrences and proposes h[e*..min(e* + K, L)) for the latest such
occurrence e*; without one it proposes nothing.
"""
from __future__ import annotations

import numpy as np


def propose_sequence(history, n_min: int, n_max: int, min_hits: int, K: int):
    """One history.  Returns (draft [K] int32 with -1 padding, count)."""
    h = np.asarray(history, dtype=np.int64)
    L = len(h)
    draft = np.full(K, -1, np.int32)
    for n in range(min(n_max, L), n_min - 1, -1):
        if n < 1:
            break
        suffix = h[L - n:]
        ends = [e for e in range(n, L) if np.array_equal(h[e - n:e], suffix)]
        if len(ends) >= min_hits and ends:
            e = max(ends)
            cont = h[e:min(e + K, L)]
            draft[: len(cont)] = cont
            return draft, len(cont)
    return draft, 0


def propose(histories, lengths, n_min: int, n_max: int, min_hits: int, K: int):
    """A batch: histories [B, L_max] (padded), lengths [B].  Returns (draft
    [B, K], count [B])."""
    B = len(lengths)
    out = np.full((B, K), -1, np.int32)
    cnt = np.zeros(B, np.int32)
    for b in range(B):
        out[b], cnt[b] = propose_sequence(np.asarray(histories[b])[: int(lengths[b])], n_min, n_max, min_hits, K)
    return out, cnt
