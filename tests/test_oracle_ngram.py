"""Pins of the n-gram (prompt-lookup) proposer oracle: the pages' worked
example and an independent formulation by string search."""
import json
import os
import re

import numpy as np

from oracle import ngram

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ngram_example.json")


def test_the_pages_function_header_example():
    g = json.load(open(GOLDEN))
    words = g["history"]
    vocab = {w: i for i, w in enumerate(dict.fromkeys(words))}
    h = np.array([vocab[w] for w in words])
    draft, count = ngram.propose_sequence(h, 1, g["n_max"], 1, g["K"])
    inv = {i: w for w, i in vocab.items()}
    assert [inv[t] for t in draft[:count]] == g["proposal"]


def _by_string_search(h, n_min, n_max, min_hits, K):
    """The same rule through Python's string search: tokens joined with
    separators; occurrences of the suffix found by an overlapping regular
    expression search, the latest by position."""
    s = "," + ",".join(map(str, h)) + ","
    starts = np.cumsum([1] + [len(str(t)) + 1 for t in h])   # offset of token i in s
    L = len(h)
    for n in range(min(n_max, L), n_min - 1, -1):
        pat = "," + ",".join(map(str, h[L - n:])) + ","
        offs = [m.start() for m in re.finditer("(?=" + re.escape(pat) + ")", s)]
        ends = [int(np.searchsorted(starts, o + 1)) + n for o in offs]   # token index after the n-gram
        ends = [e for e in ends if e <= L - 1]
        if len(ends) >= min_hits and ends:
            e = max(ends)
            return list(h[e:min(e + K, L)])
    return []


def test_agrees_with_string_search_on_random_histories():
    rng = np.random.default_rng(0)
    for _ in range(400):
        L = int(rng.integers(1, 60))
        h = rng.integers(0, int(rng.integers(2, 6)), L)
        n_max = int(rng.integers(1, 6))
        n_min = int(rng.integers(1, n_max + 1))
        min_hits = int(rng.integers(1, 4))
        K = int(rng.integers(1, 6))
        draft, count = ngram.propose_sequence(h, n_min, n_max, min_hits, K)
        assert list(draft[:count]) == _by_string_search(h, n_min, n_max, min_hits, K)
        assert np.all(draft[count:] == -1)


def test_periodic_history_continues_its_period():
    """The latest occurrence of the 4-gram (2, 3, 1, 2) ends three tokens
    before the end, so the proposal continues the period and stops at the
    history's end."""
    h = np.array([1, 2, 3] * 5 + [1, 2])
    draft, count = ngram.propose_sequence(h, 1, 4, 1, 4)
    assert count == 3 and draft.tolist() == [3, 1, 2, -1]


def test_no_earlier_occurrence_proposes_nothing():
    draft, count = ngram.propose_sequence(np.arange(20), 1, 3, 1, 4)
    assert count == 0 and np.all(draft == -1)
    draft, count = ngram.propose_sequence(np.array([5, 5]), 2, 3, 1, 4)   # shorter than the smallest n + 1
    assert count == 0
