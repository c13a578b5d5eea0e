"""Pins for the oracle's suffix matcher (CopyLoop §2 "Block Construction").

The matcher is pinned against an independent brute force that enumerates
every (length, start) pair and picks the best by (longest length, latest
start), over every sequence of length <= 10 on small alphabets, plus seeded
fuzz at realistic length and the hand-worked cases in
tests/golden/suffix_cases.txt.
"""
import itertools
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "suffix_cases.txt")


def brute(x, max_n, min_n, K):
    T = len(x)
    best = None
    for n in range(min_n, max_n + 1):
        for p in range(0, T):
            if p + n > T - 1:          # the match must be followed by a token
                continue
            if n > T - 1:
                continue
            if list(x[p:p + n]) == list(x[T - n:]):
                key = (n, p)
                if best is None or key > best:
                    best = key
    if best is None:
        return [], -1
    n, p = best
    return list(x[p + n:p + n + K]), p + n


@pytest.mark.parametrize("alphabet", [2, 3])
def test_exhaustive_small(alphabet):
    for T in range(0, 11 if alphabet == 2 else 9):
        for seq in itertools.product(range(alphabet), repeat=T):
            for K in (1, 2, 4):
                got, pos = oracle.suffix_match(seq, 4, 1, K)
                exp, epos = brute(seq, 4, 1, K)
                assert list(got) == exp and pos == epos, (seq, K)


def test_min_ngram_above_one():
    r = np.random.default_rng(5)
    for _ in range(500):
        x = list(r.integers(0, 3, size=int(r.integers(2, 14))))
        for mn in (2, 3):
            got, pos = oracle.suffix_match(x, 4, mn, 3)
            exp, epos = brute(x, 4, mn, 3)
            assert list(got) == exp and pos == epos


def test_fuzz_zipf_long():
    r = synth.rng(123)
    for trial in range(40):
        T = int(r.integers(200, 4096))
        x = synth.zipf_ids(r, T, 32000)
        if trial % 3 == 0:  # plant a repeat of the tail
            n = int(r.integers(1, 6))
            p = int(r.integers(0, T - n - 1))
            x[T - n:] = x[p:p + n]
        got, pos = oracle.suffix_match(x, 4, 1, 8)
        exp, epos = brute_fast(x, 4, 1, 8)
        assert list(got) == exp and pos == epos


def brute_fast(x, max_n, min_n, K):
    """Vectorised brute force: for each n, a boolean vector of match starts."""
    x = np.asarray(x)
    T = len(x)
    best = None
    for n in range(min_n, max_n + 1):
        if n > T - 1:
            break
        starts = np.arange(0, T - n)          # p + n <= T - 1
        ok = np.ones(len(starts), dtype=bool)
        for j in range(n):
            ok &= x[starts + j] == x[T - n + j]
        if ok.any():
            best = (n, int(starts[ok].max()))
    if best is None:
        return [], -1
    n, p = best
    return list(x[p + n:p + n + K]), p + n


def load_golden():
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            hist, k, exp, pos = [s.strip() for s in line.split("|")]
            cases.append(([int(t) for t in hist.split()], int(k),
                          [int(t) for t in exp.split()] if exp else [], int(pos)))
    return cases


def test_golden_cases():
    cases = load_golden()
    assert len(cases) >= 6
    for hist, K, exp, pos in cases:
        got, gpos = oracle.suffix_match(hist, 4, 1, K)
        assert list(got) == exp and gpos == pos, (hist, K)
