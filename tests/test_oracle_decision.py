"""Pins for masked argmax and acceptance (CPU only).

Masked argmax (Copy-as-Decode §2.3) is pinned against a pure-Python brute
force over every id with deliberately constructed ties.  Acceptance
(CopyLoop §2 "Shallow Screening" / "Full-Depth Verification";
Copy-as-Decode Fig. 1) is pinned by planting: a span built from the model's
own greedy chain must be accepted whole with the next greedy token as the
bonus; corrupting position j must give exactly j; COMMIT always gives N.
"""
import numpy as np
import pytest

import oracle
from oracle.decision import COMMIT, VERIFY
from oracle.decoder import Config, KVCache
import synth


def brute_argmax(row, words):
    best = -1
    for v in range(len(row)):
        if words is not None and not (int(words[v // 32]) >> (v % 32)) & 1:
            continue
        if best < 0 or row[v] > row[best]:
            best = v
    return best


def test_masked_argmax_brute_force_with_ties():
    r = np.random.default_rng(0)
    for V in (1, 5, 31, 32, 33, 64, 100):
        for _ in range(30):
            N = 4
            logits = r.integers(-3, 4, size=(N, V)).astype(np.float64)   # many ties
            allowed = r.random((N, V)) < r.uniform(0.0, 1.0)
            mask = synth.pack_mask(allowed)
            got = oracle.masked_argmax(logits, mask)
            for k in range(N):
                assert got[k] == brute_argmax(logits[k], mask[k])
            got_nm = oracle.masked_argmax(logits, None)
            for k in range(N):
                assert got_nm[k] == brute_argmax(logits[k], None)


def test_masked_argmax_lowest_id_on_tie_and_empty_row():
    logits = np.array([[1.0, 5.0, 5.0, 2.0], [0.0, 0.0, 0.0, 0.0]])
    assert list(oracle.masked_argmax(logits, None)) == [1, 0]
    mask = synth.pack_mask(np.array([[False, False, True, True], [False] * 4]))
    assert list(oracle.masked_argmax(logits, mask)) == [2, -1]


def brute_margin(row, words):
    """Top-2 gap by pairs: the best allowed value minus the best allowed
    value at any *other* allowed id (a tie at the top gives 0); fewer than
    two allowed ids give inf."""
    ids = [v for v in range(len(row)) if words is None or (int(words[v // 32]) >> (v % 32)) & 1]
    if len(ids) < 2:
        return np.inf
    top = ids[0]
    for v in ids:
        if row[v] > row[top]:
            top = v
    rival = None
    for v in ids:
        if v != top and (rival is None or row[v] > row[rival]):
            rival = v
    return row[top] - row[rival]


def test_top2_margin_hand_worked_cases():
    logits = np.array([[1.0, 5.0, 5.0, 2.0],      # tie at the top: 0
                       [1.0, 5.0, 4.0, 2.0],      # 5 - 4
                       [9.0, 5.0, 4.0, 2.0],      # masked below: the 9 is banned, 5 - 4
                       [9.0, 5.0, 4.0, 2.0],      # one allowed id: no rival
                       [9.0, 5.0, 4.0, 2.0],      # nothing allowed
                       [-3.0, -1.0, -2.5, -7.0]])  # negative logits: -1 - (-2.5)
    allowed = np.array([[True] * 4, [True] * 4, [False, True, True, True],
                        [False, False, True, False], [False] * 4, [True] * 4])
    got = oracle.top2_margin(logits, synth.pack_mask(allowed))
    assert list(got) == [0.0, 1.0, 1.0, np.inf, np.inf, 1.5]
    # unmasked: the banned 9 is back on top
    assert oracle.top2_margin(logits[2:3], None)[0] == 4.0


def test_top2_margin_brute_force():
    r = np.random.default_rng(3)
    for V in (1, 2, 31, 32, 33, 70):
        for _ in range(40):
            N = 3
            logits = r.integers(-4, 5, size=(N, V)).astype(np.float64) + r.choice([0.0, 0.25], size=(N, V))
            allowed = r.random((N, V)) < r.uniform(0.0, 1.0)
            mask = synth.pack_mask(allowed)
            got = oracle.top2_margin(logits, mask)
            got_nm = oracle.top2_margin(logits, None)
            for k in range(N):
                assert got[k] == brute_margin(logits[k], mask[k])
                assert got_nm[k] == brute_margin(logits[k], None)


def test_pack_mask_bit_order():
    allowed = np.zeros((1, 70), dtype=bool)
    allowed[0, [0, 31, 32, 69]] = True
    w = synth.pack_mask(allowed)
    assert w.shape == (1, 3)
    assert w[0, 0] == (1 | (1 << 31)) and w[0, 1] == 1 and w[0, 2] == (1 << 5)


def test_acceptance_rule_small():
    assert oracle.acceptance([9, 9, 9], [1, 2, 3], COMMIT) == 3
    assert oracle.acceptance([2, 3, 7], [1, 2, 3], VERIFY) == 3
    assert oracle.acceptance([2, 8, 7], [1, 2, 3], VERIFY) == 2
    assert oracle.acceptance([5, 3, 7], [1, 2, 3], VERIFY) == 1
    assert oracle.acceptance([4], [1], VERIFY) == 1
    with pytest.raises(ValueError):
        oracle.acceptance([], [], VERIFY)


@pytest.mark.parametrize("use_mask", [False, True])
def test_planted_acceptance(use_mask):
    shape = synth.TINY
    cfg = Config.of(shape)
    W = synth.weights_to_numpy(synth.make_weights(shape, seed=11))
    L, N = 24, 10
    prompt = synth.uniform_prompt(L, shape.vocab, seed=12)
    mask = synth.banned_ids_mask(N, shape.vocab, 16, seed=13) if use_mask else None
    base = KVCache.empty(1, 4, L + N + 1, 64)
    oracle.prefill(cfg, W, base, prompt)
    # greedy chain: s[0] given, s[j] = masked argmax after s[j-1]
    kv = base.copy()
    span = [int(prompt[-1]) ^ 5]
    bonus = None
    for j in range(N):
        lg = oracle.decode_step(cfg, W, kv, L + j, span[j])[None]
        a = int(oracle.masked_argmax(lg, None if mask is None else mask[j:j + 1])[0])
        if j + 1 < N:
            span.append(a)
        else:
            bonus = a
    kv1 = base.copy()
    lg = oracle.splice(cfg, W, kv1, L, span)
    a = oracle.masked_argmax(lg, mask)
    assert oracle.acceptance(a, span, VERIFY) == N
    assert a[N - 1] == bonus
    assert oracle.acceptance(a, span, COMMIT) == N
    for j in (1, 4, N - 1):
        bad = list(span)
        bad[j] = (bad[j] + 1) % shape.vocab
        kv2 = base.copy()
        a2 = oracle.masked_argmax(oracle.splice(cfg, W, kv2, L, bad), mask)
        assert oracle.acceptance(a2, bad, VERIFY) == j
        assert a2[j - 1] == span[j]          # the correction is the greedy token
        assert oracle.acceptance(a2, bad, COMMIT) == N
