"""Pins for the looped variant and the batched form (CPU only).

* With the screening depth equal to the full depth, the looped model is a
  plain D-deep stack whose blocks all carry the shared weights (CopyLoop §2
  "Concurrent Pipeline": every depth keeps its own KV states).
* Screening keeps exactly the prefix planted to agree at the shallow depth.
* The batched splice equals independent single-sequence splices.
"""
import numpy as np

import oracle
from oracle.decision import VERIFY, COMMIT
from oracle.decoder import Config, KVCache
import synth

LOOP_SMALL = synth.Shape("loop-small", 1, 128, 4, 4, 32, 256, 300, dtype="f32", loop_depth=4)


def test_looped_equals_tied_stack():
    W = synth.weights_to_numpy(synth.make_weights(LOOP_SMALL, seed=2, std=0.05))
    cfg = Config.of(LOOP_SMALL)
    prompt = synth.uniform_prompt(20, LOOP_SMALL.vocab, seed=3)
    span = synth.uniform_prompt(5, LOOP_SMALL.vocab, seed=4)
    kv = KVCache.empty(4, 4, 32, 32)
    oracle.prefill(cfg, W, kv, prompt)
    kv_tied = kv.copy()
    res = oracle.looped_splice(cfg, W, kv, 20, span, screen_depth=4)
    tied_shape = LOOP_SMALL.replace(n_layers=4, loop_depth=1)
    Wt = dict(W, layers=[W["layers"][0]] * 4)
    lt = oracle.splice(Config.of(tied_shape), Wt, kv_tied, 20, span)
    m = res["survivors"]
    assert np.allclose(res["screen_logits"], lt, atol=1e-12)
    assert np.allclose(res["logits"], lt[:m], atol=1e-12)
    for c in range(4):
        assert np.allclose(kv.k[c][:, :20 + m], kv_tied.k[c][:, :20 + m], atol=1e-12)


def test_screening_keeps_planted_prefix():
    W = synth.weights_to_numpy(synth.make_weights(LOOP_SMALL, seed=5, std=0.05))
    cfg = Config.of(LOOP_SMALL)
    L, ds = 16, 2
    prompt = synth.uniform_prompt(L, LOOP_SMALL.vocab, seed=6)
    base = KVCache.empty(4, 4, 32, 32)
    oracle.prefill(cfg, W, base, prompt)
    # shallow greedy chain of 3 tokens after the head, then a planted wrong token
    kv = base.copy()
    span = [7]
    for j in range(3):
        lg = oracle.decode_step(cfg, W, kv, L + j, span[j], depth=ds)[None]
        span.append(int(oracle.masked_argmax(lg, None)[0]))
    span.append((span[-1] + 1) % LOOP_SMALL.vocab)
    # the planted token must disagree with the shallow prediction at position 3
    lg = oracle.decode_step(cfg, W, kv, L + 3, span[3], depth=ds)[None]
    if int(oracle.masked_argmax(lg, None)[0]) == span[4]:
        span[4] = (span[4] + 1) % LOOP_SMALL.vocab
    kv1 = base.copy()
    res = oracle.looped_splice(cfg, W, kv1, L, span, screen_depth=ds)
    assert res["survivors"] == 4
    assert list(res["argmax"][4:]) == [-1]
    # deeper caches hold only the survivors; pruned slots stay as they were
    for c in range(ds, 4):
        assert np.array_equal(kv1.k[c][:, L + 4:], base.k[c][:, L + 4:])
        assert not np.array_equal(kv1.k[c][:, L:L + 4], base.k[c][:, L:L + 4])
    assert 1 <= res["accepted"] <= 4


def test_batched_equals_independent():
    shape = synth.Shape("b-small", 2, 128, 4, 2, 32, 256, 400, dtype="f32")
    cfg = Config.of(shape)
    W = synth.weights_to_numpy(synth.make_weights(shape, seed=7))
    r = np.random.default_rng(8)
    caches, Ls, spans, masks = [], [], [], []
    for b in range(3):
        L = int(r.integers(3, 20))
        kv = KVCache.empty(2, 2, 40, 32)
        oracle.prefill(cfg, W, kv, r.integers(0, 400, size=L))
        caches.append(kv); Ls.append(L); spans.append(list(r.integers(0, 400, size=int(r.integers(1, 6)))))
        masks.append(synth.banned_ids_mask(len(spans[-1]), 400, 10, seed=b))
    ref = [c.copy() for c in caches]
    lg, am, acc = oracle.batched_splice(cfg, W, caches, Ls, spans, masks, VERIFY)
    for b in range(3):
        l1 = oracle.splice(cfg, W, ref[b], Ls[b], spans[b])
        assert np.array_equal(l1, lg[b])
        a1 = oracle.masked_argmax(l1, masks[b])
        assert np.array_equal(a1, am[b])
        assert acc[b] == oracle.acceptance(a1, spans[b], VERIFY)
