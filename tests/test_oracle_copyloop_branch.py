"""Pins for the oracle's second-readout branching (CopyLoop §A.2; CPU only).

* Full-depth verification keeps only continuations that agree with the
  verified prefix, so branching, like the pipeline it extends, must commit
  exactly full-depth greedy decoding's tokens, whatever the screening
  depth, the second readout depth, the copied-tail length and the admission
  limit (§2 "Full-Depth Verification", §A.1).
* Where no fork is ever made the run is the plain pipeline's, counter for
  counter.
* Forks are made and resolved both ways on the mixed-agreement models (the
  second line kept, and the first), so the checks above cover the paths a
  branch can get wrong: the second line's own KV states, the K/V that
  blocks older than the fork keep writing, and the resolution.  Besides the
  tokens, the cache the decoder leaves must hold a clean forward's K/V for
  every fed committed position at every depth, and every fork on a greedy
  prefix must sit where the depth-d2 and depth-ds predictions after that
  prefix differ, with those two heads.

Models: the tiny block applied 4 or 6 times with its block weights scaled
by 0.1 (every depth agrees: no fork), 0.3, 0.5 and 1.0 (shallow and deeper
readouts disagree more and more), on a seeded uniform prompt of 40 ids.
"""
import numpy as np
import pytest

import oracle
import oracle.copyloop as CL
from oracle.decoder import Config, KVCache
import synth


def _model(scale, D):
    shape = synth.TINY.replace(name=f"tiny-loop{D}", loop_depth=D)
    cfg = Config.of(shape)
    W = synth.weights_to_numpy(synth.make_weights(shape, seed=3))
    for k in ("w_qkv", "w_o", "w_gate_up", "w_down"):
        W["layers"][0][k] = W["layers"][0][k] * scale
    prompt = [int(t) for t in np.random.default_rng(7).integers(0, shape.vocab, size=40)]
    return cfg, W, prompt


def _fresh(cfg, cap=400):
    return KVCache.empty(cfg.loop_depth, cfg.n_kv_heads, cap, cfg.head_dim)


CASES = [  # scale, D, ds, d2, K, max_rows
    (0.1, 4, 1, 2, 8, 24), (0.1, 6, 2, 4, 8, 24),
    (0.3, 4, 1, 3, 8, 24), (0.3, 4, 2, 3, 8, 24), (0.3, 6, 2, 4, 8, 24),
    (0.5, 4, 1, 3, 8, 24), (0.5, 4, 2, 3, 4, 6), (1.0, 4, 1, 3, 8, 24), (1.0, 4, 1, 2, 8, 24),
    (1.0, 6, 2, 4, 3, 2),
    (1.0, 4, 1, 3, 8, 1), (0.5, 4, 2, 3, 8, 1),   # one row in flight: no tails, no room for a second child
]


def _readout(cfg, W, toks, depth):
    """depth-`depth` prediction after `toks`: a clean forward of the block
    applied `depth` times, then the final norm and head"""
    kv = _fresh(cfg)
    x = oracle.decoder.f64(W["tok_embed"])[np.asarray(toks, dtype=np.int64)]
    for d in range(depth):
        x = oracle.decoder.splice_layer(cfg, oracle.decoder._layer_weights(W, d, cfg), kv, d, x, 0)
    return int(np.argmax(oracle.final_logits(cfg, W, x[-1:])[0]))


@pytest.mark.parametrize("scale,D,ds,d2,K,max_rows", CASES)
def test_branching_equals_greedy_full_depth(scale, D, ds, d2, K, max_rows):
    """Greedy tokens; the cache the decoder leaves holds, at every depth,
    the K/V of a clean forward over every committed position that has been
    fed (the kept line's states, older blocks' writes included); every fork
    whose prefix is the greedy one was made where the depth-d2 and depth-ds
    predictions after that prefix differ, with those two heads."""
    cfg, W, prompt = _model(scale, D)
    n = 24
    want = oracle.greedy_decode(cfg, W, _fresh(cfg), prompt, n)
    kv = _fresh(cfg)
    got, st = CL.copyloop_branch_decode(cfg, W, kv, prompt, n, ds, d2, K, max_rows)
    assert got == want
    assert st["committed"] >= n and st["forks_kept"] <= st["forks"]
    full = oracle.greedy_decode(cfg, W, _fresh(cfg), prompt, st["committed"])
    P = len(prompt) + st["committed"] - 1
    ref = _fresh(cfg)
    oracle.decoder.splice_hidden(cfg, W, ref, 0, (prompt + full)[:P])
    for c in range(D):
        np.testing.assert_allclose(kv.k[c][:, :P], ref.k[c][:, :P], rtol=0, atol=1e-9)
        np.testing.assert_allclose(kv.v[c][:, :P], ref.v[c][:, :P], rtol=0, atol=1e-9)
    checked = 0
    for f in st["fork_log"]:
        if f["prefix"] != (prompt + full)[:len(f["prefix"])]:
            continue  # the parent's tail was refused later: not a greedy prefix
        assert f["h0"] == _readout(cfg, W, f["prefix"], ds)
        assert f["h1"] == _readout(cfg, W, f["prefix"], d2)
        assert f["h0"] != f["h1"]
        checked += 1
    assert checked == 0 or checked <= st["forks"]


def test_without_forks_it_is_the_pipeline():
    cfg, W, prompt = _model(0.1, 4)
    got, st = CL.copyloop_branch_decode(cfg, W, _fresh(cfg), prompt, 24, 1, 2, 8, 24)
    ref, st0 = CL.copyloop_decode(cfg, W, _fresh(cfg), prompt, 24, 1, 8, 24)
    assert st["forks"] == 0
    assert got == ref
    for k in st0:
        assert st[k] == st0[k], k
    assert st["fork_log"] == []


@pytest.mark.parametrize("scale,D,ds,d2,kept,lost", [(0.3, 4, 1, 3, True, False), (0.5, 4, 2, 3, True, False),
                                                     (1.0, 4, 1, 2, False, True)])
def test_forks_are_made_and_resolved_both_ways(scale, D, ds, d2, kept, lost):
    """The second child's line is kept in some runs and the first child's
    in another (that run checks that the second line never touched the
    first's KV states: its final cache is pinned above)."""
    cfg, W, prompt = _model(scale, D)
    _, st = CL.copyloop_branch_decode(cfg, W, _fresh(cfg), prompt, 24, ds, d2, 8, 24)
    assert st["forks"] > 0
    assert (st["forks_kept"] > 0) == kept and (st["forks_lost"] > 0) == lost
    assert st["forks_kept"] + st["forks_lost"] <= st["forks"]


def test_branch_depth_checked():
    cfg, W, prompt = _model(0.1, 4)
    for ds, d2 in ((2, 2), (3, 2), (1, 4), (0, 2)):
        with pytest.raises(ValueError):
            CL.copyloop_branch_decode(cfg, W, _fresh(cfg), prompt, 4, ds, d2, 8, 24)
