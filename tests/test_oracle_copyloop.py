"""Pins for the oracle's CopyLoop pipeline (CPU only).

CopyLoop §2 "Full-Depth Verification": every committed token is the
full-depth prediction after an already verified prefix, so the pipeline's
output must equal plain full-depth greedy decoding, whatever the screening
depth, the copied-tail length or the admission limit (§A.1).  The tick
(§2 "Concurrent Pipeline") is pinned separately: a block taken through all
D depths one tick at a time gives the looped splice's logits and caches.

The model is the tiny block applied four times with its block weights scaled
down, so that the residual update is small against the embedding: at 0.1
every depth predicts the same token (copies pay off), at 0.3 the shallow
predictions agree with the full-depth ones on 60-83 % of positions, so
screening prunes and verification discards (the paths a scheduler can get
wrong).  The prompt holds the model's own greedy continuation, so copying
from context pays.
"""
import numpy as np
import pytest

import oracle
from oracle.decoder import Config, KVCache
import synth

D = 4


def _model(scale):
    shape = synth.TINY.replace(name="tiny-loop4", loop_depth=D)
    cfg = Config.of(shape)
    W = synth.weights_to_numpy(synth.make_weights(shape, seed=3))
    for k in ("w_qkv", "w_o", "w_gate_up", "w_down"):
        W["layers"][0][k] = W["layers"][0][k] * scale
    r = np.random.default_rng(8)
    seed = [int(t) for t in r.integers(0, shape.vocab, size=24)]
    kv = KVCache.empty(D, shape.n_kv_heads, 400, shape.head_dim)
    cont = oracle.greedy_decode(cfg, W, kv, seed, 40)
    prompt = seed + cont
    return cfg, W, prompt


@pytest.fixture(scope="module", params=[0.1, 0.3], ids=["agreeing", "mixed"])
def model(request):
    return _model(request.param)


def _fresh(cfg, cap=400):
    return KVCache.empty(cfg.loop_depth, cfg.n_kv_heads, cap, cfg.head_dim)


@pytest.mark.parametrize("ds,K,max_rows", [(1, 4, 64), (2, 4, 64), (3, 6, 64), (1, 0, 64), (2, 4, 3), (1, 3, 1)])
def test_pipeline_equals_greedy_full_depth(model, ds, K, max_rows):
    """Every committed token equals full-depth greedy decoding's, on the
    model whose depths agree and on the one whose screening and verification
    reject (at least one case there prunes and discards: see below)."""
    cfg, W, prompt = model
    n = 30
    want = oracle.greedy_decode(cfg, W, _fresh(cfg), prompt, n)
    got, st = oracle.copyloop_decode(cfg, W, _fresh(cfg), prompt, n, ds, K, max_rows)
    assert got == want
    assert st["committed"] >= n
    # every block costs one row per depth at least; nothing runs beyond the limit
    assert st["rows_run"] <= st["ticks"] * max_rows
    if K == 0:
        assert st["proposed"] == 0 and st["screened_out"] == 0


def test_copies_pay_off():
    """With the model's own continuation in the prompt, copied tails survive
    screening and verification: far fewer ticks than the n x D of
    token-by-token full-depth decoding."""
    cfg, W, prompt = _model(0.1)
    n = 30
    got, st = oracle.copyloop_decode(cfg, W, _fresh(cfg), prompt, n, 1, 6, 64)
    assert got == oracle.greedy_decode(cfg, W, _fresh(cfg), prompt, n)
    assert st["proposed"] > st["screened_out"]
    assert st["ticks"] < n * cfg.loop_depth // 2


def test_ticks_through_all_depths_equal_the_looped_splice(model):
    cfg, W, prompt = model
    L, span = len(prompt), [5, 900, 17, 17, 3]
    kv_a, kv_b = _fresh(cfg), _fresh(cfg)
    x = oracle.decoder.splice_hidden(cfg, W, kv_a, 0, prompt)
    oracle.decoder.splice_hidden(cfg, W, kv_b, 0, prompt)
    want = oracle.final_logits(cfg, W, oracle.decoder.splice_hidden(cfg, W, kv_a, L, span))
    state = np.zeros((8, cfg.d_model))
    for d in range(cfg.loop_depth):
        lg = oracle.loop_step(cfg, W, kv_b, [dict(pos=L, rows=len(span), depth=d, state=2,
                                                    readout=int(d == cfg.loop_depth - 1))], span, state)
    assert np.allclose(lg[0], want, rtol=1e-12, atol=1e-12)
    for c in range(cfg.loop_depth):
        assert np.array_equal(kv_a.k[c][:, :L + len(span)], kv_b.k[c][:, :L + len(span)])
        assert np.array_equal(kv_a.v[c][:, :L + len(span)], kv_b.v[c][:, :L + len(span)])


def test_tick_groups_at_mixed_depths_are_independent(model):
    """Two groups in one tick (an older one deeper) give what each gives alone."""
    cfg, W, prompt = model
    L = len(prompt)
    kv = _fresh(cfg)
    oracle.decoder.splice_hidden(cfg, W, kv, 0, prompt)
    st = np.zeros((8, cfg.d_model))
    a, b = [7, 8, 9], [11, 12]
    for d in range(2):                                   # the older group reaches depth 2
        oracle.loop_step(cfg, W, kv, [dict(pos=L, rows=3, depth=d, state=0, readout=0)], a, st)
    kv1, st1 = kv.copy(), st.copy()
    both = oracle.loop_step(cfg, W, kv1, [dict(pos=L, rows=3, depth=2, state=0, readout=1),
                                          dict(pos=L + 3, rows=2, depth=0, state=3, readout=1)], a + b, st1)
    kv2, st2 = kv.copy(), st.copy()
    one = oracle.loop_step(cfg, W, kv2, [dict(pos=L, rows=3, depth=2, state=0, readout=1)], a, st2)
    two = oracle.loop_step(cfg, W, kv2, [dict(pos=L + 3, rows=2, depth=0, state=3, readout=1)], b, st2)
    assert np.array_equal(both[0], one[0]) and np.array_equal(both[1], two[0])
    assert np.array_equal(st1, st2)


def test_mixed_model_exercises_pruning_and_discards():
    cfg, W, prompt = _model(0.3)
    n = 30
    for ds, K in ((1, 6), (2, 4)):
        got, st = oracle.copyloop_decode(cfg, W, _fresh(cfg), prompt, n, ds, K, 64)
        assert got == oracle.greedy_decode(cfg, W, _fresh(cfg), prompt, n)
        assert st["screened_out"] > 0 and st["discarded"] > 0


def _shallow_continuation(cfg, W, seed, n, depth):
    """The model's greedy continuation of ``seed`` read out at ``depth``."""
    kv = _fresh(cfg)
    x = oracle.decoder.splice_hidden(cfg, W, kv, 0, seed)
    out = [int(np.argmax(oracle.final_logits(cfg, W, x[-1:])[0]))]
    while len(out) < n:
        lg = oracle.decoder.decode_step(cfg, W, kv, len(seed) + len(out) - 1, out[-1], depth=depth)
        out.append(int(np.argmax(lg)))
    return out


def test_copies_that_pass_screening_but_fail_verification():
    """A prompt holding the model's greedy continuation read out at the
    screening depth: copies taken from it tend to agree with the shallow
    predictions, survive screening and are refused at full depth, where the
    correction token must take over."""
    cfg, W, _ = _model(0.3)
    for seed_id, ds in ((11, 2), (10, 1)):
        r = np.random.default_rng(seed_id)
        seed = [int(t) for t in r.integers(0, cfg.vocab, size=24)]
        sh = _shallow_continuation(cfg, W, seed, 40, ds)
        prompt = seed + sh if ds == 2 else seed + sh + seed + sh[:5]
        n = 30
        got, st = oracle.copyloop_decode(cfg, W, _fresh(cfg), prompt, n, ds, 6, 64)
        assert got == oracle.greedy_decode(cfg, W, _fresh(cfg), prompt, n)
        assert st["rejected"] > 0
