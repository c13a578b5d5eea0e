"""Pins for the oracle's Copy-as-Decode program decoder (CPU only).

The automaton (Copy-as-Decode §2.3 and the appendix paragraph "States.") is
pinned by brute force: for every document size U up to 120, every range
"a-b" with 1 <= a <= b <= U can be spelled digit by digit under the masks,
and every other digit string (leading zero, 0, above U, b below a) is
refused at some digit; random walks that pick any allowed id at every
decision always form a program that an independent parser of the grammar
(§2.1) accepts.  The decoder is pinned by what the pages fix: drafts inside a
gen body change nothing (§5 "Composition with speculative decoding": the
verification is lossless), every decision equals the masked argmax of
feeding the same stream one token at a time (the splice is N decode steps,
§2.4), and a copy op resolves to the document's lines (or tokens, §5
"Token-level extension").
"""
import numpy as np
import pytest

import oracle
from oracle import cad_program as CP
from oracle.decoder import Config, KVCache
import synth

# ids of the structural literals in the tiny vocabulary (tokenizer-specific
# tables are resolved once at load; these are arbitrary distinct ids)
T = CP.Table(lt=27, lt_slash=522, gt=29, copy=856, gen=437, program=149, kw=512, eq_quote=428,
             quote=1, slash_gt=257, hyphen=12, digits=tuple(range(15, 25)))


def _spell(n):
    return [T.digits[int(c)] for c in str(n)]


def _walk(fsm, seq):
    """Feed a sequence of chosen ids; False at the first one the masks refuse."""
    for tok in seq:
        allowed = fsm.allowed()
        if allowed is not None and tok not in allowed:
            return False
        fsm.choose(tok)
    return True


@pytest.mark.parametrize("U", [1, 7, 9, 10, 11, 19, 20, 99, 100, 101, 120])
def test_range_masks_brute_force(U):
    for a in range(0, U + 3):
        for b in range(0, U + 3):
            f = CP.Fsm(T, U, 8, 16)
            f.choose(T.lt)
            f.choose(T.copy)
            seq = _spell(a) + [T.hyphen] + _spell(b) + [T.quote]
            ok = _walk(f, seq)
            assert ok == (1 <= a <= b <= U), (U, a, b)
            if ok:
                assert f.ops[-1] == {"op": "copy", "a": a, "b": b} and f.state == CP.AWAIT_OP
    f = CP.Fsm(T, 50, 8, 16)
    f.choose(T.lt)
    f.choose(T.copy)
    assert not _walk(f, [T.digits[0]])        # no leading zero
    f = CP.Fsm(T, 50, 8, 16)
    assert f.allowed() == [T.lt]              # at least one op before the end
    f.choose(T.lt)
    assert sorted(f.allowed()) == sorted([T.copy, T.gen])


def parse(stream, U, doc_lines, unit):
    """Independent reading of the grammar over a token stream: returns the
    ops, or raises on the first deviation."""
    i, ops = 0, []

    def expect(seq):
        nonlocal i
        assert stream[i:i + len(seq)] == list(seq), (i, stream[i:i + len(seq)], seq)
        i += len(seq)

    def number():
        nonlocal i
        ds = []
        while i < len(stream) and stream[i] in T.digits:
            ds.append(T.digits.index(stream[i]))
            i += 1
        assert ds and ds[0] != 0
        return int("".join(map(str, ds)))
    while True:
        if stream[i] == T.lt_slash:
            assert ops, "a program needs an op"
            expect([T.lt_slash, T.program, T.gt])
            assert i == len(stream)
            return ops
        expect([T.lt])
        if stream[i] == T.copy:
            expect([T.copy, T.kw, T.eq_quote])
            a = number()
            expect([T.hyphen])
            b = number()
            expect([T.quote, T.slash_gt])
            assert 1 <= a <= b <= U
            expect(CP.span_units(doc_lines, a, b, unit))
            ops.append(("copy", a, b))
        else:
            expect([T.gen, T.gt])
            body = []
            while stream[i:i + 3] != [T.lt_slash, T.gen, T.gt]:
                body.append(stream[i])
                i += 1
            expect([T.lt_slash, T.gen, T.gt])
            ops.append(("gen", tuple(body)))


@pytest.mark.parametrize("seed", range(40))
def test_random_walks_form_valid_programs(seed):
    """Any id the masks allow, at every decision, gives a parsable program
    (gen bodies drawn from a small alphabet that includes the end-of-gen ids,
    so bodies end by the window as well as by the length cap)."""
    r = np.random.default_rng(seed)
    doc = [[int(x) for x in r.integers(600, 700, size=int(r.integers(1, 5)))] for _ in range(int(r.integers(1, 30)))]
    unit = "lines" if seed % 2 == 0 else "tokens"
    U = len(doc) if unit == "lines" else sum(map(len, doc))
    f = CP.Fsm(T, U, int(r.integers(1, 6)), int(r.integers(1, 9)))
    stream = []
    while f.state != CP.DONE:
        allowed = f.allowed()
        if allowed is None:
            pool = [T.lt_slash, T.gen, T.gt, 700, 701]
            tok = int(pool[r.integers(0, len(pool))])
        else:
            tok = int(allowed[r.integers(0, len(allowed))])
        feed = f.choose(tok)
        if feed is None:
            op = f.ops[-1]
            feed = [T.quote, T.slash_gt] + CP.span_units(doc, op["a"], op["b"], unit)
        stream += feed
        assert len(stream) < 5000
    ops = parse(stream, U, doc, unit)
    assert len(ops) == len(f.ops) <= f.max_ops
    for o, fo in zip(ops, f.ops):
        if o[0] == "copy":
            assert fo == {"op": "copy", "a": o[1], "b": o[2]}
        else:
            assert tuple(fo["body"]) == o[1] and len(o[1]) <= f.max_gen


@pytest.fixture(scope="module")
def tiny():
    shape = synth.TINY
    cfg = Config.of(shape)
    W = synth.weights_to_numpy(synth.make_weights(shape, seed=5))
    r = np.random.default_rng(6)
    doc = [[int(x) for x in r.integers(600, 1000, size=int(r.integers(3, 9)))] for _ in range(14)]
    prompt = [int(x) for x in r.integers(0, 1000, size=20)] + [x for line in doc for x in line] + [T.lt, T.program,
                                                                                                  T.gt]
    return cfg, W, doc, prompt


def _decode(cfg, W, prompt, doc, **kw):
    kv = KVCache.empty(1, cfg.n_kv_heads, 1200, cfg.head_dim)
    return CP.program_decode(cfg, W, kv, prompt, doc, T, **kw)


@pytest.mark.parametrize("unit,max_ops,max_gen", [("lines", 6, 12), ("tokens", 5, 10), ("lines", 3, 40)])
def test_decoder_stream_is_a_program_and_drafts_are_lossless(tiny, unit, max_ops, max_gen):
    cfg, W, doc, prompt = tiny
    s0, ops0, out0, st0 = _decode(cfg, W, prompt, doc, unit=unit, max_ops=max_ops, max_gen=max_gen)
    U = len(doc) if unit == "lines" else sum(map(len, doc))
    parse(s0, U, doc, unit)
    for k in (1, 3, 6):
        s1, ops1, out1, st1 = _decode(cfg, W, prompt, doc, unit=unit, max_ops=max_ops, max_gen=max_gen, draft_k=k)
        assert (s1, ops1, out1) == (s0, ops0, out0)
        assert st1["forwards"] <= st0["forwards"] + st1["drafts"]
    # resolution: copies expand to the document, gen bodies stay as generated
    expect = []
    for op in ops0:
        expect += CP.span_units(doc, op["a"], op["b"], unit) if op["op"] == "copy" else op["body"]
    assert out0 == expect


def test_every_decision_is_the_masked_argmax_of_the_sequential_stream(tiny):
    """Feed prompt + stream one token at a time, replaying the automaton on
    the stream: wherever the automaton takes a decision, the decoder's choice
    is the masked argmax after that prefix (splices are sequential steps)."""
    cfg, W, doc, prompt = tiny
    stream, ops, out, st = _decode(cfg, W, prompt, doc, unit="lines", max_ops=4, max_gen=8)
    assert st["copies"] + sum(1 for o in ops if o["op"] == "gen") == len(ops)
    kv = KVCache.empty(1, cfg.n_kv_heads, 1200, cfg.head_dim)
    lg = oracle.decoder.splice(cfg, W, kv, 0, prompt)[-1:]
    f = CP.Fsm(T, len(doc), 4, 8)
    pending = []           # forced ids still to be fed, not decisions
    for j, tok in enumerate(stream):
        if not pending:
            assert tok == int(oracle.masked_argmax(lg, f.mask(cfg.vocab))[0]), j
            feed = f.choose(tok)
            if feed is None:
                op = f.ops[-1]
                feed = [T.quote, T.slash_gt] + CP.span_units(doc, op["a"], op["b"], "lines")
            pending = list(feed[1:])
        else:
            assert tok == pending.pop(0)
        lg = oracle.decoder.decode_step(cfg, W, kv, len(prompt) + j, tok)[None]
    assert f.state == CP.DONE and not pending
