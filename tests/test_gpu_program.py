"""GPU parity of Copy-as-Decode program decoding (``cad_program_decode``:
the grammar automaton, its masks, feeds and stream on the device; §2.1-§2.4,
the appendix's "States.", "Forced prefills." and "Token-sequence end-of-gen
detector."; §5 "Token-level extension." and "Composition with speculative
decoding.") against the float64 oracle ``oracle.cad_program.program_decode``.

The fed stream, the op records, the resolved output and the counters that
do not depend on how many forwards a draft path takes (masked steps,
template feeds, copies, copied ids) must equal the oracle's, for chains of
1, 4 and 64 launched steps, with and without drafts (which must not change
anything but the forward count: the verification is lossless).  Every
decision the oracle takes is replayed on the sequential stream (one
token at a time) and its masked top-2 margin must exceed 2e-4, twice the
fp32 logit bar of the tiny model (asserted), so the GPU path must take the
same ones.

Workloads (seeded, synthetic; the tiny fp32 model):
* random-init weights and a seeded 14-line document of ids 600..999 inside
  the prompt: programs mixing copies and gen bodies that end by the length
  cap, with line and token ranges, and a stream limit that stops inside a
  gen body;
* the block weights scaled by 0.1 (the next id then depends mostly on the
  current one, so generation walks a cycle of the id graph) with "</",
  "gen", ">" set to three consecutive ids of a 23-id cycle and "<" to a
  later one: gen bodies end by the end-of-gen window after 20 ids, repeat
  (drafts are accepted, the window closes inside accepted drafts), and also
  end by the cap; the same model with "<" elsewhere on the cycle gives six
  copies in a row;
* degenerate programs on the same models: at most one op (a copy; a gen
  body that reaches the length cap), gen bodies capped at one id (mixed with
  a copy; six in a row), and a stream limit of three ids.

The bf16 cases run the same shape in bfloat16 (the weights rounded from the
same draws) with the LM head scaled by 32, a power of two and so exact in
bf16: the argmax of every step is unchanged by the scale, and the masked
top-2 margins of the decisions grow with it past 0.1, the decision bar of
the bf16 parity tests (five times their 2e-2 logit bar).  A splice over the
prompt checks that bar on the scaled model first.  The eog-window case
stays fp32-only: in bf16 its id cycle closes the end-of-gen window only
once and some of its decision margins stay below the bar.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import cad_program as CP
from oracle.decoder import Config, KVCache
import synth

pytestmark = pytest.mark.gpu

cad = pytest.importorskip("verify_forward_amd")

BLK = cad.CAD_KV_BLOCK
BASE = dict(lt=27, lt_slash=522, gt=29, copy=856, gen=437, program=149, kw=512, eq_quote=428,
            quote=1, slash_gt=257, hyphen=12, digits=tuple(range(15, 25)))
CYCLE = dict(lt_slash=804, gen=390, gt=699)   # three consecutive ids of a cycle of the 0.1-scaled model


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return "cuda"


def _model(scale, dtype="f32"):
    shape = synth.TINY if dtype == "f32" else synth.TINY.replace(name="tiny-bf16", dtype="bf16")
    Wt = synth.make_weights(shape, seed=5)
    if scale != 1.0:
        for k in ("w_qkv", "w_o", "w_gate_up", "w_down"):
            Wt["layers"][0][k].mul_(scale)
    if dtype == "bf16":
        Wt["lm_head"].mul_(BF16_HEAD_SCALE)
    return shape, Wt, synth.weights_to_numpy(Wt)


def _doc_prompt(table, seed):
    r = np.random.default_rng(seed)
    doc = [[int(x) for x in r.integers(600, 1000, size=int(r.integers(3, 9)))] for _ in range(14)]
    pre = [int(x) for x in r.integers(0, 1000, size=20)] + [x for line in doc for x in line]
    return doc, pre + [table.lt, table.program, table.gt]


def _replay_min_margin(cfg, W, prompt, stream, doc, table, unit, max_ops, max_gen):
    """Feed prompt + stream one id at a time, replaying the automaton: the
    smallest masked top-2 margin over the decisions the stream holds."""
    U = len(doc) if unit == "lines" else sum(map(len, doc))
    kv = KVCache.empty(1, cfg.n_kv_heads, len(prompt) + len(stream) + 8, cfg.head_dim)
    lg = oracle.decoder.splice(cfg, W, kv, 0, prompt)[-1:]
    f = CP.Fsm(table, U, max_ops, max_gen)
    pending, worst = [], np.inf
    for j, tok in enumerate(stream):
        if not pending:
            m = f.mask(cfg.vocab)
            assert tok == int(oracle.masked_argmax(lg, m)[0]), j
            worst = min(worst, float(oracle.top2_margin(lg, m)[0]))
            feed = f.choose(tok)
            if feed is None:
                op = f.ops[-1]
                feed = [table.quote, table.slash_gt] + CP.span_units(doc, op["a"], op["b"], unit)
            pending = list(feed[1:])
        else:
            assert tok == pending.pop(0)
        lg = oracle.decoder.decode_step(cfg, W, kv, len(prompt) + j, tok)[None]
    return worst


# name: (weight scale, table overrides, unit, max_ops, max_gen, max_stream, document/prompt seed); the
# programs they give are noted (g<n>: a gen op with n body ids, c<a>: a copy from unit a)
CASES = {
    "mixed-lines": (1.0, {}, "lines", 6, 12, 512, 39),       # g12 c9 c9 c9 c8 g12
    "mixed-tokens": (1.0, {}, "tokens", 5, 10, 512, 13),     # g10 c77 c72 c72 c30
    "long-gen": (1.0, {}, "lines", 3, 40, 512, 35),          # g40 c9 c9
    "stream-limit": (1.0, {}, "lines", 6, 12, 40, 58),       # c8 c8 c8 g1 (stopped inside the body)
    "eog-window": (0.1, dict(CYCLE, lt=646), "lines", 6, 30, 512, 58),  # g20 g20 g30 g30 g30 g30
    "copies": (0.1, dict(CYCLE, lt=334), "lines", 6, 30, 512, 6),       # c7 x 6
    # degenerate programs: one op allowed, one-id gen bodies, a stream limit inside the first template
    "one-op": (1.0, {}, "lines", 1, 12, 512, 18),                       # c8
    "one-op-gen": (0.1, dict(CYCLE, lt=646), "lines", 1, 30, 512, 18),  # g30 (the length cap)
    "gen1-mixed": (1.0, {}, "lines", 6, 1, 512, 19),                    # g1 g1 g1 g1 c9 g1
    "gen1-cycle": (0.1, dict(CYCLE, lt=646), "lines", 6, 1, 512, 67),   # g1 x 6
    "stream3": (1.0, {}, "lines", 6, 12, 3, 19),                        # three ids: stopped inside a template
}
MARGIN = 2e-4   # twice the fp32 tiny model's logit bar (1e-4 absolute)
BF16_CASES = ["mixed-lines", "mixed-tokens", "long-gen", "copies", "one-op-gen", "gen1-mixed", "stream-limit"]
BF16_HEAD_SCALE = 32.0
BF16_MARGIN = 0.1    # five times the bf16 logit bar (2e-2)
BF16_TOL = 2e-2

_ref_cache = {}


def _reference(name, dtype="f32"):
    if (name, dtype) not in _ref_cache:
        scale, over, unit, max_ops, max_gen, max_stream, seed = CASES[name]
        shape, Wt, W = _model(scale, dtype)
        cfg = Config.of(shape)
        table = CP.Table(**{**BASE, **over})
        doc, prompt = _doc_prompt(table, seed)
        kv = KVCache.empty(1, cfg.n_kv_heads, 2048, cfg.head_dim)
        ref = CP.program_decode(cfg, W, kv, prompt, doc, table, unit=unit, max_ops=max_ops, max_gen=max_gen,
                                max_stream=max_stream)
        margin = _replay_min_margin(cfg, W, prompt, ref[0], doc, table, unit, max_ops, max_gen)
        _ref_cache[name, dtype] = (shape, Wt, W, cfg, table, doc, prompt, ref, margin)
    return _ref_cache[name, dtype]


def _to_dev(Wt, dev):
    return {k: (v.to(dev) if torch.is_tensor(v) else [{kk: vv.to(dev) for kk, vv in lw.items()} for lw in v])
            for k, v in Wt.items()}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("draft_k,chain", [(0, 1), (0, 4), (0, 64), (3, 4), (8, 2)])
def test_program_decode_matches_oracle(name, draft_k, chain):
    _check_program(name, "f32", MARGIN, draft_k, chain)


@pytest.mark.parametrize("name", BF16_CASES)
@pytest.mark.parametrize("draft_k,chain", [(0, 1), (0, 64), (8, 2)])
def test_program_decode_bf16_matches_oracle(name, draft_k, chain):
    """The same comparison on the bfloat16 model (the product's dtype)."""
    dev = _dev()
    shape, Wt, W, cfg, table, doc, prompt, ref, margin = _reference(name, "bf16")
    # the logit bar on this model: a splice over the prompt against the oracle
    nb = (len(prompt) + BLK - 1) // BLK
    kv = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
    model = cad.cad_model_create(shape, _to_dev(Wt, dev), max_tokens=len(prompt))
    o = {"argmax": torch.empty(len(prompt), dtype=torch.int32, device=dev),
         "accepted": torch.empty(1, dtype=torch.int32, device=dev),
         "logits": torch.empty(len(prompt), shape.vocab, dtype=torch.float32, device=dev),
         "status": torch.zeros(1, dtype=torch.int32, device=dev)}
    cad.cad_splice_forward(model, kv, 0, torch.tensor(prompt, dtype=torch.int32, device=dev), None, cad.CAD_COMMIT,
                           o["argmax"], o["accepted"], o["logits"], o["status"])
    lref = oracle.splice(cfg, W, KVCache.empty(1, cfg.n_kv_heads, len(prompt), cfg.head_dim), 0, prompt)
    torch.cuda.synchronize()
    cad.cad_model_destroy(model)
    err = float(np.max(np.abs(o["logits"].cpu().numpy() - lref)))
    print(f"{name} bf16 prompt logits max|diff| {err:.3e} (logit std {lref.std():.2f})", flush=True)
    assert int(o["status"][0]) == 0 and err <= BF16_TOL
    _check_program(name, "bf16", BF16_MARGIN, draft_k, chain)


def _check_program(name, dtype, bar, draft_k, chain):
    dev = _dev()
    shape, Wt, W, cfg, table, doc, prompt, ref, margin = _reference(name, dtype)
    scale, over, unit, max_ops, max_gen, max_stream, seed = CASES[name]
    stream_ref, ops_ref, out_ref, st_ref = ref
    assert margin > bar, margin
    if draft_k:   # the oracle's drafts are lossless too
        kv_o = KVCache.empty(1, cfg.n_kv_heads, 2048, cfg.head_dim)
        alt = CP.program_decode(cfg, W, kv_o, prompt, doc, table, unit=unit, max_ops=max_ops, max_gen=max_gen,
                                max_stream=max_stream, draft_k=draft_k)
        assert alt[:3] == ref[:3]
    max_doc = 128
    cap = len(prompt) + max_stream + 2 * max_doc + 2 * draft_k + chain + 64
    nb = (cap + BLK - 1) // BLK
    kv = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
    model = cad.cad_model_create(shape, _to_dev(Wt, dev), max_tokens=64)
    prog = cad.cad_program_create(model, nb * BLK, table, max_doc=max_doc, max_stream=max_stream, max_ops=max_ops,
                                  max_gen=max_gen, draft_k=draft_k, chain=chain)
    print(f"{name} {dtype} draft_k={draft_k} chain={chain} (oracle margin {margin:.3g})", flush=True)
    got, ops, out, st = cad.cad_program_decode(prog, kv, prompt, doc, unit=unit)
    print(f"  stats {st}", flush=True)
    assert st["fsm_error"] == 0 and st["dev_status"] == 0
    assert got == stream_ref
    assert ops == ops_ref
    assert out == out_ref
    for k in ("masked_steps", "forced_prefills", "copies", "copied_tokens"):
        assert st[k] == st_ref[k], (k, st[k], st_ref[k])
    if draft_k == 0:
        assert st["forwards"] == st_ref["forwards"]
        assert st["drafts"] == 0
    else:
        assert st["forwards"] <= st_ref["forwards"]
    if chain == 1 and draft_k == 0:   # one step launched ahead after each template or copy, no more
        assert st["idle_steps"] <= st["forced_prefills"] + st["copies"]
    cad.cad_program_destroy(prog)
    cad.cad_model_destroy(model)


def test_program_decode_repeated_bodies_use_drafts():
    """Repeated gen bodies (the id cycle) are mostly verified from drafts:
    more than half the stream comes from accepted drafts, and the decode
    takes fewer than half the oracle's one-forward-per-feed count."""
    dev = _dev()
    shape, Wt, W, cfg, table, doc, prompt, ref, margin = _reference("eog-window")
    assert margin > MARGIN
    stream_ref, ops_ref, out_ref, st_ref = ref
    assert sum(1 for o in ops_ref if o["op"] == "gen" and len(o["body"]) < 30) >= 2
    nb = 64
    kv = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
    model = cad.cad_model_create(shape, _to_dev(Wt, dev), max_tokens=64)
    prog = cad.cad_program_create(model, nb * BLK, table, max_doc=128, max_stream=512, max_ops=6, max_gen=30,
                                  draft_k=8, chain=4)
    got, ops, out, st = cad.cad_program_decode(prog, kv, prompt, doc, unit="lines")
    print(f"  stats {st}", flush=True)
    assert (got, ops, out) == (stream_ref, ops_ref, out_ref)
    assert st["draft_accepted"] > st["stream_n"] // 2
    assert st["forwards"] < st_ref["forwards"] // 2
    cad.cad_program_destroy(prog)
    cad.cad_model_destroy(model)
