"""GPU parity of CopyLoop's concurrent pipeline on a looped decoder (CopyLoop
§2 "Concurrent Pipeline", "Shallow Screening", "Full-Depth Verification";
§A.1 "Decoding algorithm") against the float64 oracle.

* ``cad_loop_step`` (one tick: groups of positions at different depths, each
  on its own depth's cache, with their residual streams carried in a state
  buffer): a block taken through three ticks, then joined by a younger block
  at depth 0 and a third at depth 0 a tick later, with readouts along the
  way; the states, the readout logits and decisions and the K/V written at
  every depth are compared with ``oracle.loop_step``.  Two groups at the
  same positions through block-table rows 0 and 1 each match the oracle on
  a cache of their own, and each row's blocks hold only their group's K/V.  The fp32 tiny block
  (1e-4 bar) and the bf16 looped shape (d 2048, 16 x 128 heads, FFN 5632, depth
  8; logits 2e-2, K/V 2e-2 plus half a bfloat16 spacing, argmax where the
  oracle's top-2 margin exceeds 0.1).
* ``cad_loop_decode`` (the native scheduler): on the fp32 tiny block applied
  four times, with its block weights scaled by 0.3 so that shallow and
  full-depth predictions agree on most positions but not all, and a prompt
  holding the model's own greedy continuation read out at the screening
  depth (copies survive screening and are refused at full depth): the
  committed tokens and every pipeline counter (ticks, rows, blocks,
  proposals, screened, refused and discarded rows) equal the oracle's
  pipeline, whose tokens equal greedy full-depth decoding; every decision
  the oracle takes has a top-2 margin above 1e-3 (asserted, so the GPU must
  take the same ones).  On the bf16 looped shape (random-init, repeated-line
  prompt of 256 tokens): the committed tokens equal the oracle's greedy
  full-depth decoding, every one of whose decisions has a margin above 0.1
  (asserted).
* ``cad_loop_decode`` with second-readout branching (CopyLoop §A.2): on the
  fp32 tiny block applied 4 or 6 times, weights scaled by 0.3, 0.5 and 1.0,
  seeded uniform prompts of 40 ids chosen so that forks are made, kept and
  lost (one case), one of them without context copies (K = 0), and every
  decision the oracle takes has a margin above 1e-3: the committed tokens and every counter, fork counters included,
  equal ``oracle.copyloop_branch_decode``'s, and the cache the decoder
  leaves holds a clean forward's K/V for every fed committed position at
  every depth (1e-4), the second line's states copied back where it was
  kept.  The bf16 looped shape with branching commits greedy full-depth
  decoding's tokens.  Bad branching arguments are refused on the host.
* The regime the method is built for, at the looped shape: the block scaled
  by 0.03 (shallow readouts agree with full depth) on a prompt ending in the
  model's own continuation; with and without branching the pipeline commits
  device full-depth greedy decoding's tokens, most of them from accepted
  copies, in fewer ticks than tokens.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.copyloop as CL
from oracle.decoder import Config, KVCache
import synth

pytestmark = pytest.mark.gpu

cad = pytest.importorskip("verify_forward_amd")
import gpu_helpers as H  # noqa: E402

BLK = cad.CAD_KV_BLOCK


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return "cuda"


def _tiny_loop(scale, D=4):
    shape = synth.TINY.replace(name="tiny-loop4", loop_depth=D)
    Wt = synth.make_weights(shape, seed=3)
    for k in ("w_qkv", "w_o", "w_gate_up", "w_down"):
        Wt["layers"][0][k].mul_(scale)
    return shape, Wt, synth.weights_to_numpy(Wt)


def _to(W, dev):
    return {k: (v.to(dev) if torch.is_tensor(v) else [{kk: vv.to(dev) for kk, vv in lw.items()} for lw in v])
            for k, v in W.items()}


def _f64(W):
    conv = lambda t: np.asarray(t, dtype=np.float64)
    return {"tok_embed": conv(W["tok_embed"]), "final_norm": conv(W["final_norm"]), "lm_head": conv(W["lm_head"]),
            "layers": [{k: conv(v) for k, v in lw.items()} for lw in W["layers"]]}


# ---------------------------------------------------------------------------
# one tick
# ---------------------------------------------------------------------------

# (ticks) each a list of groups (pos offset from L, rows, depth, state row, readout)
TICKS = [
    [(0, 3, 0, 0, 0)],
    [(0, 3, 1, 0, 0)],
    [(0, 3, 2, 0, 1), (3, 2, 0, 4, 1)],
    [(0, 3, 3, 0, 1), (3, 2, 1, 4, 0), (5, 1, 0, 8, 1)],
]
TOKENS = {0: [7, 900, 31], 3: [15, 15], 5: [600]}


def _run_ticks(shape, Wd, W64, kl, vl, L, tol, margin, dev, mask=None):
    cfg = Config.of(shape)
    D = shape.loop_depth
    nb = (L + 16 + BLK - 1) // BLK
    kv = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
    H.write_prefix(kv, kl, vl)
    okv = KVCache.from_prefix(kl.double().cpu().numpy(), vl.double().cpu().numpy(), L + 16)
    model = cad.cad_model_create(shape, Wd, max_tokens=16)
    state = torch.zeros((12, shape.d_model), dtype=torch.float32, device=dev)
    ostate = np.zeros((12, shape.d_model))
    worst = 0.0
    for t, tick in enumerate(TICKS):
        groups = [(L + p, r, d, st, ro) for p, r, d, st, ro in tick]
        toks = [x for p, r, d, st, ro in tick for x in TOKENS[p]]
        n = len(toks)
        am = torch.full((n,), -9, dtype=torch.int32, device=dev)
        acc = torch.full((len(groups),), -9, dtype=torch.int32, device=dev)
        lg = torch.zeros((n, shape.vocab), dtype=torch.float32, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        cad.cad_loop_step(model, kv, groups, H.tensors_i32(toks), state, None, am, acc, lg, status)
        ref = oracle.loop_step(cfg, W64, okv, [dict(pos=g[0], rows=g[1], depth=g[2], state=g[3], readout=g[4])
                                               for g in groups], toks, ostate)
        torch.cuda.synchronize()
        assert int(status[0]) == 0
        lg, am, acc = lg.cpu().numpy(), am.cpu().numpy(), acc.cpu().numpy()
        r0 = 0
        for gi, (p, r, d, st, ro) in enumerate(tick):
            if ro:
                err = float(np.max(np.abs(lg[r0:r0 + r] - ref[gi])))
                worst = max(worst, err)
                assert err <= tol, (t, gi, err)
                sure = oracle.top2_margin(ref[gi], None) > margin
                a_ref = oracle.masked_argmax(ref[gi], None)
                assert np.array_equal(am[r0:r0 + r][sure], a_ref[sure])
                # the group's acceptance follows its argmax on the device
                # (equal to the oracle's wherever the examined rows are graded)
                assert acc[gi] == oracle.acceptance(am[r0:r0 + r], TOKENS[p], oracle.decision.VERIFY)
            r0 += r
    st_err = float(np.max(np.abs(state.cpu().numpy()[[0, 1, 2, 4, 5, 8]] - ostate[[0, 1, 2, 4, 5, 8]])))
    gk, gv = H.read_span(kv, L, 6)
    print(f"{shape.name}: tick logits max|diff| {worst:.3e}, state max|diff| {st_err:.3e}", flush=True)
    # depths 0..3 of the oldest block's rows (L .. L+2) were all written; the
    # younger blocks' rows only at the depths they reached
    for c, rows in ((0, 6), (1, 5), (2, 3), (3, 3)):
        g = gk[c, :, :rows]
        o = okv.k[c][:, L:L + rows]
        if shape.dtype == "bf16":
            assert H.kv_close(g, o, tol)[0], c
            assert H.kv_close(gv[c, :, :rows], okv.v[c][:, L:L + rows], tol)[0], c
        else:
            assert np.max(np.abs(g - o)) <= tol and np.max(np.abs(gv[c, :, :rows] - okv.v[c][:, L:L + rows])) <= tol
    assert st_err <= (tol if shape.dtype == "f32" else 5e-2)
    cad.cad_model_destroy(model)


def test_loop_step_mixed_depths_fp32():
    dev = _dev()
    shape, Wt, Wn = _tiny_loop(0.3)
    L = 40
    kl, vl = synth.random_kv_logical(shape, L, seed=71, device=dev)
    _run_ticks(shape, _to(Wt, dev), _f64(Wn), kl, vl, L, 1e-4, 1e-3, dev)


def test_loop_step_mixed_depths_looped_bf16():
    dev = _dev()
    shape = synth.LOOPED
    W = synth.make_weights(shape, device=dev)
    W64 = {"tok_embed": W["tok_embed"].double().cpu().numpy(), "final_norm": W["final_norm"].double().cpu().numpy(),
           "lm_head": W["lm_head"].double().cpu().numpy(),
           "layers": [{k: v.double().cpu().numpy() for k, v in lw.items()} for lw in W["layers"]]}
    L = 1000
    kl, vl = synth.random_kv_logical(shape, L, seed=72, device=dev)
    _run_ticks(shape, W, W64, kl, vl, L, 2e-2, 0.1, dev)


def test_loop_step_mixed_depths_edge_width_bf16():
    """The same ticks at widths that leave partial tiles and odd k-step
    counts in every projection (d_model 1088, 17 query heads of 64 over one
    KV head, FFN 2112), one block applied 4 times."""
    dev = _dev()
    shape = synth.Shape("edge-loop4", 1, 1088, 17, 1, 64, 2112, 4096, loop_depth=4)
    Wc = synth.make_weights(shape, device="cpu")
    L = 300
    kl, vl = synth.random_kv_logical(shape, L, seed=73, device="cpu")
    _run_ticks(shape, _to(Wc, dev), _f64({k: (v.double().numpy() if torch.is_tensor(v) else
                                                [{n: t.double().numpy() for n, t in lw.items()} for lw in v])
                                            for k, v in Wc.items()}),
               kl.to(dev), vl.to(dev), L, 2e-2, 0.1, dev)


def test_loop_step_table_rows_keep_lines_apart():
    """Two groups at the same positions and depth in one tick, the first
    through block-table row 0, the second through row 1 (disjoint blocks
    holding the same prefix): each group's readout equals the oracle's tick
    on a cache of its own, and each row's blocks end up with exactly its own
    group's K/V (a group written through the wrong row would mix them)."""
    dev = _dev()
    shape, Wt, Wn = _tiny_loop(0.3)
    cfg = Config.of(shape)
    W64 = _f64(Wn)
    L = 40
    nb = (L + 16 + BLK - 1) // BLK
    table = torch.zeros((2, nb), dtype=torch.int32)
    table[0] = torch.arange(nb, dtype=torch.int32)
    table[1] = torch.arange(nb, 2 * nb, dtype=torch.int32).flip(0)   # other blocks, in another order
    kv = cad.KVCache.alloc(shape, 2 * nb, table, device=dev)
    kl, vl = synth.random_kv_logical(shape, L, seed=71, device=dev)
    H.write_prefix(kv, kl, vl, seq=0)
    H.write_prefix(kv, kl, vl, seq=1)
    model = cad.cad_model_create(shape, _to(Wt, dev), max_tokens=16)
    toks = [[7, 900, 31], [15, 15]]
    groups = [(L, 3, 0, 0, 1, 0), (L, 2, 0, 4, 1, 1)]
    flat = toks[0] + toks[1]
    state = torch.zeros((8, shape.d_model), dtype=torch.float32, device=dev)
    am = torch.full((5,), -9, dtype=torch.int32, device=dev)
    acc = torch.full((2,), -9, dtype=torch.int32, device=dev)
    lg = torch.zeros((5, shape.vocab), dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    cad.cad_loop_step(model, kv, groups, H.tensors_i32(flat), state, None, am, acc, lg, status)
    torch.cuda.synchronize()
    assert int(status[0]) == 0
    lg = lg.cpu().numpy()
    kl64, vl64 = kl.double().cpu().numpy(), vl.double().cpu().numpy()
    r0 = 0
    for gi, (t, g) in enumerate(zip(toks, groups)):
        okv = KVCache.from_prefix(kl64, vl64, L + 16)
        ref = oracle.loop_step(cfg, W64, okv, [dict(pos=g[0], rows=g[1], depth=0, state=0, readout=1)], t,
                               np.zeros((4, shape.d_model)))[0]
        n = g[1]
        assert float(np.max(np.abs(lg[r0:r0 + n] - ref))) <= 1e-4, gi
        gk, gv = H.read_span(kv, L, n, seq=gi)
        assert float(np.max(np.abs(gk[0] - okv.k[0][:, L:L + n]))) <= 1e-4, gi
        assert float(np.max(np.abs(gv[0] - okv.v[0][:, L:L + n]))) <= 1e-4, gi
        r0 += n
    cad.cad_model_destroy(model)


# ---------------------------------------------------------------------------
# the native scheduler
# ---------------------------------------------------------------------------

def _shallow_continuation(cfg, W, seed, n, depth):
    kv = KVCache.empty(cfg.loop_depth, cfg.n_kv_heads, len(seed) + n + 1, cfg.head_dim)
    x = oracle.decoder.splice_hidden(cfg, W, kv, 0, seed)
    out = [int(np.argmax(oracle.final_logits(cfg, W, x[-1:])[0]))]
    while len(out) < n:
        lg = oracle.decoder.decode_step(cfg, W, kv, len(seed) + len(out) - 1, out[-1], depth=depth)
        out.append(int(np.argmax(lg)))
    return out


@pytest.mark.parametrize("seed_id,ds", [(18, 2), (16, 3), (29, 1)])
def test_loop_decode_matches_oracle_pipeline_fp32(seed_id, ds, monkeypatch):
    dev = _dev()
    shape, Wt, Wn = _tiny_loop(0.3)
    cfg = Config.of(shape)
    W64 = _f64(Wn)
    r = np.random.default_rng(seed_id)
    seed = [int(t) for t in r.integers(0, cfg.vocab, size=24)]
    prompt = seed + _shallow_continuation(cfg, W64, seed, 40, ds)
    n, K = 30, 6
    margins = []
    real = CL.masked_argmax

    def recording(lg, mask):
        margins.extend(oracle.top2_margin(lg, mask))
        return real(lg, mask)
    monkeypatch.setattr(CL, "masked_argmax", recording)
    cap = len(prompt) + n + shape.loop_depth * (K + 1) + 1
    want, st_ref = oracle.copyloop_decode(cfg, W64, KVCache.empty(4, 4, cap, 64), prompt, n, ds, K, 64)
    monkeypatch.undo()
    assert min(margins) > 1e-3
    assert want == oracle.greedy_decode(cfg, W64, KVCache.empty(4, 4, cap, 64), prompt, n)
    nb = (cap + BLK - 1) // BLK
    kv = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
    model = cad.cad_model_create(shape, _to(Wt, dev), max_tokens=64)
    loop = cad.cad_loop_create(model, cap, ds, K, 64)
    got, st = cad.cad_loop_decode(loop, kv, prompt, n)
    print(f"fp32 seed {seed_id} ds {ds}: {st}", flush=True)
    assert got == want
    assert st["dev_status"] == 0
    for k in ("ticks", "rows_run", "blocks", "proposed", "screened_out", "rejected", "discarded", "committed"):
        assert st[k] == st_ref[k], (k, st[k], st_ref[k])
    cad.cad_loop_destroy(loop)
    cad.cad_model_destroy(model)


_bf16_ref = {}


@pytest.mark.parametrize("d2", [0, 5])
def test_loop_decode_looped_bf16_equals_greedy_full_depth(d2):
    dev = _dev()
    shape = synth.LOOPED
    cfg = Config.of(shape)
    Wt = synth.make_weights(shape, seed=0)          # on the host, so the oracle's run is reproducible
    W64 = _f64(synth.weights_to_numpy(Wt))
    prompt = [int(t) for t in synth.make_line_prompt(256, shape.vocab, seed=5, line_len_range=(8, 16)).tokens]
    n, K, ds = 16, 8, 2
    cap = len(prompt) + n + shape.loop_depth * (K + 1) + 1
    if "want" not in _bf16_ref:
        okv = KVCache.empty(shape.loop_depth, shape.n_kv_heads, cap, shape.head_dim)
        x = oracle.decoder.splice_hidden(cfg, W64, okv, 0, prompt)
        lg = oracle.final_logits(cfg, W64, x[-1:])
        want, margins = [int(np.argmax(lg[0]))], [float(oracle.top2_margin(lg, None)[0])]
        while len(want) < n:
            lg = oracle.decoder.decode_step(cfg, W64, okv, len(prompt) + len(want) - 1, want[-1])[None]
            margins.append(float(oracle.top2_margin(lg, None)[0]))
            want.append(int(np.argmax(lg[0])))
        _bf16_ref.update(want=want, margin=min(margins))
    want = _bf16_ref["want"]
    assert _bf16_ref["margin"] > 0.1
    if d2:
        kv, nb = _branch_kv(shape, cap, K, dev)
    else:
        nb = (cap + BLK - 1) // BLK
        kv = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
    model = cad.cad_model_create(shape, _to(Wt, dev), max_tokens=512)
    loop = cad.cad_loop_create(model, cap, ds, K, 64, branch_depth=d2)
    got, st = cad.cad_loop_decode(loop, kv, prompt, n)
    print(f"looped bf16 d2={d2}: {st}; tokens {got}", flush=True)
    assert got == want
    assert st["dev_status"] == 0 and st["committed"] >= n
    cad.cad_loop_destroy(loop)
    cad.cad_model_destroy(model)


_edge_ref = {}


@pytest.mark.parametrize("d2", [0, 3])
def test_loop_decode_edge_width_bf16_equals_greedy_full_depth(d2):
    """CopyLoop decoding (and branching at d2 = 3) of a block at the edge
    widths (d_model 1088, 17 query heads of 64 over one KV head, FFN 2112,
    vocab 4096) applied 4 times, screened at depth 2: the committed tokens
    equal the oracle's full-depth greedy decode, whose every decision has a
    top-2 margin above 0.1 for this prompt (asserted)."""
    dev = _dev()
    shape = synth.Shape("edge-loop4", 1, 1088, 17, 1, 64, 2112, 4096, loop_depth=4)
    cfg = Config.of(shape)
    Wt = synth.make_weights(shape, seed=0)
    W64 = _f64(synth.weights_to_numpy(Wt))
    prompt = [int(t) for t in synth.make_line_prompt(256, shape.vocab, seed=8, line_len_range=(8, 16)).tokens]
    n, K, ds = 16, 8, 2
    cap = len(prompt) + n + shape.loop_depth * (K + 1) + 1
    if "want" not in _edge_ref:
        okv = KVCache.empty(shape.loop_depth, shape.n_kv_heads, cap, shape.head_dim)
        x = oracle.decoder.splice_hidden(cfg, W64, okv, 0, prompt)
        lg = oracle.final_logits(cfg, W64, x[-1:])
        want, margins = [int(np.argmax(lg[0]))], [float(oracle.top2_margin(lg, None)[0])]
        while len(want) < n:
            lg = oracle.decoder.decode_step(cfg, W64, okv, len(prompt) + len(want) - 1, want[-1])[None]
            margins.append(float(oracle.top2_margin(lg, None)[0]))
            want.append(int(np.argmax(lg[0])))
        _edge_ref.update(want=want, margin=min(margins))
    want = _edge_ref["want"]
    assert _edge_ref["margin"] > 0.1
    if d2:
        kv, nb = _branch_kv(shape, cap, K, dev)
    else:
        nb = (cap + BLK - 1) // BLK
        kv = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
    model = cad.cad_model_create(shape, _to(Wt, dev), max_tokens=512)
    loop = cad.cad_loop_create(model, cap, ds, K, 64, branch_depth=d2)
    got, st = cad.cad_loop_decode(loop, kv, prompt, n)
    print(f"edge-width bf16 d2={d2}: {st}; tokens {got}", flush=True)
    assert got == want
    assert st["dev_status"] == 0 and st["committed"] >= n
    cad.cad_loop_destroy(loop)
    cad.cad_model_destroy(model)


# ---------------------------------------------------------------------------
# second-readout branching
# ---------------------------------------------------------------------------

def _branch_kv(shape, cap, K, dev):
    """A pool holding the request's blocks (block-table row 0, in order)
    and the spare blocks the second line maps its positions to (row 1)."""
    nb = (cap + BLK - 1) // BLK
    spare = -(-(shape.loop_depth * (K + 1) + 16) // 16) + 1
    table = torch.zeros((2, max(nb, spare)), dtype=torch.int32)
    table[0, :nb] = torch.arange(nb, dtype=torch.int32)
    table[1, :spare] = torch.arange(nb, nb + spare, dtype=torch.int32)
    return cad.KVCache.alloc(shape, nb + spare, table, device=dev), nb


# name: (block scale, depth D, ds, d2, K, max_rows, prompt seed); the oracle's forks (kept, lost) noted
BRANCH_CASES = {
    "scale0.3": (0.3, 4, 1, 3, 8, 24, 11),    # 5 forks, 5 kept
    "rows6": (0.5, 4, 2, 3, 4, 6, 5),         # 20 forks, 20 kept, at most 6 rows in flight
    "scale1": (1.0, 4, 1, 3, 8, 24, 1),       # 14 forks, 8 kept
    "lost": (1.0, 4, 2, 3, 8, 24, 1),         # 10 forks, 7 kept, 1 lost
    "depth6": (0.3, 6, 2, 4, 8, 24, 11),      # 4 forks, 2 kept
    "no-copies": (0.5, 4, 1, 3, 0, 24, 2),    # K = 0: 19 forks, 12 kept (no proposals anywhere)
    "rows1": (1.0, 4, 1, 3, 8, 1, 3),         # one row in flight: no tails, never room for a second child
}
NO_ROOM = {"rows1"}
COUNTERS = ("ticks", "rows_run", "blocks", "proposed", "screened_out", "rejected", "discarded", "committed",
            "forks", "forks_kept", "forks_lost", "fork_rows_dropped")


@pytest.mark.parametrize("name", list(BRANCH_CASES))
def test_loop_decode_branching_matches_oracle(name, monkeypatch):
    dev = _dev()
    scale, D, ds, d2, K, max_rows, pseed = BRANCH_CASES[name]
    shape, Wt, Wn = _tiny_loop(scale, D)
    cfg = Config.of(shape)
    W64 = _f64(Wn)
    prompt = [int(t) for t in np.random.default_rng(pseed).integers(0, shape.vocab, size=40)]
    n = 24
    margins = []
    real = CL.masked_argmax

    def recording(lg, mask):
        margins.extend(oracle.top2_margin(lg, mask))
        return real(lg, mask)
    monkeypatch.setattr(CL, "masked_argmax", recording)
    cap = len(prompt) + n + D * (K + 1) + 1
    ocap = cap + 2 * D * (K + 1)
    want, st_ref = CL.copyloop_branch_decode(cfg, W64, KVCache.empty(D, 4, ocap, 64), prompt, n, ds, d2, K, max_rows)
    monkeypatch.undo()
    assert min(margins) > 1e-3, min(margins)
    assert (st_ref["forks"] == 0) == (name in NO_ROOM)
    if name == "lost":
        assert st_ref["forks_lost"] > 0 and st_ref["forks_kept"] > 0
    full = oracle.greedy_decode(cfg, W64, KVCache.empty(D, 4, ocap, 64), prompt, st_ref["committed"])
    assert want == full[:n]
    kv, nb = _branch_kv(shape, cap, K, dev)
    model = cad.cad_model_create(shape, _to(Wt, dev), max_tokens=64)
    loop = cad.cad_loop_create(model, cap, ds, K, max_rows, branch_depth=d2)
    print(f"branching {name}: D {D} ds {ds} d2 {d2} K {K} max_rows {max_rows}", flush=True)
    got, st = cad.cad_loop_decode(loop, kv, prompt, n)
    print(f"  {st}", flush=True)
    assert got == want
    assert st["dev_status"] == 0
    for k in COUNTERS:
        assert st[k] == st_ref[k], (k, st[k], st_ref[k])
    # every fed committed position's K/V at every depth, through row 0
    P = len(prompt) + st["committed"] - 1
    ref = KVCache.empty(D, 4, ocap, 64)
    oracle.decoder.splice_hidden(cfg, W64, ref, 0, (prompt + full)[:P])
    gk, gv = H.read_span(kv, 0, P)
    for c in range(D):
        ek = float(np.max(np.abs(gk[c] - ref.k[c][:, :P])))
        ev = float(np.max(np.abs(gv[c] - ref.v[c][:, :P])))
        assert ek <= 1e-4 and ev <= 1e-4, (c, ek, ev)
    cad.cad_loop_destroy(loop)
    cad.cad_model_destroy(model)


def test_loop_branching_arguments_checked():
    dev = _dev()
    shape, Wt, Wn = _tiny_loop(0.3)
    model = cad.cad_model_create(shape, _to(Wt, dev), max_tokens=64)
    for ds, d2 in ((2, 2), (2, 1), (1, 4)):
        with pytest.raises(cad.CadError) as e:
            cad.cad_loop_create(model, 256, ds, 8, 24, branch_depth=d2)
        assert e.value.status == cad.CAD_E_ARG
    loop = cad.cad_loop_create(model, 256, 1, 8, 24, branch_depth=3)
    prompt = list(range(40))
    # a one-row table
    nb = 16
    kv1 = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
    with pytest.raises(cad.CadError):
        cad.cad_loop_decode(loop, kv1, prompt, 8)
    # spare blocks that are also the request's, or outside the pool
    kv, _ = _branch_kv(shape, 256, 8, dev)
    for bad in (3, kv.num_blocks):
        kv.block_table[1, 0] = bad
        with pytest.raises(cad.CadError) as e:
            cad.cad_loop_decode(loop, kv, prompt, 8)
        assert e.value.status == cad.CAD_E_ARG
    cad.cad_loop_destroy(loop)
    cad.cad_model_destroy(model)


def test_loop_decode_agreeing_depths_copies_pay():
    """The looped shape (bf16, d 2048, depth 8) with its block scaled by 0.03
    (each application moves the residual stream little, so the depth-2
    readouts mostly name the depth-8 token) on a prompt of 3840 line tokens
    followed by 256 tokens of the model's own greedy continuation: with and
    without branching the pipeline commits the tokens of device-resident
    full-depth greedy decoding (the looped splice, one token at a time), more
    than half of them copied from the context (accepted tails), in fewer
    ticks than tokens."""
    dev = _dev()
    shape = synth.LOOPED
    D = shape.loop_depth
    W = synth.make_weights(shape, device=dev)
    for k in ("w_qkv", "w_o", "w_gate_up", "w_down"):
        W["layers"][0][k].mul_(0.03)
    L0, n, K, ds = 4096, 64, 8, 2
    lines = [int(t) for t in synth.make_line_prompt(L0, shape.vocab).tokens]
    cap = L0 + n + D * (K + 1) + 16
    kv, nb = _branch_kv(shape, cap, K, dev)
    model = cad.cad_model_create(shape, W, max_tokens=L0)

    def greedy(prompt, count):
        pr = torch.tensor(prompt, dtype=torch.int32, device=dev)
        gen = torch.empty(count, dtype=torch.int32, device=dev)
        sa = torch.empty(len(prompt), dtype=torch.int32, device=dev)
        am = torch.empty(len(prompt), dtype=torch.int32, device=dev)
        one = torch.empty(1, dtype=torch.int32, device=dev)
        sv = torch.empty(1, dtype=torch.int32, device=dev)
        acc = torch.empty(1, dtype=torch.int32, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        L = len(prompt)
        cad.cad_splice_forward_looped(model, kv, 0, pr, D, None, sa, sv, am, acc, None, status)
        gen[0:1].copy_(sa[L - 1:L])
        for i in range(1, count):
            cad.cad_splice_forward_looped(model, kv, L + i - 1, gen[i - 1:i], D, None, gen[i:i + 1], sv, one, acc,
                                          None, status)
        torch.cuda.synchronize()
        assert int(status[0]) == 0
        return [int(t) for t in gen.cpu()]

    prompt = lines[:L0 - 256] + greedy(lines[:L0 - 256], 256)
    want = greedy(prompt, n)
    for d2 in (0, 5):
        loop = cad.cad_loop_create(model, cap, ds, K, 64, branch_depth=d2)
        got, st = cad.cad_loop_decode(loop, kv, prompt, n)
        print(f"agreeing depths d2={d2}: {st}", flush=True)
        assert got == want
        assert st["dev_status"] == 0
        copied = st["proposed"] - st["screened_out"] - st["rejected"]
        assert copied > n // 2, copied
        assert st["ticks"] < n
        cad.cad_loop_destroy(loop)
    cad.cad_model_destroy(model)
