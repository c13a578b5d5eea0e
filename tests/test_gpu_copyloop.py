"""GPU parity of CopyLoop's concurrent pipeline on a looped decoder (CopyLoop
§2 "Concurrent Pipeline", "Shallow Screening", "Full-Depth Verification";
§A.1 "Decoding algorithm") against the float64 oracle.

* ``cad_loop_step`` (one tick: groups of positions at different depths, each
  on its own depth's cache, with their residual streams carried in a state
  buffer): a block taken through three ticks, then joined by a younger block
  at depth 0 and a third at depth 0 a tick later, with readouts along the
  way; the states, the readout logits and decisions and the K/V written at
  every depth are compared with ``oracle.loop_step``.  The fp32 tiny block
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


def test_loop_decode_looped_bf16_equals_greedy_full_depth():
    dev = _dev()
    shape = synth.LOOPED
    cfg = Config.of(shape)
    Wt = synth.make_weights(shape, seed=0)          # on the host, so the oracle's run is reproducible
    W64 = _f64(synth.weights_to_numpy(Wt))
    prompt = [int(t) for t in synth.make_line_prompt(256, shape.vocab, seed=5, line_len_range=(8, 16)).tokens]
    n, K, ds = 16, 8, 2
    cap = len(prompt) + n + shape.loop_depth * (K + 1) + 1
    okv = KVCache.empty(shape.loop_depth, shape.n_kv_heads, cap, shape.head_dim)
    x = oracle.decoder.splice_hidden(cfg, W64, okv, 0, prompt)
    lg = oracle.final_logits(cfg, W64, x[-1:])
    want, margins = [int(np.argmax(lg[0]))], [float(oracle.top2_margin(lg, None)[0])]
    while len(want) < n:
        lg = oracle.decoder.decode_step(cfg, W64, okv, len(prompt) + len(want) - 1, want[-1])[None]
        margins.append(float(oracle.top2_margin(lg, None)[0]))
        want.append(int(np.argmax(lg[0])))
    assert min(margins) > 0.1
    nb = (cap + BLK - 1) // BLK
    kv = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
    model = cad.cad_model_create(shape, _to(Wt, dev), max_tokens=512)
    loop = cad.cad_loop_create(model, cap, ds, K, 64)
    got, st = cad.cad_loop_decode(loop, kv, prompt, n)
    print(f"looped bf16: {st}; tokens {got}", flush=True)
    assert got == want
    assert st["dev_status"] == 0 and st["committed"] >= n
    cad.cad_loop_destroy(loop)
    cad.cad_model_destroy(model)
