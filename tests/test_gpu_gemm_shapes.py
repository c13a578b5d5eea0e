"""GPU parity at model shapes that put the tiled projections and the LM
head's argmax epilogue on their edges, against the float64 CPU oracle.

"odd-steps": 2 layers, d_model 1088 (17 x 64), 17 query heads of 64 over one
KV head (17 query heads per KV head, so every call takes the LDS-staged
attention), SwiGLU FFN 2112 (33 x 64), vocab 4096.  With these widths the
k loops of the tiled projections run odd step counts (1088 / 64 = 17 steps
on the 128-row tiles; 34 steps of 32 split into two odd halves on the
256-row tiles; the down projection's 66 steps split 16 / 17 / 16 / 17),
the weight tiles end part-way through a tile (1216 QKV rows over 192-row
tiles, 1088 over 256), and the gate/up projection splits K and leaves its
sums to the reduce kernel.  The spans cover the weight-streaming path
(5 and 16 rows), the 128-row activation tiles (17, 40 and 128 rows; QKV,
O and down there on 128-row weight tiles, 1216 and 1088 rows ending
part-way through one) and the 256-row tiles (129 rows, one full activation
tile and one row of the next; 300 rows, the second partial; and 200 rows
on an empty cache, where attention sees only the span's own keys).

"ragged-vocab": 2 layers, d_model 1152, 9 query heads of 128 over 3 KV
heads, FFN 2240, vocab 1001: the LM head's last weight tile holds 9 ids
(the masked argmax candidates of a partial tile, at every path).

"tp8-share": two layers of one GPU's share of the 7B shape at 8-way tensor
parallelism (d_model 4096, one KV head and its 4 query heads of 128, FFN
1792, vocab 4000): attention and O projection 512 wide against a 4096-wide
residual stream.

"big-vocab": a vocabulary of 128256 ids over a 256-wide model: the masked
argmax reduces 501 candidates per row from the tiled LM head (2004 from the
weight-streaming one), and the LM head dominates the call.

"mha64" and "g8-128": the attention group sizes the production shapes do
not use, one query head per KV head at head_dim 64 (the register-fragment
kernel up to 16 rows) and eight at head_dim 128 (that kernel up to 2 rows).

"f32-odd": the fp32 path (64 x 64 VALU tiles, one wave per row and head in
attention) at widths that are not multiples of 64 (d_model 320, FFN 576,
5 query heads over one KV head, vocab 1001), to 1e-4 with decisions
graded at a 1e-3 margin.

In all of them, the mask of row 0 allows only the vocabulary's last six
ids, so its argmax must come from the last weight tile.  The same shapes also run a
batched call (five sequences of 1 to 130 rows over a shuffled pool), and
the odd-steps widths a looped block (applied 3 times, screened at depth 1
or 2).

Bars: logits max|diff| <= 2e-2 (bf16 models); appended K/V within the same
bound; argmax bit-exact where the oracle's masked top-2 margin exceeds 0.1.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.decoder import Config, KVCache
import synth

pytestmark = pytest.mark.gpu

cad = pytest.importorskip("verify_forward_amd")
import gpu_helpers as H  # noqa: E402

TOL = 2e-2
MARGIN = 0.1


def _bars(shape):
    """(logit tolerance, grading margin, K/V check) of a model's precision:
    the bf16 bars above, or 1e-4 / 1e-3 and a plain 1e-4 on K/V for fp32"""
    if shape.dtype == "f32":
        return 1e-4, 1e-3, lambda g, o: (bool(np.max(np.abs(g - o)) <= 1e-4), float(np.max(np.abs(g - o))))
    return TOL, MARGIN, lambda g, o: H.kv_close(g, o, TOL)
BLK = cad.CAD_KV_BLOCK
SHAPES = {
    "odd-steps": synth.Shape("odd-steps", 2, 1088, 17, 1, 64, 2112, 4096),
    "ragged-vocab": synth.Shape("ragged-vocab", 2, 1152, 9, 3, 128, 2240, 1001),
    "tp8-share": synth.LLAMA_7B_TP8.replace(name="tp8-share-2layer", n_layers=2),
    "big-vocab": synth.Shape("big-vocab", 2, 256, 4, 2, 64, 512, 128256),
    "mha64": synth.Shape("mha64", 2, 1024, 16, 16, 64, 2048, 4096),
    "g8-128": synth.Shape("g8-128", 2, 1024, 8, 1, 128, 2048, 4096),
    "f32-odd": synth.Shape("f32-odd", 2, 320, 5, 1, 64, 576, 1001, dtype="f32"),
}


@pytest.fixture(scope="module", params=sorted(SHAPES))
def edge_model(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    shape = SHAPES[request.param]
    # generated on the CPU (the CPU generator fixes the values, and with them
    # which rows clear the margin), then moved to the device
    Wc = synth.make_weights(shape, seed=synth.SEED_WEIGHTS, device="cpu")
    W = {k: (v.cuda() if torch.is_tensor(v) else [{n: t.cuda() for n, t in lw.items()} for lw in v])
         for k, v in Wc.items()}
    return shape, W, synth.weights_to_numpy(Wc)


# 16 / 17 and 128 / 129 rows are where the projections change kernels
# (weight streaming -> 128-row tiles -> 256-row tiles)
@pytest.mark.parametrize("L,N", [(300, 5), (300, 16), (300, 17), (300, 40), (123, 128), (123, 129), (211, 300),
                                 (0, 200)])
def test_edge_shapes(edge_model, L, N):
    SHAPE, W, Wn = edge_model
    cfg = Config.of(SHAPE)
    print(f"shape={SHAPE.name} L={L} N={N}", flush=True)
    kl, vl = synth.random_kv_logical(SHAPE, L, seed=5 + L, device="cpu")
    prompt = synth.make_line_prompt(max(L, 512), SHAPE.vocab, seed=11)
    span = synth.pick_span(prompt, N)
    nb = (L + N + BLK - 1) // BLK + 2
    kv = cad.KVCache.alloc(SHAPE, nb, synth.shuffled_block_table(nb, nb, seed=N), device="cuda")
    H.write_prefix(kv, kl.cuda(), vl.cuda())
    mask = synth.banned_ids_mask(N, SHAPE.vocab, 64, seed=N)
    mask[0] = 0
    for t in range(SHAPE.vocab - 6, SHAPE.vocab):
        mask[0, t // 32] |= np.uint32(1) << np.uint32(t % 32)
    model = cad.cad_model_create(SHAPE, W, max_tokens=N)
    o = H.outputs(N, SHAPE.vocab)
    cad.cad_splice_forward(model, kv, L, H.tensors_i32(span), torch.from_numpy(mask.view(np.int32)).cuda(),
                           cad.CAD_VERIFY, o["argmax"], o["accepted"], o["logits"], o["status"])
    okv = KVCache.from_prefix(kl.double().cpu().numpy(), vl.double().cpu().numpy(), L + N)
    ref = oracle.splice(cfg, Wn, okv, L, span)
    torch.cuda.synchronize()
    cad.cad_model_destroy(model)
    assert int(o["status"][0]) == 0
    tol, margin, kv_ok = _bars(SHAPE)
    err = float(np.max(np.abs(o["logits"].cpu().numpy() - ref)))
    print(f"  logits max|diff| = {err:.3e}", flush=True)
    assert err <= tol
    sure = oracle.top2_margin(ref, mask) > margin
    a_ref = oracle.masked_argmax(ref, mask)
    assert sure.any()
    assert np.array_equal(o["argmax"].cpu().numpy()[sure], a_ref[sure])
    gk, gv = H.read_seq(kv, L + N)
    ok_k, ek = kv_ok(gk[:, :, L:], np.stack([okv.k[c][:, L:] for c in range(cfg.n_layers)]))
    ok_v, ev = kv_ok(gv[:, :, L:], np.stack([okv.v[c][:, L:] for c in range(cfg.n_layers)]))
    print(f"  kv max|diff| = {ek:.3e} / {ev:.3e}", flush=True)
    assert ok_k and ok_v


def test_edge_shapes_batched(edge_model):
    """A batched call at the edge shapes: five sequences over one shuffled
    pool, a one-token step on a one-key cache, copies of 40 and 130 rows, a
    7-row copy and a one-token step on a 300-key cache; every sequence
    against its own oracle splice."""
    SHAPE, W, Wn = edge_model
    cfg = Config.of(SHAPE)
    Ls = [1, 17, 211, 64, 300]
    Ns = [1, 40, 7, 130, 1]
    prompt = synth.make_line_prompt(512, SHAPE.vocab, seed=13)
    spans = [synth.pick_span(prompt, n) for n in Ns]
    offsets = np.concatenate([[0], np.cumsum(Ns)]).astype(np.int32)
    total = int(offsets[-1])
    mask = synth.banned_ids_mask(total, SHAPE.vocab, 64, seed=3)
    need = [(L + n + BLK - 1) // BLK for L, n in zip(Ls, Ns)]
    pool = int(sum(need)) + 3
    perm = synth.shuffled_block_table(pool, pool, seed=21).numpy()
    table = np.full((len(Ls), max(need)), -1, dtype=np.int32)
    used = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[used:used + nb]
        used += nb
    kv = cad.KVCache.alloc(SHAPE, pool, torch.from_numpy(table), device="cuda")
    pre = []
    for b, L in enumerate(Ls):
        kl, vl = synth.random_kv_logical(SHAPE, L, seed=60 + b, device="cpu")
        H.write_prefix(kv, kl.cuda(), vl.cuda(), seq=b)
        pre.append((kl, vl))
    model = cad.cad_model_create(SHAPE, W, max_tokens=total)
    o = H.outputs(total, SHAPE.vocab, n_seq=len(Ls))
    cad.cad_splice_forward_batched(model, kv, Ls, offsets, H.tensors_i32(np.concatenate(spans)),
                                   torch.from_numpy(mask.view(np.int32)).cuda(), cad.CAD_VERIFY,
                                   o["argmax"], o["accepted"], o["logits"], o["status"])
    torch.cuda.synchronize()
    cad.cad_model_destroy(model)
    assert int(o["status"][0]) == 0
    lg, am = o["logits"].cpu().numpy(), o["argmax"].cpu().numpy()
    tol, margin, kv_ok = _bars(SHAPE)
    graded = 0
    for b, (L, n) in enumerate(zip(Ls, Ns)):
        s0, s1 = int(offsets[b]), int(offsets[b + 1])
        kl, vl = pre[b]
        okv = KVCache.from_prefix(kl.double().numpy(), vl.double().numpy(), L + n)
        ref = oracle.splice(cfg, Wn, okv, L, spans[b])
        err = float(np.max(np.abs(lg[s0:s1] - ref)))
        print(f"{SHAPE.name} seq {b}: L={L} N={n} logits max|diff| {err:.3e}", flush=True)
        assert err <= tol
        sure = oracle.top2_margin(ref, mask[s0:s1]) > margin
        graded += int(sure.sum())
        assert np.array_equal(am[s0:s1][sure], oracle.masked_argmax(ref, mask[s0:s1])[sure])
        gk, gv = H.read_seq(kv, L + n, seq=b)
        ok_k, _ = kv_ok(gk[:, :, L:], np.stack([okv.k[c][:, L:] for c in range(cfg.n_layers)]))
        ok_v, _ = kv_ok(gv[:, :, L:], np.stack([okv.v[c][:, L:] for c in range(cfg.n_layers)]))
        assert ok_k and ok_v
    assert graded > 0


def _depth_chain(cfg, Wn, kl, vl, L, head, n, depth):
    """The oracle's greedy chain at readout depth ``depth`` from ``head``."""
    chain = KVCache.from_prefix(kl.double().numpy(), vl.double().numpy(), L + n)
    span = [head]
    for j in range(n - 1):
        lg = oracle.decode_step(cfg, Wn, chain, L + j, span[j], depth=depth)[None]
        span.append(int(oracle.masked_argmax(lg, None)[0]))
    return np.asarray(span, dtype=np.int32)


@pytest.mark.parametrize("N,ds,planted", [(9, 1, False), (40, 2, False), (40, 2, True)])
def test_edge_shape_looped(N, ds, planted):
    """The looped path at the odd-steps widths (one block applied 3 times):
    screening at depth ds, then the survivors at full depth, under a mask
    built from the oracle's own logits so that every decision has a 0.5
    margin; screening argmax, survivors, full-depth logits, argmax and
    acceptance against the oracle.  40 rows put the block on the 128-row
    tiles; the planted span is the oracle's own depth-ds greedy chain, so
    every row survives screening and all 40 go to full depth."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    shape = SHAPES["odd-steps"].replace(name="odd-steps-loop3", n_layers=1, loop_depth=3)
    cfg = Config.of(shape)
    Wc = synth.make_weights(shape, seed=synth.SEED_WEIGHTS, device="cpu")
    W = {k: (v.cuda() if torch.is_tensor(v) else [{n: t.cuda() for n, t in lw.items()} for lw in v])
         for k, v in Wc.items()}
    Wn = synth.weights_to_numpy(Wc)
    L = 300
    kl, vl = synth.random_kv_logical(shape, L, seed=77, device="cpu")
    if planted:
        span = _depth_chain(cfg, Wn, kl, vl, L, 29, N, ds)
    else:
        span = synth.pick_span(synth.make_line_prompt(512, shape.vocab, seed=17), N)
    kl64, vl64 = kl.double().numpy(), vl.double().numpy()
    res0 = oracle.looped_splice(cfg, Wn, KVCache.from_prefix(kl64, vl64, L + N), L, span, ds)
    mask = H.clear_margin_mask(res0["screen_logits"], res0["logits"], 0.5)
    res = oracle.looped_splice(cfg, Wn, KVCache.from_prefix(kl64, vl64, L + N), L, span, ds, mask)
    m = res["survivors"]
    assert m == res0["survivors"]
    if planted:
        assert m == N
    nb = (L + N + BLK - 1) // BLK
    kv = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device="cuda")
    H.write_prefix(kv, kl.cuda(), vl.cuda())
    model = cad.cad_model_create(shape, W, max_tokens=N)
    sa = torch.full((N,), -9, dtype=torch.int32, device="cuda")
    sv = torch.full((1,), -9, dtype=torch.int32, device="cuda")
    o = H.outputs(N, shape.vocab)
    cad.cad_splice_forward_looped(model, kv, L, H.tensors_i32(span), ds,
                                  torch.from_numpy(mask.view(np.int32).copy()).cuda(), sa, sv, o["argmax"],
                                  o["accepted"], o["logits"], o["status"])
    torch.cuda.synchronize()
    cad.cad_model_destroy(model)
    assert int(o["status"][0]) == 0
    err = float(np.max(np.abs(o["logits"].cpu().numpy()[:m] - res["logits"])))
    print(f"looped N={N} ds={ds}: survivors {int(sv[0])} (oracle {m}), full-depth logits of {m} rows "
          f"max|diff| {err:.3e}", flush=True)
    assert np.array_equal(sa.cpu().numpy(), res["screen_argmax"])
    assert int(sv[0]) == m
    assert err <= TOL
    assert np.array_equal(o["argmax"].cpu().numpy(), res["argmax"])
    assert int(o["accepted"][0]) == res["accepted"]
