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
(5 rows), the 128-row tiles (40 rows) and the 256-row tiles (300 rows,
two activation tiles, the second partial; and 200 rows on an empty cache,
where attention sees only the span's own keys).

"ragged-vocab": 2 layers, d_model 1152, 9 query heads of 128 over 3 KV
heads, FFN 2240, vocab 1001: the LM head's last weight tile holds 9 ids
(the masked argmax candidates of a partial tile, at every path).

In both, the mask of row 0 allows only the vocabulary's last six ids, so
its argmax must come from the last weight tile.

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
BLK = cad.CAD_KV_BLOCK
SHAPES = {
    "odd-steps": synth.Shape("odd-steps", 2, 1088, 17, 1, 64, 2112, 4096),
    "ragged-vocab": synth.Shape("ragged-vocab", 2, 1152, 9, 3, 128, 2240, 1001),
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


@pytest.mark.parametrize("L,N", [(300, 5), (300, 40), (211, 300), (0, 200)])
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
    err = float(np.max(np.abs(o["logits"].cpu().numpy() - ref)))
    print(f"  logits max|diff| = {err:.3e}", flush=True)
    assert err <= TOL
    sure = oracle.top2_margin(ref, mask) > MARGIN
    a_ref = oracle.masked_argmax(ref, mask)
    assert sure.any()
    assert np.array_equal(o["argmax"].cpu().numpy()[sure], a_ref[sure])
    gk, gv = H.read_seq(kv, L + N)
    ok_k, ek = H.kv_close(gk[:, :, L:], np.stack([okv.k[c][:, L:] for c in range(cfg.n_layers)]), TOL)
    ok_v, ev = H.kv_close(gv[:, :, L:], np.stack([okv.v[c][:, L:] for c in range(cfg.n_layers)]), TOL)
    print(f"  kv max|diff| = {ek:.3e} / {ev:.3e}", flush=True)
    assert ok_k and ok_v
