"""GPU parity at a long cache (L = 65573: 65536 keys and a ragged tail of
37) against the float64 CPU oracle, for both head sizes:

* the 1B shape cut to two layers (head_dim 64, 32 query heads over 8 KV
  heads);
* two layers of one GPU's share of the 7B shape at 8-way tensor
  parallelism (head_dim 128, 4 query heads over 1 KV head).

A one-token step takes the short-span attention kernel, a 64-row span the
LDS-staged one; the launcher splits the key axis into 32 partitions per KV
head for the 1B shape and 256 for the single KV head of the share (merged
by the many-partition merge kernel), and both read the cache through a
shuffled block table of ~4100 blocks.

Bars: logits max|diff| <= 2e-2 (bf16 models); appended K/V within the same
bound; argmax bit-exact where the oracle's top-2 margin exceeds 0.1.
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
L_LONG = 65536 + 37
SHAPES = {
    "1b-2layer": synth.LLAMA_1B.replace(name="llama-1b-2layer", n_layers=2),
    "tp8-share-2layer": synth.LLAMA_7B_TP8.replace(name="tp8-share-2layer", n_layers=2),
}


@pytest.fixture(scope="module", params=sorted(SHAPES))
def long_model(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    shape = SHAPES[request.param]
    Wc = synth.make_weights(shape, seed=synth.SEED_WEIGHTS, device="cpu")
    W = {k: (v.cuda() if torch.is_tensor(v) else [{n: t.cuda() for n, t in lw.items()} for lw in v])
         for k, v in Wc.items()}
    kl, vl = synth.random_kv_logical(shape, L_LONG, seed=8, device="cpu")
    return shape, W, synth.weights_to_numpy(Wc), kl, vl


@pytest.mark.parametrize("N", [1, 64])
def test_long_cache(long_model, N):
    shape, W, Wn, kl, vl = long_model
    cfg = Config.of(shape)
    L = L_LONG
    print(f"shape={shape.name} L={L} N={N}", flush=True)
    span = synth.pick_span(synth.make_line_prompt(4096, shape.vocab, seed=12), N)
    nb = (L + N + BLK - 1) // BLK + 1
    kv = cad.KVCache.alloc(shape, nb, synth.shuffled_block_table(nb, nb, seed=N), device="cuda")
    H.write_prefix(kv, kl.cuda(), vl.cuda())
    model = cad.cad_model_create(shape, W, max_tokens=N)
    o = H.outputs(N, shape.vocab)
    cad.cad_splice_forward(model, kv, L, H.tensors_i32(span), None, cad.CAD_VERIFY, o["argmax"], o["accepted"],
                           o["logits"], o["status"])
    okv = KVCache.from_prefix(kl.double().numpy(), vl.double().numpy(), L + N)
    ref = oracle.splice(cfg, Wn, okv, L, span)
    torch.cuda.synchronize()
    cad.cad_model_destroy(model)
    assert int(o["status"][0]) == 0
    err = float(np.max(np.abs(o["logits"].cpu().numpy() - ref)))
    print(f"  logits max|diff| = {err:.3e}", flush=True)
    assert err <= TOL
    sure = oracle.top2_margin(ref, None) > MARGIN
    assert sure.any()
    assert np.array_equal(o["argmax"].cpu().numpy()[sure], oracle.masked_argmax(ref, None)[sure])
    gk, gv = H.read_span(kv, L, N)
    ok_k, ek = H.kv_close(gk, np.stack([okv.k[c][:, L:L + N] for c in range(cfg.n_layers)]), TOL)
    ok_v, ev = H.kv_close(gv, np.stack([okv.v[c][:, L:L + N] for c in range(cfg.n_layers)]), TOL)
    print(f"  kv max|diff| = {ek:.3e} / {ev:.3e}", flush=True)
    assert ok_k and ok_v
