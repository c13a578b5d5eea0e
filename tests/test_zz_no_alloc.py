"""GPU test of the allocation-free decode step (``cad_decode_step_noalloc``,
the entry point for callers that cannot allocate device memory), called
through the C ABI.

Two calls in a row on the Llama-style 7B shape: the first over a cache of
8000 tokens, the second over 1500 (fewer attention partitions, so the
scratch it shares with the first call holds a larger layout's leftovers).
Each is compared with ``cad_decode_step`` on an identical copy of the cache,
to the bf16 bars of the splice: logits within 2e-2, the appended K/V within
2e-2 plus half a bfloat16 spacing, argmax bit-exact where the reference
logits' masked top-2 margin exceeds 0.1.  (The two entry points run the same
kernels with the same split counts, so in practice they agree bit for bit.)
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

cad = pytest.importorskip("verify_forward_amd")
import gpu_helpers as H  # noqa: E402

TOL = 2e-2
BLK = cad.CAD_KV_BLOCK


def test_decode_step_noalloc_matches_decode_step():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = "cuda"
    shape = synth.LLAMA_7B
    W = synth.make_weights(shape, device=dev)
    model = cad.cad_model_create(shape, W, max_tokens=64)
    words = (shape.vocab + 31) // 32
    for i, L in enumerate((8000, 1500)):
        nb = (L + 1 + BLK - 1) // BLK
        kl, vl = synth.random_kv_logical(shape, L, seed=500 + i, device=dev)
        kv_ref = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
        H.write_prefix(kv_ref, kl, vl)
        kv_na = cad.KVCache(kv_ref.k.clone(), kv_ref.v.clone(), kv_ref.block_table.clone())
        del kl, vl
        token = H.tensors_i32([1234 + 77 * i])
        mask = synth.allowed_fraction_mask(1, shape.vocab, int(0.6 * shape.vocab), which=i)
        mask_t = torch.from_numpy(mask.view(np.int32)).to(dev)
        o_ref, o_na = H.outputs(1, shape.vocab), H.outputs(1, shape.vocab)
        cad.cad_decode_step(model, kv_ref, L, token, mask_t, o_ref["argmax"], o_ref["logits"], o_ref["status"])
        cad.cad_decode_step_noalloc(model, kv_na, L, token, mask_t, o_na["argmax"], o_na["logits"], o_na["status"])
        torch.cuda.synchronize()
        assert int(o_ref["status"][0]) == 0 and int(o_na["status"][0]) == 0
        lr, ln = o_ref["logits"].cpu().numpy(), o_na["logits"].cpu().numpy()
        err = float(np.max(np.abs(lr - ln)))
        kr, vr = H.read_span(kv_ref, L, 1)
        kn, vn = H.read_span(kv_na, L, 1)
        ok_k, ek = H.kv_close(kn, kr, TOL)
        ok_v, ev = H.kv_close(vn, vr, TOL)
        print(f"call {i}: L={L} logits max|diff| {err:.3e} (bit-equal: {np.array_equal(lr, ln)}), "
              f"K {ek:.3e}, V {ev:.3e}, argmax {int(o_ref['argmax'][0])} / {int(o_na['argmax'][0])}", flush=True)
        assert err <= TOL
        assert ok_k and ok_v
        if oracle.top2_margin(lr.astype(np.float64), mask)[0] > 0.1:
            assert int(o_na["argmax"][0]) == int(o_ref["argmax"][0])
        # slots before L are untouched by either call
        assert torch.equal(kv_na.k[:, : L // BLK], kv_ref.k[:, : L // BLK])
        del kv_ref, kv_na
    cad.cad_model_destroy(model)


@pytest.mark.parametrize("shape", [synth.Shape("odd-steps", 2, 1088, 17, 1, 64, 2112, 4096),
                                   synth.Shape("ragged-vocab", 2, 1152, 9, 3, 128, 2240, 1001)],
                         ids=["odd-steps", "ragged-vocab"])
def test_decode_step_noalloc_edge_shapes(shape):
    """The same comparison at widths that leave partial tiles in every
    projection and a ragged vocabulary (after the 7B test in the same
    process, the shared scratch starts with another model's leftovers)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = "cuda"
    W = synth.make_weights(shape, device=dev)
    model = cad.cad_model_create(shape, W, max_tokens=16)
    for i, L in enumerate((900, 37)):
        nb = (L + 1 + BLK - 1) // BLK
        kl, vl = synth.random_kv_logical(shape, L, seed=600 + i, device=dev)
        kv_ref = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
        H.write_prefix(kv_ref, kl, vl)
        kv_na = cad.KVCache(kv_ref.k.clone(), kv_ref.v.clone(), kv_ref.block_table.clone())
        token = H.tensors_i32([(311 + 97 * i) % shape.vocab])
        mask = synth.banned_ids_mask(1, shape.vocab, 64, seed=i)
        mask_t = torch.from_numpy(mask.view(np.int32)).to(dev)
        o_ref, o_na = H.outputs(1, shape.vocab), H.outputs(1, shape.vocab)
        cad.cad_decode_step(model, kv_ref, L, token, mask_t, o_ref["argmax"], o_ref["logits"], o_ref["status"])
        cad.cad_decode_step_noalloc(model, kv_na, L, token, mask_t, o_na["argmax"], o_na["logits"], o_na["status"])
        torch.cuda.synchronize()
        assert int(o_ref["status"][0]) == 0 and int(o_na["status"][0]) == 0
        lr, ln = o_ref["logits"].cpu().numpy(), o_na["logits"].cpu().numpy()
        err = float(np.max(np.abs(lr - ln)))
        kr, vr = H.read_span(kv_ref, L, 1)
        kn, vn = H.read_span(kv_na, L, 1)
        ok_k, _ = H.kv_close(kn, kr, TOL)
        ok_v, _ = H.kv_close(vn, vr, TOL)
        print(f"{shape.name} call {i}: L={L} logits max|diff| {err:.3e} (bit-equal: {np.array_equal(lr, ln)})",
              flush=True)
        assert err <= TOL
        assert ok_k and ok_v
        if oracle.top2_margin(lr.astype(np.float64), mask)[0] > 0.1:
            assert int(o_na["argmax"][0]) == int(o_ref["argmax"][0])
        del kv_ref, kv_na
    cad.cad_model_destroy(model)
