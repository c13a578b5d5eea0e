"""GPU parity at the full Llama-style 7B shape, in the launch configuration
the benchmark times (32 layers, d_model 4096, 32 query / 8 KV heads of 128,
SwiGLU 14336, vocab 32000, bf16 weights; KV cache of L = 16384 tokens; a copy
span of N = 512 tokens from a duplicated line of the repeated-line prompt;
a per-position mask allowing 60% of the vocabulary; COMMIT mode), plus
splices of N = 128 (the other span length of the 7B configuration, on the
17-128-row projection kernels), N = 16 (the weight-streaming path) and N = 4
(the sliced RMSNorm folded into the projections, and attention with
fragments loaded straight from the paged cache) over the same cache.

The float64 oracle computes every row of both splices, layer by layer, with
each layer's weights widened to float64 once (about a minute of CPU).

A second test runs the batched editing-serve configuration's launch shape
at the 7B size: four sequences with cache lengths up to 8190 in one shuffled
paged pool, one of them splicing a copy of about 48 tokens of whole
duplicated lines and the others one-token steps, COMMIT mode, no mask (as
the serve benchmark calls it), again against the oracle layer by layer.

Bars: logits within 2e-2; appended K/V within 2e-2 plus half a bfloat16
spacing (the cache stores bfloat16); masked argmax bit-exact where the
oracle's top-2 margin exceeds 0.1; acceptance N in COMMIT mode.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.decoder import Config, KVCache, splice_layer, final_logits
import synth

pytestmark = pytest.mark.gpu

cad = pytest.importorskip("verify_forward_amd")
import gpu_helpers as H  # noqa: E402

TOL = 2e-2
MARGIN = 0.1
BLK = cad.CAD_KV_BLOCK


def _rows(kv, first, n):
    """GPU K/V of tokens first..first+n-1 (identity block table, block-aligned
    start), as float64 [layers][Hkv][n][hd]."""
    assert first % BLK == 0 and n % BLK == 0
    b0, nb = first // BLK, n // BLK
    k = kv.k[:, b0:b0 + nb].permute(0, 2, 1, 3, 4).reshape(kv.k.shape[0], kv.k.shape[2], n, -1)
    v = kv.v[:, b0:b0 + nb].permute(0, 2, 1, 4, 3).reshape(kv.v.shape[0], kv.v.shape[2], n, -1)
    return k.to(torch.float64).cpu().numpy(), v.to(torch.float64).cpu().numpy()


def _check_decisions(ref, mask, a_gpu):
    a_ref = oracle.masked_argmax(ref, mask)
    sure = oracle.top2_margin(ref, mask) > MARGIN
    assert np.array_equal(a_gpu[sure], a_ref[sure]), (a_gpu[sure], a_ref[sure])
    return int(sure.sum())


def test_llama7b_bench_configuration():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = "cuda"
    shape = synth.LLAMA_7B
    cfg = Config.of(shape)
    L, N, NM, NS, NT = 16384, 512, 128, 16, 4
    W = synth.make_weights(shape, device=dev)
    k_log, v_log = synth.random_kv_logical(shape, L, device=dev)
    prompt = synth.make_line_prompt(L, shape.vocab)
    span = synth.pick_span(prompt, N)
    span16 = synth.pick_span(prompt, NS, which=1)
    span128 = synth.pick_span(prompt, NM, which=2)
    span4 = synth.pick_span(prompt, NT, which=3)
    n_allowed = int(round(0.6 * shape.vocab))
    mask = synth.allowed_fraction_mask(N, shape.vocab, n_allowed)
    mask16 = synth.allowed_fraction_mask(NS, shape.vocab, n_allowed, which=1)
    mask128 = synth.allowed_fraction_mask(NM, shape.vocab, n_allowed, which=2)
    mask4 = synth.allowed_fraction_mask(NT, shape.vocab, n_allowed, which=3)
    model = cad.cad_model_create(shape, W, max_tokens=N)

    # ---- GPU: the benchmarked splice, and an N = 16 splice on a fresh copy
    nb = (L + N) // BLK
    kv = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
    H.write_prefix(kv, k_log, v_log)
    o = H.outputs(N, shape.vocab)
    cad.cad_splice_forward(model, kv, L, H.tensors_i32(span), torch.from_numpy(mask.view(np.int32)).to(dev),
                           cad.CAD_COMMIT, o["argmax"], o["accepted"], o["logits"], o["status"])
    nb16 = (L + NS) // BLK
    kv16 = cad.KVCache.alloc(shape, nb16, synth.identity_block_table(nb16), device=dev)
    H.write_prefix(kv16, k_log, v_log)
    o16 = H.outputs(NS, shape.vocab)
    cad.cad_splice_forward(model, kv16, L, H.tensors_i32(span16), torch.from_numpy(mask16.view(np.int32)).to(dev),
                           cad.CAD_COMMIT, o16["argmax"], o16["accepted"], o16["logits"], o16["status"])
    nb128 = (L + NM) // BLK
    kv128 = cad.KVCache.alloc(shape, nb128, synth.identity_block_table(nb128), device=dev)
    H.write_prefix(kv128, k_log, v_log)
    o128 = H.outputs(NM, shape.vocab)
    cad.cad_splice_forward(model, kv128, L, H.tensors_i32(span128),
                           torch.from_numpy(mask128.view(np.int32)).to(dev), cad.CAD_COMMIT, o128["argmax"],
                           o128["accepted"], o128["logits"], o128["status"])
    nb4 = (L + NT + BLK - 1) // BLK
    kv4 = cad.KVCache.alloc(shape, nb4, synth.identity_block_table(nb4), device=dev)
    H.write_prefix(kv4, k_log, v_log)
    o4 = H.outputs(NT, shape.vocab)
    cad.cad_splice_forward(model, kv4, L, H.tensors_i32(span4), torch.from_numpy(mask4.view(np.int32)).to(dev),
                           cad.CAD_COMMIT, o4["argmax"], o4["accepted"], o4["logits"], o4["status"])
    torch.cuda.synchronize()
    assert int(o["status"][0]) == 0 and int(o16["status"][0]) == 0 and int(o128["status"][0]) == 0
    assert int(o4["status"][0]) == 0 and int(o4["accepted"][0]) == NT
    assert int(o["accepted"][0]) == N and int(o16["accepted"][0]) == NS and int(o128["accepted"][0]) == NM
    gk, gv = _rows(kv, L, N)          # appended K/V of all 512 rows
    gk16, gv16 = _rows(kv16, L, NS)
    gk128, gv128 = _rows(kv128, L, NM)
    lg = o["logits"].cpu().numpy()
    lg16 = o16["logits"].cpu().numpy()
    lg128 = o128["logits"].cpu().numpy()
    lg4 = o4["logits"].cpu().numpy()
    # the four appended rows sit in slots 0..3 of block L / 16 (identity table)
    gk4 = kv4.k[:, L // BLK, :, :NT, :].to(torch.float64).cpu().numpy()
    gv4 = kv4.v[:, L // BLK, :, :, :NT].transpose(2, 3).to(torch.float64).cpu().numpy()

    # ---- oracle, layer by layer: pass A (all N rows), pass B (N = 128), pass C (N = 16)
    emb = W["tok_embed"]
    xa = emb[torch.as_tensor(span, device=dev).long()].double().cpu().numpy()
    xc = emb[torch.as_tensor(span16, device=dev).long()].double().cpu().numpy()
    xb = emb[torch.as_tensor(span128, device=dev).long()].double().cpu().numpy()
    xd = emb[torch.as_tensor(span4, device=dev).long()].double().cpu().numpy()
    ka, va, kc, vc, kb, vb, kd, vd = [], [], [], [], [], [], [], []
    hd, hkv = shape.head_dim, shape.n_kv_heads
    for ci in range(shape.n_layers):
        lw = {k: t.double().cpu().numpy() for k, t in W["layers"][ci].items()}
        kp = k_log[ci].double().cpu().numpy()
        vp = v_log[ci].double().cpu().numpy()
        zn, z16, z128 = np.zeros((hkv, N, hd)), np.zeros((hkv, NS, hd)), np.zeros((hkv, NM, hd))
        cache_a = KVCache([np.concatenate([kp, zn], axis=1)], [np.concatenate([vp, zn], axis=1)])
        xa = splice_layer(cfg, lw, cache_a, 0, xa, L)
        ka.append(cache_a.k[0][:, L:]); va.append(cache_a.v[0][:, L:])
        cache_c = KVCache([np.concatenate([kp, z16], axis=1)], [np.concatenate([vp, z16], axis=1)])
        xc = splice_layer(cfg, lw, cache_c, 0, xc, L)
        kc.append(cache_c.k[0][:, L:]); vc.append(cache_c.v[0][:, L:])
        cache_b = KVCache([np.concatenate([kp, z128], axis=1)], [np.concatenate([vp, z128], axis=1)])
        xb = splice_layer(cfg, lw, cache_b, 0, xb, L)
        kb.append(cache_b.k[0][:, L:]); vb.append(cache_b.v[0][:, L:])
        z4 = np.zeros((hkv, NT, hd))
        cache_d = KVCache([np.concatenate([kp, z4], axis=1)], [np.concatenate([vp, z4], axis=1)])
        xd = splice_layer(cfg, lw, cache_d, 0, xd, L)
        kd.append(cache_d.k[0][:, L:]); vd.append(cache_d.v[0][:, L:])
        del lw, kp, vp, cache_a, cache_b, cache_c, cache_d
    top = {"final_norm": W["final_norm"].double().cpu().numpy(), "lm_head": W["lm_head"].double().cpu().numpy()}
    ref_a, ref_b, ref_c = final_logits(cfg, top, xa), final_logits(cfg, top, xb), final_logits(cfg, top, xc)
    ref_d = final_logits(cfg, top, xd)

    errs = {"N=512": np.max(np.abs(lg - ref_a)), "N=128": np.max(np.abs(lg128 - ref_b)),
            "N=16": np.max(np.abs(lg16 - ref_c)), "N=4": np.max(np.abs(lg4 - ref_d))}
    kv_checks = {"kv N=512": [(gk, np.stack(ka)), (gv, np.stack(va))],
                 "kv N=128": [(gk128, np.stack(kb)), (gv128, np.stack(vb))],
                 "kv N=16": [(gk16, np.stack(kc)), (gv16, np.stack(vc))],
                 "kv N=4": [(gk4, np.stack(kd)), (gv4, np.stack(vd))]}
    kv_ok = {}
    for k, pairs in kv_checks.items():
        res = [H.kv_close(g, r, TOL) for g, r in pairs]
        kv_ok[k] = all(ok for ok, _ in res)
        errs[k] = max(e for _, e in res)
    print("7B max|diff|: " + ", ".join(f"{k} {v:.3e}" for k, v in errs.items()), flush=True)
    for k in ("N=512", "N=128", "N=16", "N=4"):
        assert errs[k] <= TOL, (k, errs[k])
    for k, ok in kv_ok.items():
        assert ok, (k, errs[k])
    graded = _check_decisions(ref_a, mask, o["argmax"].cpu().numpy())
    graded += _check_decisions(ref_b, mask128, o128["argmax"].cpu().numpy())
    graded += _check_decisions(ref_c, mask16, o16["argmax"].cpu().numpy())
    graded += _check_decisions(ref_d, mask4, o4["argmax"].cpu().numpy())
    print(f"7B argmax bit-exact on {graded}/{N + NM + NS + NT} graded rows", flush=True)


def test_llama7b_batched_serve_shape():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = "cuda"
    shape = synth.LLAMA_7B
    cfg = Config.of(shape)
    W = synth.make_weights(shape, device=dev)
    Ls = [8190, 3001, 4100, 1024]
    n_seq = len(Ls)
    r = synth.rng(41, 7)
    prompt = synth.make_line_prompt(8192, shape.vocab, seed=1200, line_len_range=(8, 16))
    st = int(prompt.dup_starts[5])
    idx = int(np.searchsorted(prompt.line_starts, st))
    end = int(prompt.line_starts[idx + 4])                # four whole lines (about 48 tokens)
    spans = [prompt.tokens[st:end].astype(np.int32)]
    spans += [np.array([int(r.integers(0, shape.vocab))], dtype=np.int32) for _ in range(n_seq - 1)]
    offsets = np.concatenate([[0], np.cumsum([len(x) for x in spans])]).astype(np.int32)
    total = int(offsets[-1])
    need = [(Ls[b] + len(spans[b]) + BLK - 1) // BLK for b in range(n_seq)]
    pool = int(sum(need)) + 3
    perm = synth.shuffled_block_table(pool, pool, seed=8).numpy()
    table = np.full((n_seq, max(need)), -1, dtype=np.int32)
    used = 0
    for b in range(n_seq):
        table[b, :need[b]] = perm[used:used + need[b]]
        used += need[b]
    kv = cad.KVCache.alloc(shape, pool, torch.from_numpy(table), device=dev)
    pre = []
    for b in range(n_seq):
        kl, vl = synth.random_kv_logical(shape, Ls[b], seed=300 + b, device=dev)
        H.write_prefix(kv, kl, vl, seq=b)
        pre.append((kl, vl))
    model = cad.cad_model_create(shape, W, max_tokens=total)
    o = H.outputs(total, shape.vocab, n_seq=n_seq)
    cad.cad_splice_forward_batched(model, kv, Ls, offsets, H.tensors_i32(np.concatenate(spans)), None,
                                   cad.CAD_COMMIT, o["argmax"], o["accepted"], o["logits"], o["status"])
    torch.cuda.synchronize()
    assert int(o["status"][0]) == 0
    assert list(o["accepted"].cpu().numpy()) == [len(x) for x in spans]
    lg = o["logits"].cpu().numpy()
    am = o["argmax"].cpu().numpy()
    gkv = [H.read_span(kv, Ls[b], len(spans[b]), seq=b) for b in range(n_seq)]

    emb = W["tok_embed"]
    xs = [emb[torch.as_tensor(sp, device=dev).long()].double().cpu().numpy() for sp in spans]
    ks = [[] for _ in range(n_seq)]
    vs = [[] for _ in range(n_seq)]
    hd, hkv = shape.head_dim, shape.n_kv_heads
    for ci in range(shape.n_layers):
        lw = {k: t.double().cpu().numpy() for k, t in W["layers"][ci].items()}
        for b in range(n_seq):
            n = len(spans[b])
            kp = pre[b][0][ci].double().cpu().numpy()
            vp = pre[b][1][ci].double().cpu().numpy()
            z = np.zeros((hkv, n, hd))
            cache = KVCache([np.concatenate([kp, z], axis=1)], [np.concatenate([vp, z], axis=1)])
            xs[b] = splice_layer(cfg, lw, cache, 0, xs[b], Ls[b])
            ks[b].append(cache.k[0][:, Ls[b]:])
            vs[b].append(cache.v[0][:, Ls[b]:])
        del lw
    top = {"final_norm": W["final_norm"].double().cpu().numpy(), "lm_head": W["lm_head"].double().cpu().numpy()}
    graded = 0
    for b in range(n_seq):
        s0, s1 = int(offsets[b]), int(offsets[b + 1])
        ref = final_logits(cfg, top, xs[b])
        err = float(np.max(np.abs(lg[s0:s1] - ref)))
        ok_k, ek = H.kv_close(gkv[b][0], np.stack(ks[b]), TOL)
        ok_v, ev = H.kv_close(gkv[b][1], np.stack(vs[b]), TOL)
        print(f"7B batched seq {b}: L={Ls[b]} N={s1 - s0} logits max|diff| {err:.3e}, K {ek:.3e}, V {ev:.3e}",
              flush=True)
        assert err <= TOL
        assert ok_k and ok_v
        graded += _check_decisions(ref, None, am[s0:s1])
    print(f"7B batched argmax bit-exact on {graded}/{total} graded rows", flush=True)
