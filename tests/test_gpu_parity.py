"""GPU parity: libcad (through the C ABI) against the float64 CPU oracle.

Bars (floating point): logits max|diff| <= 1e-4 in fp32 and <= 2e-2 in bf16;
appended KV within the same bound; argmax bit-exact at every position whose
oracle top-2 masked margin exceeds 0.1; accepted bit-exact when every
position it examines has such a margin.  Integer work (suffix match) is
bit-exact everywhere.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.decision import COMMIT, VERIFY
from oracle.decoder import Config, KVCache
import synth

pytestmark = pytest.mark.gpu

cad = pytest.importorskip("verify_forward_amd")
import gpu_helpers as H  # noqa: E402

TOL = {"f32": 1e-4, "bf16": 2e-2}
MARGIN = 0.1


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return "cuda"


def check_decisions(lg_ref, mask, a_gpu, span, mode, acc_gpu):
    a_ref = oracle.masked_argmax(lg_ref, mask)
    margin = oracle.top2_margin(lg_ref, mask)
    sure = margin > MARGIN
    assert np.array_equal(a_gpu[sure], a_ref[sure]), (a_gpu[sure], a_ref[sure])
    acc_ref = oracle.acceptance(a_ref, span, mode)
    examined = acc_ref if acc_ref < len(span) else len(span) - 1
    if mode == COMMIT or sure[:examined].all():
        assert acc_gpu == acc_ref
    return a_ref, acc_ref, sure


# ---------------------------------------------------------------------------
# suffix match: bit-exact
# ---------------------------------------------------------------------------

def test_suffix_match_exhaustive_and_fuzz():
    dev = _dev()
    cases = []
    import itertools
    for T in range(0, 11):
        for seq in itertools.product(range(2), repeat=T):
            cases.append((list(seq), 1 + (T % 4)))
    r = synth.rng(77)
    for _ in range(300):
        T = int(r.integers(2, 5000))
        x = synth.zipf_ids(r, T, 32000)
        if r.random() < 0.5:
            n = int(r.integers(1, 6))
            p = int(r.integers(0, max(1, T - n - 1)))
            x[T - n:] = x[p:p + n]
        cases.append((list(x), int(r.integers(1, 9))))
    n = len(cases)
    outs = torch.full((n, 8), -9, dtype=torch.int32, device=dev)
    lens = torch.full((n,), -9, dtype=torch.int32, device=dev)
    poss = torch.full((n,), -9, dtype=torch.int64, device=dev)
    toks = [torch.tensor(c[0] if c[0] else [0], dtype=torch.int32, device=dev) for c in cases]
    for i, (seq, K) in enumerate(cases):
        cad.cad_propose_suffix_match(toks[i], 4, 1, K, outs[i], lens[i:i + 1], poss[i:i + 1], T=len(seq))
    torch.cuda.synchronize()
    outs, lens, poss = outs.cpu().numpy(), lens.cpu().numpy(), poss.cpu().numpy()
    for i, (seq, K) in enumerate(cases):
        exp, pos = oracle.suffix_match(seq, 4, 1, K)
        assert lens[i] == len(exp) and poss[i] == pos, (seq, K)
        assert list(outs[i, :lens[i]]) == list(exp)


# ---------------------------------------------------------------------------
# tiny fp32 model: prefill + splice + sequential, everything vs the oracle
# ---------------------------------------------------------------------------

def test_tiny_fp32_end_to_end():
    dev = _dev()
    shape = synth.TINY
    cfg = Config.of(shape)
    Wc = synth.make_weights(shape, seed=0)
    Wn = synth.weights_to_numpy(Wc)
    Wd = {k: (v.to(dev) if torch.is_tensor(v) else [{kk: vv.to(dev) for kk, vv in lw.items()} for lw in v])
          for k, v in Wc.items()}
    L, N = 512, 32
    prompt = synth.uniform_prompt(L, shape.vocab)
    span = prompt[100:132].copy()
    mask = synth.banned_ids_mask(N, shape.vocab, 16)
    nb = (L + N + 15) // 16
    kv = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
    model = cad.cad_model_create(shape, Wd, max_tokens=L)
    o = H.outputs(L, shape.vocab)
    cad.cad_splice_forward(model, kv, 0, H.tensors_i32(prompt), None, cad.CAD_COMMIT, o["argmax"],
                           o["accepted"], o["logits"], o["status"])
    okv = KVCache.empty(1, 4, L + N, 64)
    lp = oracle.prefill(cfg, Wn, okv, prompt)
    torch.cuda.synchronize()
    assert int(o["accepted"][0]) == L and int(o["status"][0]) == 0
    assert np.max(np.abs(o["logits"].cpu().numpy() - lp)) <= TOL["f32"]
    gk, gv = H.read_seq(kv, L)
    assert np.max(np.abs(gk[0] - okv.k[0][:, :L])) <= TOL["f32"]
    assert np.max(np.abs(gv[0] - okv.v[0][:, :L])) <= TOL["f32"]
    # splice in VERIFY mode with the banned-ids mask
    o2 = H.outputs(N, shape.vocab)
    mask_t = torch.from_numpy(mask.view(np.int32)).to(dev)
    cad.cad_splice_forward(model, kv, L, H.tensors_i32(span), mask_t, cad.CAD_VERIFY, o2["argmax"],
                           o2["accepted"], o2["logits"], o2["status"])
    okv_seq = okv.copy()
    ls = oracle.splice(cfg, Wn, okv, L, span)
    torch.cuda.synchronize()
    assert np.max(np.abs(o2["logits"].cpu().numpy() - ls)) <= TOL["f32"]
    check_decisions(ls, mask, o2["argmax"].cpu().numpy(), span, VERIFY, int(o2["accepted"][0]))
    gk, gv = H.read_seq(kv, L + N)
    assert np.max(np.abs(gk[0] - okv.k[0][:, :L + N])) <= TOL["f32"]
    assert np.max(np.abs(gv[0] - okv.v[0][:, :L + N])) <= TOL["f32"]
    # the same span as N decode steps on the GPU equals the splice
    kv2 = cad.KVCache(kv.k.clone(), kv.v.clone(), kv.block_table)
    seq_logits = torch.empty((N, shape.vocab), dtype=torch.float32, device=dev)
    am = torch.empty(N, dtype=torch.int32, device=dev)
    span_t = H.tensors_i32(span)
    for j in range(N):
        cad.cad_decode_step(model, kv2, L + j, span_t[j:j + 1], mask_t[j], am[j:j + 1], seq_logits[j])
    torch.cuda.synchronize()
    assert torch.max(torch.abs(seq_logits - o2["logits"])).item() <= TOL["f32"]
    assert torch.max(torch.abs(kv2.k.float() - kv.k.float())).item() <= TOL["f32"]
    lseq = oracle.sequential(cfg, Wn, okv_seq, L, span)
    assert np.max(np.abs(seq_logits.cpu().numpy() - lseq)) <= TOL["f32"]


def test_tiny_fp32_batched():
    """The fp32 path (its own projection and attention kernels) in a batched
    call: sequences of different cache lengths (empty, ragged, one slot
    short of a block) and span lengths share a shuffled paged pool."""
    dev = _dev()
    shape = synth.TINY
    cfg = Config.of(shape)
    Wc = synth.make_weights(shape, seed=0)
    Wn = synth.weights_to_numpy(Wc)
    Wd = {k: (v.to(dev) if torch.is_tensor(v) else [{kk: vv.to(dev) for kk, vv in lw.items()} for lw in v])
          for k, v in Wc.items()}
    Ls, Ns = [0, 200, 511, 47], [5, 1, 32, 9]
    n_seq = len(Ls)
    r = synth.rng(71)
    spans = [r.integers(0, shape.vocab, size=n).astype(np.int32) for n in Ns]
    offsets = np.concatenate([[0], np.cumsum(Ns)]).astype(np.int32)
    need = [(Ls[b] + Ns[b] + 15) // 16 for b in range(n_seq)]
    pool = sum(need) + 3
    perm = synth.shuffled_block_table(pool, pool, seed=72).numpy()
    table = np.full((n_seq, max(need)), -1, dtype=np.int32)
    used = 0
    for b in range(n_seq):
        table[b, :need[b]] = perm[used:used + need[b]]
        used += need[b]
    kv = cad.KVCache.alloc(shape, pool, torch.from_numpy(table), device=dev)
    kv.k.fill_(float("nan"))
    kv.v.fill_(float("nan"))
    pre = []
    for b in range(n_seq):
        kl, vl = synth.random_kv_logical(shape, Ls[b], seed=80 + b, device=dev)
        if Ls[b]:
            H.write_prefix(kv, kl, vl, seq=b)
        pre.append((kl, vl))
    model = cad.cad_model_create(shape, Wd, max_tokens=int(offsets[-1]))
    o = H.outputs(int(offsets[-1]), shape.vocab, n_seq=n_seq)
    cad.cad_splice_forward_batched(model, kv, Ls, offsets, H.tensors_i32(np.concatenate(spans)), None,
                                   cad.CAD_VERIFY, o["argmax"], o["accepted"], o["logits"], o["status"])
    torch.cuda.synchronize()
    assert int(o["status"][0]) == 0
    lg = o["logits"].cpu().numpy()
    for b in range(n_seq):
        s0, s1 = int(offsets[b]), int(offsets[b + 1])
        kl, vl = pre[b]
        okv = KVCache.from_prefix(kl.double().cpu().numpy(), vl.double().cpu().numpy(), Ls[b] + Ns[b])
        ref = oracle.splice(cfg, Wn, okv, Ls[b], spans[b])
        err = float(np.max(np.abs(lg[s0:s1] - ref)))
        print(f"  seq {b}: L={Ls[b]} N={Ns[b]} logits max|diff| {err:.3e}", flush=True)
        assert err <= TOL["f32"]
        check_decisions(ref, None, o["argmax"].cpu().numpy()[s0:s1], spans[b], VERIFY, int(o["accepted"][b]))
        gk, gv = H.read_seq(kv, Ls[b] + Ns[b], seq=b)
        assert np.max(np.abs(gk[0][:, Ls[b]:] - okv.k[0][:, Ls[b]:])) <= TOL["f32"]
        assert np.max(np.abs(gv[0][:, Ls[b]:] - okv.v[0][:, Ls[b]:])) <= TOL["f32"]


def test_masked_argmax_edge_rows_fp32():
    """Masked argmax on the device for a vocabulary that is neither a multiple
    of 32 nor of 4 (1001 ids: a partial last mask word, scalar logit loads):
    an empty row gives -1 and the empty-mask status bit, a single allowed id
    (the last one, or a low one) is returned as is, set bits past the
    vocabulary are ignored, and random rows match the oracle where the masked
    top-2 margin clears the fp32 bar by far."""
    dev = _dev()
    shape = synth.Shape("tiny-v1001", 1, 256, 4, 4, 64, 1024, 1001, dtype="f32")
    cfg = Config.of(shape)
    Wc = synth.make_weights(shape, seed=0)
    Wn = synth.weights_to_numpy(Wc)
    Wd = {k: (v.to(dev) if torch.is_tensor(v) else [{kk: vv.to(dev) for kk, vv in lw.items()} for lw in v])
          for k, v in Wc.items()}
    L, N, V = 64, 8, shape.vocab
    words = (V + 31) // 32
    prompt = synth.uniform_prompt(L, V)
    span = prompt[10:10 + N].copy()
    allowed = np.random.default_rng(5).random((N, words * 32)) < 0.5
    allowed[0] = False                      # empty row
    allowed[1] = False
    allowed[1, V - 1] = True                # only the last id
    allowed[2] = False
    allowed[2, 7] = True                    # only a low id
    allowed[3] = False
    allowed[3, 992:] = True                 # the last word, bits past V set too
    mask = np.packbits(allowed, axis=1, bitorder="little").view("<u4").copy()
    nb = (L + N + 15) // 16
    kv = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
    model = cad.cad_model_create(shape, Wd, max_tokens=L)
    o = H.outputs(L, V)
    cad.cad_splice_forward(model, kv, 0, H.tensors_i32(prompt), None, cad.CAD_COMMIT, o["argmax"],
                           o["accepted"], o["logits"], o["status"])
    o2 = H.outputs(N, V)
    cad.cad_splice_forward(model, kv, L, H.tensors_i32(span), torch.from_numpy(mask.view(np.int32)).to(dev),
                           cad.CAD_COMMIT, o2["argmax"], o2["accepted"], o2["logits"], o2["status"])
    okv = KVCache.empty(1, 4, L + N, 64)
    oracle.prefill(cfg, Wn, okv, prompt)
    ls = oracle.splice(cfg, Wn, okv, L, span)
    torch.cuda.synchronize()
    assert int(o["status"][0]) == 0
    assert np.max(np.abs(o2["logits"].cpu().numpy() - ls)) <= TOL["f32"]
    a = o2["argmax"].cpu().numpy()
    assert a[0] == -1 and a[1] == V - 1 and a[2] == 7
    assert int(o2["status"][0]) == 2 and int(o2["accepted"][0]) == N
    a_ref = oracle.masked_argmax(ls, mask)
    sure = oracle.top2_margin(ls, mask) > 1e-3
    assert a_ref[0] == -1 and a_ref[1] == V - 1 and a_ref[2] == 7
    assert np.array_equal(a[3:][sure[3:]], a_ref[3:][sure[3:]])
    assert sure[3:].sum() >= 4


def test_tiny_fp32_planted_verify():
    """VERIFY accepts a span planted from the oracle's greedy chain whole and
    stops exactly at a corrupted position."""
    dev = _dev()
    shape = synth.TINY
    cfg = Config.of(shape)
    # wider weights make the greedy chain's top-2 margins clear 0.1
    Wc = synth.make_weights(shape, seed=28, std=0.15)
    Wn = synth.weights_to_numpy(Wc)
    Wd = {k: (v.to(dev) if torch.is_tensor(v) else [{kk: vv.to(dev) for kk, vv in lw.items()} for lw in v])
          for k, v in Wc.items()}
    L, N = 64, 12
    prompt = synth.uniform_prompt(L, shape.vocab, seed=22)
    okv = KVCache.empty(1, 4, L + N, 64)
    oracle.prefill(cfg, Wn, okv, prompt)
    chain = okv.copy()
    span = [5]
    for j in range(N - 1):
        span.append(int(oracle.masked_argmax(oracle.decode_step(cfg, Wn, chain, L + j, span[j])[None], None)[0]))
    ref = oracle.splice(cfg, Wn, okv.copy(), L, span)
    margin = oracle.top2_margin(ref, None)
    if not (margin[:N - 1] > MARGIN).all():
        pytest.skip("planted chain has a near-tie (margin <= 0.1); acceptance not graded")
    nb = (L + N + 15) // 16
    kv = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
    model = cad.cad_model_create(shape, Wd, max_tokens=L)
    o = H.outputs(L, shape.vocab)
    cad.cad_splice_forward(model, kv, 0, H.tensors_i32(prompt), None, cad.CAD_COMMIT, o["argmax"], o["accepted"])
    for bad_at in (None, 1, 5, N - 1):
        s = list(span)
        if bad_at is not None:
            s[bad_at] = (s[bad_at] + 1) % shape.vocab
        o2 = H.outputs(N, shape.vocab)
        cad.cad_splice_forward(model, kv, L, H.tensors_i32(s), None, cad.CAD_VERIFY, o2["argmax"], o2["accepted"])
        torch.cuda.synchronize()
        assert int(o2["accepted"][0]) == (N if bad_at is None else bad_at)


# ---------------------------------------------------------------------------
# bf16: the 1B shape over a random prefix cache of L = 4096
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def llama1b():
    dev = _dev()
    shape = synth.LLAMA_1B
    W = synth.make_weights(shape, seed=synth.SEED_WEIGHTS, device=dev)
    Wn = synth.weights_to_numpy(W)
    L = 4096
    kl, vl = synth.random_kv_logical(shape, L, device=dev)
    return shape, W, Wn, L, kl, vl


@pytest.mark.parametrize("N", [1, 4, 8, 16, 64, 256])
def test_llama1b_bf16_splice(llama1b, N):
    dev = _dev()
    shape, W, Wn, L, kl, vl = llama1b
    cfg = Config.of(shape)
    prompt = synth.make_line_prompt(L, shape.vocab)
    span = synth.pick_span(prompt, N)
    nb = (L + 256 + 15) // 16 + 1
    kv = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
    kv.k.fill_(7.0)
    kv.v.fill_(7.0)
    H.write_prefix(kv, kl, vl)
    k_before = kv.k.clone()
    v_before = kv.v.clone()
    model = cad.cad_model_create(shape, W, max_tokens=256)
    o = H.outputs(N, shape.vocab)
    cad.cad_splice_forward(model, kv, L, H.tensors_i32(span), None, cad.CAD_VERIFY, o["argmax"], o["accepted"],
                           o["logits"], o["status"])
    okv = KVCache.from_prefix(kl.float().cpu().numpy(), vl.float().cpu().numpy(), L + N)
    ref = oracle.splice(cfg, Wn, okv, L, span)
    torch.cuda.synchronize()
    assert int(o["status"][0]) == 0
    err = np.max(np.abs(o["logits"].cpu().numpy() - ref))
    print(f"N={N} logits max|diff| = {err:.3e}", flush=True)
    assert err <= TOL["bf16"]
    check_decisions(ref, None, o["argmax"].cpu().numpy(), span, VERIFY, int(o["accepted"][0]))
    gk, gv = H.read_seq(kv, L + N)
    okk, ek = H.kv_close(gk[:, :, L:], np.stack([okv.k[c][:, L:L + N] for c in range(cfg.n_layers)]), TOL["bf16"])
    okv_, ev = H.kv_close(gv[:, :, L:], np.stack([okv.v[c][:, L:L + N] for c in range(cfg.n_layers)]), TOL["bf16"])
    print(f"N={N} kv max|diff| = {ek:.3e} / {ev:.3e}", flush=True)
    assert okk and okv_
    # canaries: the prefix and every slot past L + N are bit-unchanged
    nfull = L // 16
    assert torch.equal(kv.k[:, :nfull], k_before[:, :nfull])
    assert torch.equal(kv.v[:, :nfull], v_before[:, :nfull])
    end = L + N
    eb = (end + 15) // 16
    assert torch.equal(kv.k[:, eb:], k_before[:, eb:])
    if end % 16:
        assert torch.equal(kv.k[:, eb - 1, :, end % 16:], k_before[:, eb - 1, :, end % 16:])
        assert torch.equal(kv.v[:, eb - 1, :, :, end % 16:], v_before[:, eb - 1, :, :, end % 16:])


def test_llama1b_splice_equals_decode_steps(llama1b):
    dev = _dev()
    shape, W, Wn, L, kl, vl = llama1b
    N = 8
    prompt = synth.make_line_prompt(L, shape.vocab)
    span = synth.pick_span(prompt, N, which=3)
    nb = (L + N + 15) // 16
    kv = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
    H.write_prefix(kv, kl, vl)
    kv2 = cad.KVCache(kv.k.clone(), kv.v.clone(), kv.block_table)
    model = cad.cad_model_create(shape, W, max_tokens=N)
    o = H.outputs(N, shape.vocab)
    span_t = H.tensors_i32(span)
    cad.cad_splice_forward(model, kv, L, span_t, None, cad.CAD_COMMIT, o["argmax"], o["accepted"], o["logits"])
    lg = torch.empty((N, shape.vocab), dtype=torch.float32, device=dev)
    am = torch.empty(N, dtype=torch.int32, device=dev)
    for j in range(N):
        cad.cad_decode_step(model, kv2, L + j, span_t[j:j + 1], None, am[j:j + 1], lg[j])
    torch.cuda.synchronize()
    assert torch.max(torch.abs(lg - o["logits"])).item() <= TOL["bf16"]
    # both caches hold bfloat16: the splice reads its own keys at half
    # precision, the steps read earlier steps' keys back from the cache
    ok_k, _ = H.kv_close_stored(kv2.k.float().cpu().numpy(), kv.k.float().cpu().numpy(), TOL["bf16"])
    ok_v, _ = H.kv_close_stored(kv2.v.float().cpu().numpy(), kv.v.float().cpu().numpy(), TOL["bf16"])
    assert ok_k and ok_v


def test_deterministic_rerun(llama1b):
    dev = _dev()
    shape, W, Wn, L, kl, vl = llama1b
    N = 64
    prompt = synth.make_line_prompt(L, shape.vocab)
    span = H.tensors_i32(synth.pick_span(prompt, N, which=5))
    nb = (L + N + 15) // 16
    kv = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
    H.write_prefix(kv, kl, vl)
    model = cad.cad_model_create(shape, W, max_tokens=N)
    res = []
    for _ in range(2):
        o = H.outputs(N, shape.vocab)
        cad.cad_splice_forward(model, kv, L, span, None, cad.CAD_COMMIT, o["argmax"], o["accepted"], o["logits"])
        torch.cuda.synchronize()
        res.append(o["logits"].clone())
    assert torch.equal(res[0], res[1])
