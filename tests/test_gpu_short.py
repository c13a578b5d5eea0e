"""GPU parity for short spans against the float64 CPU oracle.

Short spans take their own kernels: attention with matrix-core fragments
loaded straight from the paged cache (at most 16 query rows per KV head),
the sliced RMSNorm whose consumers normalise while staging (at most 8
rows), and the rotary append on one work-group per KV group.  These cases
put them at ragged cache lengths (partial 32-key tiles and 16-slot
blocks), on an empty cache, in batched calls of short sequences, with every
stale cache slot holding NaN (a masked key must contribute nothing, not
NaN * 0), with a block id outside the pool and with token ids outside the
vocabulary (status bits, no access out of range).
Batched calls that mix one-token steps with longer copies send every
sequence through the LDS-staged attention instead, at 64-row query tiles
(at most 64 query rows per sequence on average) and at 256-row tiles
(more), with ragged last tiles in both.  Rejected calls (span over max_tokens or
past the block table, negative length, unknown mode) must return their
status without touching outputs or cache.  A batched call at the limit of
64 sequences runs on both attention paths; one sequence more is refused.

Bars: logits max|diff| <= 2e-2 (bf16 models); appended K/V within the same
bound; argmax bit-exact where the oracle's masked top-2 margin exceeds 0.1.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.decision import VERIFY
from oracle.decoder import Config, KVCache
import synth

pytestmark = pytest.mark.gpu

cad = pytest.importorskip("verify_forward_amd")
import gpu_helpers as H  # noqa: E402

TOL = 2e-2
MARGIN = 0.1
BLK = cad.CAD_KV_BLOCK

SHAPES = {
    # the 1B shape cut to two layers (head_dim 64, four query heads per KV head)
    "1b-2layer": synth.LLAMA_1B.replace(name="llama-1b-2layer", n_layers=2),
    # a small GQA model with the 7B head size (head_dim 128, G = 4)
    "gqa128": synth.Shape("gqa-128", 2, 1024, 8, 2, 128, 2048, 4096),
}


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return "cuda"


@pytest.fixture(scope="module", params=sorted(SHAPES))
def model_w(request):
    dev = _dev()
    shape = SHAPES[request.param]
    W = synth.make_weights(shape, seed=synth.SEED_WEIGHTS, device=dev)
    return shape, W, synth.weights_to_numpy(W)


def _prefix(shape, L, seed, dev):
    if L == 0:
        z = torch.zeros((shape.cache_layers, shape.n_kv_heads, 0, shape.head_dim), dtype=shape.torch_dtype, device=dev)
        return z, z.clone()
    return synth.random_kv_logical(shape, L, seed=seed, device=dev)


def _bits(t):
    return t.view(torch.int16)


@pytest.mark.parametrize("L,N", [(1000, 1), (1000, 3), (0, 3), (1037, 6)])
def test_short_splice_ragged_nan_slots(model_w, L, N):
    dev = _dev()
    shape, W, Wn = model_w
    cfg = Config.of(shape)
    print(f"shape={shape.name} L={L} N={N}", flush=True)
    kl, vl = _prefix(shape, L, seed=41 + L, dev=dev)
    prompt = synth.make_line_prompt(max(L, 256), shape.vocab, seed=7)
    span = synth.pick_span(prompt, N)
    nb = (L + N + BLK - 1) // BLK + 3
    table = synth.shuffled_block_table(nb, nb, seed=L + N)
    kv = cad.KVCache.alloc(shape, nb, table, device=dev)
    kv.k.fill_(float("nan"))
    kv.v.fill_(float("nan"))
    H.write_prefix(kv, kl, vl)
    k_before, v_before = kv.k.clone(), kv.v.clone()
    mask = synth.banned_ids_mask(N, shape.vocab, 64, seed=N)
    model = cad.cad_model_create(shape, W, max_tokens=16)
    o = H.outputs(N, shape.vocab)
    cad.cad_splice_forward(model, kv, L, H.tensors_i32(span), torch.from_numpy(mask.view(np.int32)).to(dev),
                           cad.CAD_VERIFY, o["argmax"], o["accepted"], o["logits"], o["status"])
    okv = KVCache.from_prefix(kl.double().cpu().numpy(), vl.double().cpu().numpy(), L + N)
    ref = oracle.splice(cfg, Wn, okv, L, span)
    torch.cuda.synchronize()
    assert int(o["status"][0]) == 0
    lg = o["logits"].cpu().numpy()
    assert np.isfinite(lg).all()
    err = float(np.max(np.abs(lg - ref)))
    print(f"  logits max|diff| = {err:.3e}", flush=True)
    assert err <= TOL
    sure = oracle.top2_margin(ref, mask) > MARGIN
    a_ref = oracle.masked_argmax(ref, mask)
    assert np.array_equal(o["argmax"].cpu().numpy()[sure], a_ref[sure])
    gk, gv = H.read_seq(kv, L + N)
    ok_k, ek = H.kv_close(gk[:, :, L:], np.stack([okv.k[c][:, L:] for c in range(cfg.n_layers)]), TOL)
    ok_v, ev = H.kv_close(gv[:, :, L:], np.stack([okv.v[c][:, L:] for c in range(cfg.n_layers)]), TOL)
    print(f"  kv max|diff| = {ek:.3e} / {ev:.3e}", flush=True)
    assert ok_k and ok_v
    # every slot outside [L, L + N) keeps its bits (NaN included)
    tab = table.long().to(dev)
    used = set()
    for t in range(L, L + N):
        used.add((int(tab[t // BLK]), t % BLK))
    kb, ke = _bits(kv.k), _bits(k_before)
    vb, ve = _bits(kv.v), _bits(v_before)
    changed_k = (kb != ke).any(dim=4).any(dim=2).any(dim=0)  # [block][slot]
    changed_v = (vb != ve).any(dim=3).any(dim=2).any(dim=0)
    for blk, slot in zip(*torch.nonzero(changed_k | changed_v, as_tuple=True)):
        assert (int(blk), int(slot)) in used


def _batched_case(shape, W, Wn, Ls, Ns, seed):
    dev = _dev()
    cfg = Config.of(shape)
    n_seq = len(Ls)
    r = synth.rng(seed)
    spans = [synth.zipf_ids(r, n, shape.vocab).astype(np.int32) for n in Ns]
    offsets = np.concatenate([[0], np.cumsum(Ns)]).astype(np.int32)
    total = int(offsets[-1])
    need = [(Ls[b] + Ns[b] + BLK - 1) // BLK for b in range(n_seq)]
    pool = int(sum(need)) + 5
    perm = synth.shuffled_block_table(pool, pool, seed=seed).numpy()
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
        kl, vl = _prefix(shape, Ls[b], seed=300 + b, dev=dev)
        H.write_prefix(kv, kl, vl, seq=b)
        pre.append((kl, vl))
    model = cad.cad_model_create(shape, W, max_tokens=total)
    o = H.outputs(total, shape.vocab, n_seq=n_seq)
    cad.cad_splice_forward_batched(model, kv, Ls, offsets, H.tensors_i32(np.concatenate(spans)), None,
                                   cad.CAD_VERIFY, o["argmax"], o["accepted"], o["logits"], o["status"])
    torch.cuda.synchronize()
    assert int(o["status"][0]) == 0
    lg = o["logits"].cpu().numpy()
    am = o["argmax"].cpu().numpy()
    for b in range(n_seq):
        s0, s1 = int(offsets[b]), int(offsets[b + 1])
        kl, vl = pre[b]
        okv = KVCache.from_prefix(kl.double().cpu().numpy(), vl.double().cpu().numpy(), Ls[b] + Ns[b])
        ref = oracle.splice(cfg, Wn, okv, Ls[b], spans[b])
        err = float(np.max(np.abs(lg[s0:s1] - ref)))
        print(f"  seq {b}: L={Ls[b]} N={Ns[b]} logits max|diff| {err:.3e}", flush=True)
        assert err <= TOL
        sure = oracle.top2_margin(ref, None) > MARGIN
        assert np.array_equal(am[s0:s1][sure], oracle.masked_argmax(ref, None)[sure])
        gk, gv = H.read_seq(kv, Ls[b] + Ns[b], seq=b)
        ok_k, _ = H.kv_close(gk[:, :, Ls[b]:], np.stack([okv.k[c][:, Ls[b]:] for c in range(cfg.n_layers)]), TOL)
        ok_v, _ = H.kv_close(gv[:, :, Ls[b]:], np.stack([okv.v[c][:, Ls[b]:] for c in range(cfg.n_layers)]), TOL)
        assert ok_k and ok_v


def test_short_batched_sequences(model_w):
    shape, W, Wn = model_w
    print(f"shape={shape.name}: 11 rows over 5 sequences", flush=True)
    _batched_case(shape, W, Wn, Ls=[0, 517, 1000, 33, 2041], Ns=[1, 4, 2, 3, 1], seed=61)
    print(f"shape={shape.name}: 7 rows over 4 sequences", flush=True)
    _batched_case(shape, W, Wn, Ls=[95, 0, 1600, 64], Ns=[1, 2, 1, 3], seed=62)


def test_batched_mixed_steps_and_copies(model_w):
    shape, W, Wn = model_w
    print(f"shape={shape.name}: 66 rows over 5 sequences (64-row query tiles)", flush=True)
    _batched_case(shape, W, Wn, Ls=[1200, 0, 900, 2047, 64], Ns=[1, 40, 1, 23, 1], seed=63)
    print(f"shape={shape.name}: 161 rows over 3 sequences (256-row query tiles)", flush=True)
    _batched_case(shape, W, Wn, Ls=[700, 1500, 31], Ns=[90, 1, 70], seed=64)


def test_batched_at_the_sequence_limit(model_w):
    dev = _dev()
    shape, W, Wn = model_w
    n = cad.CAD_MAX_SEQS
    r = synth.rng(65, n)
    Ls = [int(x) for x in r.integers(0, 400, size=n)]
    Ns = [int(x) for x in r.integers(1, 5, size=n)]
    print(f"shape={shape.name}: {sum(Ns)} rows over {n} sequences (short-span kernels)", flush=True)
    _batched_case(shape, W, Wn, Ls=Ls, Ns=Ns, seed=66)
    Ns[17] = 20
    print(f"shape={shape.name}: {sum(Ns)} rows over {n} sequences, one of 20 rows (LDS-staged)", flush=True)
    _batched_case(shape, W, Wn, Ls=Ls, Ns=Ns, seed=67)
    # one sequence more than the limit is refused before anything runs
    kv = cad.KVCache.alloc(shape, 4, synth.identity_block_table(4), device=dev)
    model = cad.cad_model_create(shape, W, max_tokens=n + 1)
    o = H.outputs(n + 1, shape.vocab, n_seq=n + 1)
    with pytest.raises(cad.CadError) as ei:
        cad.cad_splice_forward_batched(model, kv, [0] * (n + 1), list(range(n + 2)),
                                       H.tensors_i32(np.ones(n + 1)), None, cad.CAD_COMMIT, o["argmax"],
                                       o["accepted"], o["logits"], o["status"])
    assert ei.value.status == cad.CAD_E_ARG
    torch.cuda.synchronize()
    assert bool((o["argmax"] == -7).all())


def test_rejected_calls_enqueue_nothing(model_w):
    """Argument and capacity errors come back as a status before anything is
    enqueued (outputs and cache keep their bits); a call that fills the block
    table exactly then runs and matches the oracle."""
    dev = _dev()
    shape, W, Wn = model_w
    cfg = Config.of(shape)
    nb, N = 7, 3
    L = nb * BLK - N                  # L + N fills the seven blocks exactly
    kl, vl = _prefix(shape, L, seed=19, dev=dev)
    kv = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
    H.write_prefix(kv, kl, vl)
    k_before, v_before = kv.k.clone(), kv.v.clone()
    model = cad.cad_model_create(shape, W, max_tokens=8)
    o9, o = H.outputs(9, shape.vocab), H.outputs(N, shape.vocab)
    o9["logits"].fill_(123.0)
    o["logits"].fill_(123.0)
    span9 = H.tensors_i32(np.arange(1, 10))
    span = H.tensors_i32([5, 6, 7])

    def call(L_, sp, out, mode=cad.CAD_COMMIT):
        cad.cad_splice_forward(model, kv, L_, sp, None, mode, out["argmax"], out["accepted"], out["logits"],
                               out["status"])

    cases = [(lambda: call(L, span9, o9), cad.CAD_E_CAPACITY),      # N > max_tokens
             (lambda: call(L + 1, span, o), cad.CAD_E_CAPACITY),    # L + N past the block table
             (lambda: call(-1, span, o), cad.CAD_E_ARG),            # negative cache length
             (lambda: call(L, span, o, mode=7), cad.CAD_E_ARG)]     # unknown mode
    for i, (fn, st) in enumerate(cases):
        with pytest.raises(cad.CadError) as ei:
            fn()
        print(f"  case {i}: status {ei.value.status}: {ei.value}", flush=True)
        assert ei.value.status == st
    torch.cuda.synchronize()
    for out in (o9, o):
        assert bool((out["argmax"] == -7).all()) and bool((out["logits"] == 123.0).all())
    assert torch.equal(_bits(kv.k), _bits(k_before)) and torch.equal(_bits(kv.v), _bits(v_before))
    call(L, span, o)
    okv = KVCache.from_prefix(kl.double().cpu().numpy(), vl.double().cpu().numpy(), L + N)
    ref = oracle.splice(cfg, Wn, okv, L, np.array([5, 6, 7]))
    torch.cuda.synchronize()
    err = float(np.max(np.abs(o["logits"].cpu().numpy() - ref)))
    print(f"  at the table's edge (L={L}, N={N}): logits max|diff| {err:.3e}", flush=True)
    assert int(o["status"][0]) == 0 and int(o["accepted"][0]) == N
    assert err <= TOL


def test_short_bad_block_sets_status(model_w):
    dev = _dev()
    shape, W, Wn = model_w
    L, N = 1000, 1
    kl, vl = _prefix(shape, L, seed=5, dev=dev)
    nb = (L + N + BLK - 1) // BLK
    table = synth.identity_block_table(nb)
    kv = cad.KVCache.alloc(shape, nb, table, device=dev)
    H.write_prefix(kv, kl, vl)
    # a prefix block id past the pool: attention flags it and reads nothing there
    kv.block_table[5] = nb + 100
    model = cad.cad_model_create(shape, W, max_tokens=16)
    o = H.outputs(N, shape.vocab)
    cad.cad_splice_forward(model, kv, L, H.tensors_i32([3]), None, cad.CAD_COMMIT, o["argmax"], o["accepted"],
                           o["logits"], o["status"])
    torch.cuda.synchronize()
    assert int(o["status"][0]) & cad.CAD_DEV_BAD_BLOCK


@pytest.mark.parametrize("which,scale,N", [("w_qkv", 1e6, 3), ("w_gate_up", 1e3, 40)])
def test_half_range_sets_status(which, scale, N):
    """Activations beyond half precision's range are saturated where they are
    written at half precision and flag the call: q and the span's own K/V
    (the QKV weights scaled by 1e6, any span length), and the SwiGLU output
    that feeds the down projection as one half plane above 16 rows (the
    gate/up weights scaled by 1e3, 40 rows).  The unscaled model leaves the
    bit clear (every parity test asserts a zero status)."""
    dev = _dev()
    shape = SHAPES["gqa128"]
    W = synth.make_weights(shape, seed=synth.SEED_WEIGHTS, device=dev)
    for lw in W["layers"]:
        lw[which].mul_(scale)
    L = 100
    kl, vl = _prefix(shape, L, seed=9, dev=dev)
    nb = (L + N + BLK - 1) // BLK
    kv = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
    H.write_prefix(kv, kl, vl)
    model = cad.cad_model_create(shape, W, max_tokens=N)
    o = H.outputs(N, shape.vocab)
    span = synth.pick_span(synth.make_line_prompt(256, shape.vocab, seed=3), N)
    cad.cad_splice_forward(model, kv, L, H.tensors_i32(span), None, cad.CAD_COMMIT, o["argmax"], o["accepted"],
                           o["logits"], o["status"])
    torch.cuda.synchronize()
    cad.cad_model_destroy(model)
    st = int(o["status"][0])
    print(f"{which} x {scale:g}, N={N}: status {st}", flush=True)
    assert st & cad.CAD_DEV_F16_RANGE


def test_bad_token_sets_status(model_w):
    """A token id outside the vocabulary sets a status bit; its row is
    embedded as zeros (no table access out of range) and every output stays
    finite."""
    dev = _dev()
    shape, W, Wn = model_w
    L = 40
    kl, vl = _prefix(shape, L, seed=7, dev=dev)
    nb = (L + 3 + BLK - 1) // BLK
    kv = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
    H.write_prefix(kv, kl, vl)
    model = cad.cad_model_create(shape, W, max_tokens=16)
    o = H.outputs(3, shape.vocab)
    cad.cad_splice_forward(model, kv, L, H.tensors_i32([3, shape.vocab + 5, -2]), None, cad.CAD_COMMIT,
                           o["argmax"], o["accepted"], o["logits"], o["status"])
    torch.cuda.synchronize()
    assert int(o["status"][0]) & cad.CAD_DEV_BAD_TOKEN
    assert bool(torch.isfinite(o["logits"]).all())
    assert int(o["accepted"][0]) == 3

