"""GPU parity of the two splice variants against the float64 oracle.

* Batched paged splice (continuous-batching form; Copy-as-Decode §7 names
  paged attention and batching as the integration path): independent
  sequences with their own cache lengths share one paged pool through a
  shuffled block table; each sequence commits a one-token generation step or
  a copy span of whole lines.  The oracle is the per-sequence splice.
* Looped decoder with shallow screening (CopyLoop §2 "Block Construction",
  "Shallow Screening", "Full-Depth Verification"): a block [head, copied
  tail] proposed by the suffix matcher runs to the screening depth, the
  agreeing prefix survives to full depth and is verified there.  Planted
  cases take the tail from the oracle's own greedy chain at the screening
  depth (every position survives to full depth) or at full depth with
  screening there (every position is accepted, and a corrupted position
  stops acceptance exactly there).  Each looped case is masked so that
  every decision of both readouts has an oracle top-2 margin of at least
  0.5 (1e-3 for fp32): every screening argmax, survivor count, full-depth
  argmax and acceptance is compared, with no case left ungraded.

Bars as in the other parity tests: logits within 2e-2 and K/V within 2e-2
plus half a bfloat16 spacing (bf16 models), 1e-4 for fp32; argmax and
acceptance bit-exact where every position they depend on has an oracle
top-2 margin above 0.1; the suffix-match proposal is always exact.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.decision import VERIFY, COMMIT
from oracle.decoder import Config, KVCache
import synth

pytestmark = pytest.mark.gpu

cad = pytest.importorskip("verify_forward_amd")
import gpu_helpers as H  # noqa: E402

TOL = 2e-2
MARGIN = 0.1
BLK = cad.CAD_KV_BLOCK


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return "cuda"


def _f64_weights(W):
    conv = lambda t: t.double().cpu().numpy()
    return {"tok_embed": conv(W["tok_embed"]), "final_norm": conv(W["final_norm"]), "lm_head": conv(W["lm_head"]),
            "layers": [{k: conv(v) for k, v in lw.items()} for lw in W["layers"]]}


def _acceptance_graded(ref, mask, span, mode):
    """Oracle acceptance and whether every position it examined is graded."""
    a = oracle.masked_argmax(ref, mask)
    acc = oracle.acceptance(a, span, mode)
    sure = oracle.top2_margin(ref, mask) > MARGIN
    examined = acc if acc < len(span) else len(span) - 1
    return acc, a, sure, mode == COMMIT or bool(sure[:examined].all())


# ---------------------------------------------------------------------------
# batched paged splice, 1B shape
# ---------------------------------------------------------------------------

def test_batched_paged_splice_1b():
    dev = _dev()
    shape = synth.LLAMA_1B
    cfg = Config.of(shape)
    W = synth.make_weights(shape, device=dev)
    W64 = _f64_weights(W)
    r = synth.rng(31, 4)
    n_seq = 6
    Ls = [int(x) for x in r.integers(40, 1400, size=n_seq)]
    Ls[0] = 1023                       # ends one slot before a block boundary
    prompts = [synth.make_line_prompt(1600, shape.vocab, seed=100 + b, line_len_range=(8, 16)) for b in range(n_seq)]
    spans = []
    for b in range(n_seq):
        if b % 3 == 2:                 # a one-token generation step
            spans.append(np.array([int(r.integers(0, shape.vocab))], dtype=np.int32))
        else:                          # a copy of whole duplicated lines
            st = int(prompts[b].dup_starts[int(r.integers(0, len(prompts[b].dup_starts)))])
            idx = int(np.searchsorted(prompts[b].line_starts, st))
            end = int(prompts[b].line_starts[min(idx + 1 + b % 3, len(prompts[b].line_starts) - 1)])
            spans.append(prompts[b].tokens[st:max(end, st + 2)][:48].copy())
    offsets = np.concatenate([[0], np.cumsum([len(s) for s in spans])]).astype(np.int32)
    total = int(offsets[-1])
    mask = synth.banned_ids_mask(total, shape.vocab, 500, seed=9)
    # paged pool: every sequence takes its blocks from one shuffled permutation
    need = [(Ls[b] + len(spans[b]) + BLK - 1) // BLK for b in range(n_seq)]
    max_blocks = max(need)
    pool = int(sum(need)) + 7
    perm = synth.shuffled_block_table(pool, pool, seed=5).numpy()
    table = np.full((n_seq, max_blocks), -1, dtype=np.int32)
    used = 0
    for b in range(n_seq):
        table[b, :need[b]] = perm[used:used + need[b]]
        used += need[b]
    kv = cad.KVCache.alloc(shape, pool, torch.from_numpy(table), device=dev)
    kv.k.fill_(3.0)
    kv.v.fill_(3.0)
    pre = []
    for b in range(n_seq):
        kl, vl = synth.random_kv_logical(shape, Ls[b], seed=200 + b, device=dev)
        H.write_prefix(kv, kl, vl, seq=b)
        pre.append((kl, vl))
    k_before = kv.k.clone()
    model = cad.cad_model_create(shape, W, max_tokens=total)
    o = H.outputs(total, shape.vocab, n_seq=n_seq)
    cad.cad_splice_forward_batched(model, kv, Ls, offsets, H.tensors_i32(np.concatenate(spans)),
                                   torch.from_numpy(mask.view(np.int32)).to(dev), cad.CAD_VERIFY,
                                   o["argmax"], o["accepted"], o["logits"], o["status"])
    torch.cuda.synchronize()
    assert int(o["status"][0]) == 0
    lg = o["logits"].cpu().numpy()
    am = o["argmax"].cpu().numpy()
    acc = o["accepted"].cpu().numpy()
    for b in range(n_seq):
        s0, s1 = int(offsets[b]), int(offsets[b + 1])
        kl, vl = pre[b]
        okv = KVCache.from_prefix(kl.double().cpu().numpy(), vl.double().cpu().numpy(), Ls[b] + len(spans[b]))
        ref = oracle.splice(cfg, W64, okv, Ls[b], spans[b])
        err = np.max(np.abs(lg[s0:s1] - ref))
        print(f"seq {b}: L={Ls[b]} N={len(spans[b])} logits max|diff| {err:.3e}", flush=True)
        assert err <= TOL
        acc_ref, a_ref, sure, graded = _acceptance_graded(ref, mask[s0:s1], spans[b], VERIFY)
        assert np.array_equal(am[s0:s1][sure], a_ref[sure])
        if graded:
            assert acc[b] == acc_ref
        gk, gv = H.read_seq(kv, Ls[b] + len(spans[b]), seq=b)
        ok_k, _ = H.kv_close(gk[:, :, Ls[b]:], np.stack([okv.k[c][:, Ls[b]:] for c in range(cfg.n_layers)]), TOL)
        ok_v, _ = H.kv_close(gv[:, :, Ls[b]:], np.stack([okv.v[c][:, Ls[b]:] for c in range(cfg.n_layers)]), TOL)
        assert ok_k and ok_v
    # blocks no sequence owns are untouched
    free = perm[used:]
    assert torch.equal(kv.k[:, torch.as_tensor(free, device=dev).long()],
                       k_before[:, torch.as_tensor(free, device=dev).long()])


# ---------------------------------------------------------------------------
# looped shared block with shallow screening
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def looped():
    dev = _dev()
    shape = synth.LOOPED
    W = synth.make_weights(shape, device=dev)
    W64 = _f64_weights(W)
    L = 4096
    kl, vl = synth.random_kv_logical(shape, L, device=dev)
    prompt = synth.make_line_prompt(L, shape.vocab)
    model = cad.cad_model_create(shape, W, max_tokens=16)
    return shape, W, W64, L, kl, vl, prompt, model


def _looped_cache(shape, L, kl, vl, N, dev):
    nb = (L + N + BLK - 1) // BLK
    kv = cad.KVCache.alloc(shape, nb, synth.identity_block_table(nb), device=dev)
    H.write_prefix(kv, kl, vl)
    return kv


def _run_looped(model, shape, L, kl, vl, span, ds, mask, dev):
    N = len(span)
    kv = _looped_cache(shape, L, kl, vl, N, dev)
    sa = torch.full((N,), -9, dtype=torch.int32, device=dev)
    sv = torch.full((1,), -9, dtype=torch.int32, device=dev)
    o = H.outputs(N, shape.vocab)
    mask_dev = None if mask is None else torch.from_numpy(mask.view(np.int32).copy()).to(dev)
    cad.cad_splice_forward_looped(model, kv, L, H.tensors_i32(span), ds, mask_dev, sa, sv, o["argmax"],
                                  o["accepted"], o["logits"], o["status"])
    torch.cuda.synchronize()
    assert int(o["status"][0]) == 0
    return (sa.cpu().numpy(), int(sv[0]), o["argmax"].cpu().numpy(), int(o["accepted"][0]),
            o["logits"].cpu().numpy())


def _looped_case(looped_args, span, ds, label, tol=TOL, gap=0.5):
    """Oracle first (unmasked, to build a mask with clear margins), then the
    GPU call with that mask, then every output compared."""
    shape, W64, L, kl, vl, model, dev = looped_args
    cfg = Config.of(shape)
    N = len(span)
    kl64, vl64 = kl.double().cpu().numpy(), vl.double().cpu().numpy()
    res0 = oracle.looped_splice(cfg, W64, KVCache.from_prefix(kl64, vl64, L + N), L, span, ds)
    mask = H.clear_margin_mask(res0["screen_logits"], res0["logits"], gap)
    res = oracle.looped_splice(cfg, W64, KVCache.from_prefix(kl64, vl64, L + N), L, span, ds, mask)
    m = res["survivors"]
    assert m == res0["survivors"]
    assert (oracle.top2_margin(res["screen_logits"], mask) >= gap).all()
    assert (oracle.top2_margin(res["logits"], mask[:m]) >= gap).all()
    sa, surv, am, acc, lg = _run_looped(model, shape, L, kl, vl, span, ds, mask, dev)
    err = float(np.max(np.abs(lg[:m] - res["logits"])))
    print(f"{label}: N={N} screen depth {ds}: survivors {surv} (oracle {m}), accepted {acc} (oracle "
          f"{res['accepted']}), full-depth logits of {m} rows max|diff| {err:.3e}", flush=True)
    assert np.array_equal(sa, res["screen_argmax"])
    assert surv == m
    assert err <= tol
    assert np.array_equal(am, res["argmax"])
    assert acc == res["accepted"]
    return res


def test_looped_screening_natural(looped):
    """The natural block: the suffix matcher's proposal after a head equal to
    the first token of a duplicated line, screened at depth 2 and verified at
    depth 8."""
    dev = _dev()
    shape, W, W64, L, kl, vl, prompt, model = looped
    K = 8
    head = int(prompt.tokens[int(prompt.dup_starts[3])])
    hist = np.concatenate([prompt.tokens, [head]]).astype(np.int32)
    out_t = torch.full((K,), -9, dtype=torch.int32, device=dev)
    out_n = torch.full((1,), -9, dtype=torch.int32, device=dev)
    out_p = torch.full((1,), -9, dtype=torch.int64, device=dev)
    cad.cad_propose_suffix_match(H.tensors_i32(hist), 4, 1, K, out_t, out_n, out_p)
    torch.cuda.synchronize()
    prop, pos = oracle.suffix_match(hist, 4, 1, K)
    n = int(out_n[0])
    assert n == len(prop) and int(out_p[0]) == pos and list(out_t[:n].cpu().numpy()) == list(prop)
    span = np.concatenate([[head], prop]).astype(np.int32)
    _looped_case((shape, W64, L, kl, vl, model, dev), span, 2, "looped natural")


def _shallow_chain(cfg, W64, kl, vl, L, head, n, depth):
    """The oracle's own greedy chain at readout depth ``depth``: s[0] = head,
    s[j] = argmax of the depth-``depth`` readout after s[j-1]."""
    chain = KVCache.from_prefix(kl.double().cpu().numpy(), vl.double().cpu().numpy(), L + n)
    span = [head]
    for j in range(n - 1):
        lg = oracle.decode_step(cfg, W64, chain, L + j, span[j], depth=depth)[None]
        span.append(int(oracle.masked_argmax(lg, None)[0]))
    return np.asarray(span, dtype=np.int32)


def test_looped_screening_planted_shallow_chain(looped):
    """A tail planted from the depth-2 greedy chain: screening at depth 2 keeps
    all nine positions, so all nine go to depth 8 and their full-depth logits
    and the verification there are compared with the oracle."""
    dev = _dev()
    shape, W, W64, L, kl, vl, prompt, model = looped
    cfg = Config.of(shape)
    span = _shallow_chain(cfg, W64, kl, vl, L, 23, 9, 2)
    res = _looped_case((shape, W64, L, kl, vl, model, dev), span, 2, "looped planted depth-2 chain")
    assert res["survivors"] == len(span)


def test_looped_planted_full_depth_chain(looped):
    """Screening at full depth and a span planted from the oracle's own
    full-depth greedy chain: all N positions are accepted, and corrupting
    position j stops acceptance exactly there.  Each position's mask allows
    the greedy id and only ids at least 0.5 below it, so every examined
    position has a masked top-2 margin of at least 0.5; the full-depth
    logits of every survivor are compared."""
    dev = _dev()
    shape, W, W64, L, kl, vl, prompt, model = looped
    cfg = Config.of(shape)
    D, N = shape.loop_depth, 9
    span = list(_shallow_chain(cfg, W64, kl, vl, L, 17, N, D))
    for bad_at in (None, 3):
        sp = list(span)
        if bad_at is not None:
            sp[bad_at] = (sp[bad_at] + 1) % shape.vocab
        res = _looped_case((shape, W64, L, kl, vl, model, dev), np.asarray(sp, dtype=np.int32), D,
                           f"looped planted full-depth chain, corrupt at {bad_at}")
        want = N if bad_at is None else bad_at
        assert res["survivors"] == want and res["accepted"] == want


def test_looped_fp32_tiny():
    """The looped path on the fp32 kernels (tiny block applied 3 times, 1e-4
    bar, decisions graded at a 1e-3 margin): screening at depth 1 of a
    natural block and of a tail planted from the depth-1 greedy chain, and a
    chain planted from the depth-3 greedy decode screened at full depth,
    which must be accepted whole."""
    dev = _dev()
    shape = synth.TINY.replace(name="tiny-looped", loop_depth=3)
    cfg = Config.of(shape)
    Wc = synth.make_weights(shape, seed=0)
    W64 = _f64_weights(Wc)
    Wd = {k: (v.to(dev) if torch.is_tensor(v) else [{kk: vv.to(dev) for kk, vv in lw.items()} for lw in v])
          for k, v in Wc.items()}
    L, N = 300, 6
    kl, vl = synth.random_kv_logical(shape, L, seed=90, device=dev)
    model = cad.cad_model_create(shape, Wd, max_tokens=16)
    args = (shape, W64, L, kl, vl, model, dev)
    natural = np.asarray([11, 400, 7, 93, 1000, 5], dtype=np.int32)
    _looped_case(args, natural, 1, "looped fp32 natural", tol=1e-4, gap=1e-3)
    shallow = _shallow_chain(cfg, W64, kl, vl, L, 11, N, 1)
    res = _looped_case(args, shallow, 1, "looped fp32 planted depth-1 chain", tol=1e-4, gap=1e-3)
    assert res["survivors"] == N
    full = _shallow_chain(cfg, W64, kl, vl, L, 11, N, shape.loop_depth)
    res = _looped_case(args, full, shape.loop_depth, "looped fp32 planted full-depth chain", tol=1e-4, gap=1e-3)
    assert res["survivors"] == N and res["accepted"] == N
