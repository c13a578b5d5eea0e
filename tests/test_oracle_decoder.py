"""Pins for the oracle's decoder forward (CPU only).

* splice == N sequential decode steps, logits and cache (Copy-as-Decode
  §2.4 and the appendix paragraph "Position-encoding correctness");
* an independent library implementation of the same Llama-style decoder
  (HF transformers ``LlamaForCausalLM`` in float64 with eager attention and a
  DynamicCache, the API the pages' splice is written in);
* closed forms of the building blocks (RMSNorm, rotary positions, attention
  with one key, zeroed blocks).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.decoder import Config, KVCache
import synth

SMALL_GQA = synth.Shape("small-gqa", 2, 128, 4, 2, 32, 256, 512, dtype="f32")


def small_weights(shape, seed=0, std=0.02):
    return synth.weights_to_numpy(synth.make_weights(shape, seed=seed, std=std))


# ---------------------------------------------------------------------------
# splice vs sequential
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [synth.TINY, SMALL_GQA])
def test_splice_equals_sequential(shape):
    cfg = Config.of(shape)
    W = small_weights(shape)
    prompt = synth.uniform_prompt(48, shape.vocab)
    span = synth.uniform_prompt(9, shape.vocab, seed=9)
    kv_a = KVCache.empty(cfg.n_layers, cfg.n_kv_heads, 64, cfg.head_dim)
    oracle.prefill(cfg, W, kv_a, prompt)
    kv_b = kv_a.copy()
    la = oracle.splice(cfg, W, kv_a, 48, span)
    lb = oracle.sequential(cfg, W, kv_b, 48, span)
    assert np.max(np.abs(la - lb)) <= 1e-10 * max(1.0, np.max(np.abs(lb)))
    for c in range(cfg.n_layers):
        assert np.allclose(kv_a.k[c], kv_b.k[c], rtol=0, atol=1e-12)
        assert np.allclose(kv_a.v[c], kv_b.v[c], rtol=0, atol=1e-12)


def test_splice_leaves_other_slots_untouched():
    shape = SMALL_GQA
    cfg = Config.of(shape)
    W = small_weights(shape)
    r = np.random.default_rng(0)
    kv = KVCache([r.standard_normal((2, 40, 32)) for _ in range(2)],
                 [r.standard_normal((2, 40, 32)) for _ in range(2)])
    before = kv.copy()
    oracle.splice(cfg, W, kv, 20, [1, 2, 3, 4, 5])
    for c in range(2):
        for arr, ref in ((kv.k[c], before.k[c]), (kv.v[c], before.v[c])):
            assert np.array_equal(arr[:, :20], ref[:, :20])
            assert np.array_equal(arr[:, 25:], ref[:, 25:])
            assert not np.array_equal(arr[:, 20:25], ref[:, 20:25])


def test_prefix_splits_compose():
    """Prefill in one call == prefill in chunks (positions advance by N)."""
    shape = SMALL_GQA
    cfg = Config.of(shape)
    W = small_weights(shape, seed=3)
    prompt = synth.uniform_prompt(30, shape.vocab, seed=4)
    kv1 = KVCache.empty(2, 2, 32, 32)
    kv2 = KVCache.empty(2, 2, 32, 32)
    l1 = oracle.prefill(cfg, W, kv1, prompt)
    parts = [oracle.splice(cfg, W, kv2, 0, prompt[:7]), oracle.splice(cfg, W, kv2, 7, prompt[7:19]),
             oracle.splice(cfg, W, kv2, 19, prompt[19:])]
    assert np.allclose(np.concatenate(parts), l1, rtol=0, atol=1e-11)


# ---------------------------------------------------------------------------
# independent implementation: HF transformers Llama, float64, eager attention
# ---------------------------------------------------------------------------

def hf_model(shape, W):
    from transformers import LlamaConfig, LlamaForCausalLM
    conf = LlamaConfig(vocab_size=shape.vocab, hidden_size=shape.d_model,
                       intermediate_size=shape.ffn_dim, num_hidden_layers=shape.n_layers,
                       num_attention_heads=shape.n_q_heads, num_key_value_heads=shape.n_kv_heads,
                       head_dim=shape.head_dim, rms_norm_eps=shape.rms_eps,
                       rope_theta=shape.rope_theta, max_position_embeddings=4096,
                       attention_bias=False, mlp_bias=False, tie_word_embeddings=False,
                       attn_implementation="eager")
    m = LlamaForCausalLM(conf).to(torch.float64).eval()
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    hq, hkv, hd, F = shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn_dim
    with torch.no_grad():
        m.model.embed_tokens.weight.copy_(t(W["tok_embed"]))
        m.model.norm.weight.copy_(t(W["final_norm"]))
        m.lm_head.weight.copy_(t(W["lm_head"]))
        for i, lw in enumerate(W["layers"]):
            L = m.model.layers[i]
            qkv = t(lw["w_qkv"])
            L.self_attn.q_proj.weight.copy_(qkv[: hq * hd])
            L.self_attn.k_proj.weight.copy_(qkv[hq * hd:(hq + hkv) * hd])
            L.self_attn.v_proj.weight.copy_(qkv[(hq + hkv) * hd:])
            L.self_attn.o_proj.weight.copy_(t(lw["w_o"]))
            L.input_layernorm.weight.copy_(t(lw["attn_norm"]))
            L.post_attention_layernorm.weight.copy_(t(lw["ffn_norm"]))
            gu = t(lw["w_gate_up"])
            L.mlp.gate_proj.weight.copy_(gu[:F])
            L.mlp.up_proj.weight.copy_(gu[F:])
            L.mlp.down_proj.weight.copy_(t(lw["w_down"]))
    return m


@pytest.mark.parametrize("shape", [synth.TINY, SMALL_GQA])
def test_matches_hf_llama(shape):
    """HF keeps RMSNorm and the rotary tables in float32 internally, so the
    agreement is at float32 level (well below any plausible indexing or sign
    mistake, which moves logits by O(0.1))."""
    from transformers import DynamicCache
    W = small_weights(shape, seed=1, std=0.05)
    cfg = Config.of(shape)
    L, N = 40, 8
    prompt = synth.uniform_prompt(L, shape.vocab, seed=2)
    span = synth.uniform_prompt(N, shape.vocab, seed=3)
    kv = KVCache.empty(cfg.n_layers, cfg.n_kv_heads, L + N, cfg.head_dim)
    lp = oracle.prefill(cfg, W, kv, prompt)
    ls = oracle.splice(cfg, W, kv, L, span)
    m = hf_model(shape, W)
    cache = DynamicCache()
    with torch.no_grad():
        out1 = m(input_ids=torch.from_numpy(prompt.astype(np.int64))[None], past_key_values=cache,
                 use_cache=True)
        out2 = m(input_ids=torch.from_numpy(span.astype(np.int64))[None],
                 past_key_values=out1.past_key_values, use_cache=True)
    hp = out1.logits[0].numpy()
    hs = out2.logits[0].numpy()
    scale = np.max(np.abs(hs))
    assert scale > 0.1
    assert np.max(np.abs(lp - hp)) < 2e-5 * max(1, scale)
    assert np.max(np.abs(ls - hs)) < 2e-5 * max(1, scale)
    # cached keys/values (keys after rotation) agree as well
    pkv = out2.past_key_values
    for c in range(cfg.n_layers):
        hk = pkv.layers[c].keys[0].numpy() if hasattr(pkv, "layers") else pkv.key_cache[c][0].numpy()
        hv = pkv.layers[c].values[0].numpy() if hasattr(pkv, "layers") else pkv.value_cache[c][0].numpy()
        assert np.max(np.abs(kv.k[c] - hk)) < 1e-4
        assert np.max(np.abs(kv.v[c] - hv)) < 1e-4


# ---------------------------------------------------------------------------
# closed forms of the building blocks
# ---------------------------------------------------------------------------

def test_rmsnorm_closed_forms():
    x = np.full((3, 8), -2.5)
    g = np.arange(1, 9, dtype=np.float64)
    y = oracle.rms_norm(x, g, 0.0)
    assert np.allclose(y, -g[None, :])                  # constant row -> sign * gain
    x2 = np.array([[3.0, 4.0]])
    assert np.allclose(oracle.rms_norm(x2, np.ones(2), 0.0), x2 / math.sqrt(12.5))
    # scale invariance (eps = 0)
    r = np.random.default_rng(1).standard_normal((4, 16))
    assert np.allclose(oracle.rms_norm(7.0 * r, np.ones(16), 0.0), oracle.rms_norm(r, np.ones(16), 0.0))


def test_rope_properties():
    r = np.random.default_rng(2)
    x = r.standard_normal((5, 3, 16))
    pos = np.arange(5) * 37
    y = oracle.rope_rotate(x, pos, 10000.0)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1))   # norm preserving
    assert np.allclose(oracle.rope_rotate(x, np.zeros(5), 10000.0), x)             # identity at 0
    # pair (0, hd/2) rotates by angle p * theta^0 = p
    p = 3
    z = np.zeros((1, 1, 16)); z[0, 0, 0] = 1.0
    w = oracle.rope_rotate(z, np.array([p]), 10000.0)
    assert np.isclose(w[0, 0, 0], math.cos(p)) and np.isclose(w[0, 0, 8], math.sin(p))
    # the dot product depends only on the position difference
    q = r.standard_normal((1, 1, 16)); k = r.standard_normal((1, 1, 16))
    d1 = np.sum(oracle.rope_rotate(q, np.array([50]), 1e4) * oracle.rope_rotate(k, np.array([20]), 1e4))
    d2 = np.sum(oracle.rope_rotate(q, np.array([130]), 1e4) * oracle.rope_rotate(k, np.array([100]), 1e4))
    assert np.isclose(d1, d2)


def test_first_token_attention_is_value():
    """At position 0 the only key is the token's own: attention output = its V,
    so with the FFN zeroed the residual is x + W_o v (GQA-expanded)."""
    shape = SMALL_GQA.replace(n_layers=1)
    cfg = Config.of(shape)
    W = small_weights(shape, seed=5, std=0.1)
    W["layers"][0]["w_down"] = np.zeros_like(W["layers"][0]["w_down"])
    kv = KVCache.empty(1, 2, 4, 32)
    logits = oracle.decode_step(cfg, W, kv, 0, 17)
    x = W["tok_embed"][17].astype(np.float64)
    h = oracle.rms_norm(x, W["layers"][0]["attn_norm"], cfg.rms_eps)
    v = (W["layers"][0]["w_qkv"].astype(np.float64) @ h)[(4 + 2) * 32:].reshape(2, 32)
    o = np.concatenate([v[h_ // 2] for h_ in range(4)])
    x = x + W["layers"][0]["w_o"] @ o
    exp = oracle.rms_norm(x, W["final_norm"], cfg.rms_eps) @ W["lm_head"].astype(np.float64).T
    assert np.allclose(logits, exp, atol=1e-12)


def test_zero_blocks_give_embedding_logits():
    shape = SMALL_GQA
    cfg = Config.of(shape)
    W = small_weights(shape, seed=6)
    for lw in W["layers"]:
        lw["w_o"] = np.zeros_like(lw["w_o"])
        lw["w_down"] = np.zeros_like(lw["w_down"])
    kv = KVCache.empty(2, 2, 16, 32)
    span = [3, 1, 4, 1, 5]
    got = oracle.splice(cfg, W, kv, 0, span)
    e = W["tok_embed"][span].astype(np.float64)
    exp = (e / np.sqrt(np.mean(e * e, axis=1, keepdims=True) + cfg.rms_eps)) @ W["lm_head"].astype(np.float64).T
    assert np.allclose(got, exp, atol=1e-12)


def test_uniform_attention_when_keys_equal():
    """Identical keys give uniform weights: output = mean of the values."""
    shape = SMALL_GQA.replace(n_layers=1)
    cfg = Config.of(shape)
    W = small_weights(shape, seed=8)
    r = np.random.default_rng(3)
    L = 6
    k0 = r.standard_normal((2, 1, 32))
    kv = KVCache([np.zeros((2, 8, 32))], [np.zeros((2, 8, 32))])
    kv.k[0][:, :L] = k0
    kv.v[0][:, :L] = r.standard_normal((2, L, 32))
    # make the new token's key equal too: zero its K projection rows and keys at 0 -> use q = 0 instead
    W["layers"][0]["w_qkv"][: 4 * 32] = 0.0                      # q = 0 -> all scores equal
    lw = W["layers"][0]
    x = W["tok_embed"][9].astype(np.float64)
    h = oracle.rms_norm(x, lw["attn_norm"], cfg.rms_eps)
    qkv = lw["w_qkv"].astype(np.float64) @ h
    vnew = qkv[6 * 32:].reshape(2, 32)
    vals = np.concatenate([kv.v[0][:, :L], vnew[:, None]], axis=1)    # [2, L+1, 32]
    o = np.concatenate([vals[hh // 2].mean(axis=0) for hh in range(4)])
    xo = x + lw["w_o"].astype(np.float64) @ o
    h2 = oracle.rms_norm(xo, lw["ffn_norm"], cfg.rms_eps)
    gu = lw["w_gate_up"].astype(np.float64) @ h2
    F = cfg.ffn_dim
    xf = xo + lw["w_down"].astype(np.float64) @ (gu[:F] / (1 + np.exp(-gu[:F])) * gu[F:])
    exp = oracle.rms_norm(xf, W["final_norm"], cfg.rms_eps) @ W["lm_head"].astype(np.float64).T
    got = oracle.decode_step(cfg, W, kv, L, 9)
    assert np.allclose(got, exp, atol=1e-12)
