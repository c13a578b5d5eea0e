"""Float64 Llama-style decoder: one-token decode step and N-token splice.

Copy-as-Decode, §2.4: committing a span of N known tokens is one forward
``model(input_ids=span, past_key_values=KV)``; the appendix paragraph
"Position-encoding correctness" states that it advances positions by N
exactly like N decode steps.  ``decode_step`` is the autoregressive step of
§3 "Kernel microbenchmark"; ``splice`` is the one-forward form; ``sequential``
is N decode steps.  The two are written separately (row-vector loop vs.
causal-batch matrix form) so that their agreement is a real check.

Readings where the pages are silent (Llama-style decoder):

* RMSNorm: ``x / sqrt(mean(x^2) + eps) * g``.
* Rotary positions, half-split pairing: for i < hd/2 with
  ``w_i = theta^(-2i/hd)`` the pair ``(x_i, x_{i+hd/2})`` at absolute position
  p becomes ``(x_i cos(p w_i) - x_{i+hd/2} sin(p w_i),
  x_i sin(p w_i) + x_{i+hd/2} cos(p w_i))``; applied to q and k before k is
  cached; positions are 0-based (prompt 0..L-1, span L..L+N-1).
* GQA: query head h reads KV head ``h // (Hq / Hkv)``; scale 1/sqrt(hd);
  row at position p attends to keys 0..p inclusive.
* FFN: ``(silu(h W_g^T) * (h W_u^T)) W_d^T`` with ``silu(z) = z / (1 + e^-z)``.
* No biases; untied embedding and LM head.
"""
from __future__ import annotations

import dataclasses
from typing import List, Sequence

import numpy as np


@dataclasses.dataclass(frozen=True)
class Config:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    rope_theta: float = 10000.0
    rms_eps: float = 1e-5
    loop_depth: int = 1

    @staticmethod
    def of(shape) -> "Config":
        return Config(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads,
                      shape.head_dim, shape.ffn_dim, shape.vocab, float(shape.rope_theta),
                      float(shape.rms_eps), int(getattr(shape, "loop_depth", 1)))

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


class KVCache:
    """Logical cache: ``k[c]``, ``v[c]`` are float64 ``[Hkv, capacity, hd]``
    for cache index c (one per layer, or one per depth of a looped model)."""

    def __init__(self, k: List[np.ndarray], v: List[np.ndarray]):
        self.k, self.v = k, v

    @staticmethod
    def empty(n_cache: int, n_kv_heads: int, capacity: int, head_dim: int) -> "KVCache":
        z = lambda: np.zeros((n_kv_heads, capacity, head_dim), dtype=np.float64)
        return KVCache([z() for _ in range(n_cache)], [z() for _ in range(n_cache)])

    @staticmethod
    def from_prefix(k, v, capacity: int) -> "KVCache":
        """``k``, ``v``: arrays ``[n_cache][Hkv][L][hd]`` (any float dtype)."""
        n_cache, hkv, L, hd = np.shape(k)
        c = KVCache.empty(n_cache, hkv, capacity, hd)
        for i in range(n_cache):
            c.k[i][:, :L] = np.asarray(k[i], dtype=np.float64)
            c.v[i][:, :L] = np.asarray(v[i], dtype=np.float64)
        return c

    def copy(self) -> "KVCache":
        return KVCache([a.copy() for a in self.k], [a.copy() for a in self.v])


def f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def rms_norm(x: np.ndarray, gain, eps: float) -> np.ndarray:
    """RMSNorm over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * f64(gain)


def rope_rotate(x: np.ndarray, positions, theta: float) -> np.ndarray:
    """Rotate ``x[..., n_heads, hd]`` at absolute ``positions[...]`` (half-split pairs)."""
    hd = x.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=np.float64)
    freq = theta ** (-2.0 * i / hd)
    ang = np.asarray(positions, dtype=np.float64)[..., None] * freq     # [..., half]
    c = np.cos(ang)[..., None, :]
    s = np.sin(ang)[..., None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def _split_qkv(cfg: Config, qkv: np.ndarray):
    hq, hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    q = qkv[..., : hq * hd].reshape(qkv.shape[:-1] + (hq, hd))
    k = qkv[..., hq * hd:(hq + hkv) * hd].reshape(qkv.shape[:-1] + (hkv, hd))
    v = qkv[..., (hq + hkv) * hd:].reshape(qkv.shape[:-1] + (hkv, hd))
    return q, k, v


def _layer_weights(W, cache_index: int, cfg: Config):
    """Layer weights for a cache index: plain stacks index layers directly; a
    looped model applies its one shared block at every depth."""
    return W["layers"][0] if cfg.loop_depth > 1 else W["layers"][cache_index]


def final_logits(cfg: Config, W, x: np.ndarray) -> np.ndarray:
    """LM head over the final RMSNorm: ``rmsnorm(x) g_final W_head^T``."""
    return rms_norm(x, W["final_norm"], cfg.rms_eps) @ f64(W["lm_head"]).T


# ---------------------------------------------------------------------------
# autoregressive decode step: one row, explicit per-head loop
# ---------------------------------------------------------------------------

def decode_layer(cfg: Config, lw, kv: KVCache, ci: int, x: np.ndarray, pos: int) -> np.ndarray:
    """One block for one token at absolute position ``pos``; appends its K/V
    at slot ``pos`` of cache ``ci`` and attends over slots 0..pos."""
    hd, G = cfg.head_dim, cfg.group
    h = rms_norm(x, lw["attn_norm"], cfg.rms_eps)
    q, k, v = _split_qkv(cfg, f64(lw["w_qkv"]) @ h)
    q = rope_rotate(q, pos, cfg.rope_theta)
    k = rope_rotate(k, pos, cfg.rope_theta)
    kv.k[ci][:, pos] = k
    kv.v[ci][:, pos] = v
    o = np.empty((cfg.n_q_heads, hd))
    for head in range(cfg.n_q_heads):
        g = head // G
        keys = kv.k[ci][g, : pos + 1]                 # [pos+1, hd]
        vals = kv.v[ci][g, : pos + 1]
        s = keys @ q[head] / np.sqrt(hd)
        p = np.exp(s - s.max())
        p /= p.sum()
        o[head] = p @ vals
    x = x + f64(lw["w_o"]) @ o.reshape(-1)
    h2 = rms_norm(x, lw["ffn_norm"], cfg.rms_eps)
    gu = f64(lw["w_gate_up"]) @ h2
    F = cfg.ffn_dim
    return x + f64(lw["w_down"]) @ (silu(gu[:F]) * gu[F:])


def decode_step(cfg: Config, W, kv: KVCache, pos: int, token: int, depth: int = None) -> np.ndarray:
    """Logits [V] of one token at position ``pos`` after ``depth`` blocks
    (default: all of them)."""
    n = cfg.n_layers * cfg.loop_depth if depth is None else depth
    x = f64(W["tok_embed"][int(token)])
    for ci in range(n):
        x = decode_layer(cfg, _layer_weights(W, ci, cfg), kv, ci, x, pos)
    return final_logits(cfg, W, x)


def sequential(cfg: Config, W, kv: KVCache, L: int, span: Sequence[int]) -> np.ndarray:
    """N autoregressive decode steps over ``span`` starting at position L."""
    return np.stack([decode_step(cfg, W, kv, L + i, t) for i, t in enumerate(span)])


# ---------------------------------------------------------------------------
# splice: all N rows in one causal-batch pass
# ---------------------------------------------------------------------------

def splice_layer(cfg: Config, lw, kv: KVCache, ci: int, x: np.ndarray, L: int,
                 write_rows: int = None) -> np.ndarray:
    """One block over rows at positions L..L+N-1 (matrix form, causal mask).

    ``write_rows`` (default N) limits which rows' K/V are committed to the
    cache; rows beyond it are still computed but leave the cache untouched and
    their outputs are meaningless (used by the screening variant)."""
    N = x.shape[0]
    hd, G = cfg.head_dim, cfg.group
    wr = N if write_rows is None else write_rows
    pos = L + np.arange(N)
    h = rms_norm(x, lw["attn_norm"], cfg.rms_eps)
    q, k, v = _split_qkv(cfg, h @ f64(lw["w_qkv"]).T)          # [N, heads, hd]
    q = rope_rotate(q, pos, cfg.rope_theta)
    k = rope_rotate(k, pos, cfg.rope_theta)
    kk = kv.k[ci][:, : L + N].copy()
    vv = kv.v[ci][:, : L + N].copy()
    kk[:, L:] = np.transpose(k, (1, 0, 2))
    vv[:, L:] = np.transpose(v, (1, 0, 2))
    kv.k[ci][:, L:L + wr] = kk[:, L:L + wr]
    kv.v[ci][:, L:L + wr] = vv[:, L:L + wr]
    allowed = np.arange(L + N)[None, :] <= pos[:, None]          # [N, L+N]
    o = np.empty((N, cfg.n_q_heads, hd))
    for head in range(cfg.n_q_heads):
        g = head // G
        s = q[:, head] @ kk[g].T / np.sqrt(hd)                    # [N, L+N]
        s = np.where(allowed, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        o[:, head] = p @ vv[g]
    x = x + o.reshape(N, -1) @ f64(lw["w_o"]).T
    h2 = rms_norm(x, lw["ffn_norm"], cfg.rms_eps)
    gu = h2 @ f64(lw["w_gate_up"]).T
    F = cfg.ffn_dim
    return x + (silu(gu[:, :F]) * gu[:, F:]) @ f64(lw["w_down"]).T


def splice_hidden(cfg: Config, W, kv: KVCache, L: int, span: Sequence[int],
                  first: int = 0, last: int = None, x: np.ndarray = None,
                  write_rows: int = None) -> np.ndarray:
    """Residual stream after cache indices ``first..last-1``."""
    n = cfg.n_layers * cfg.loop_depth if last is None else last
    if x is None:
        x = f64(W["tok_embed"])[np.asarray(span, dtype=np.int64)]
    for ci in range(first, n):
        x = splice_layer(cfg, _layer_weights(W, ci, cfg), kv, ci, x, L, write_rows)
    return x


def splice(cfg: Config, W, kv: KVCache, L: int, span: Sequence[int]) -> np.ndarray:
    """Copy-span splice: logits [N, V] for the N span rows; the cache gains
    the span's K/V at slots L..L+N-1 (slots outside are untouched)."""
    return final_logits(cfg, W, splice_hidden(cfg, W, kv, L, span))


def prefill(cfg: Config, W, kv: KVCache, prompt: Sequence[int]) -> np.ndarray:
    """Prompt prefill is the splice from an empty cache."""
    return splice(cfg, W, kv, 0, prompt)
