"""Seeded synthetic inputs for the copy-span splice forward.

This module only draws random numbers and arranges them into the shapes the
workloads need: model weights, prompts made of repeated "lines", copy spans,
per-position vocabulary bitmasks, KV caches and the batched serving schedule.
It holds none of the method's arithmetic (no norm, rotation, attention,
projection, argmax or acceptance), so both the CPU oracle and the GPU library
can be fed from it without sharing any computation.

Shapes follow the workloads described for the copy-span splice
(Copy-as-Decode, §3 "Kernel microbenchmark" and §4.1; CopyLoop, §2 "Block
construction"): Llama-style decoders with GQA, RMSNorm, rotary positions and
a SwiGLU FFN, random-initialised with N(0, 0.02) projections and unit gains.

Random streams: every tensor gets its own ``torch.Generator`` seeded from
``(base seed, tensor index)``; token-level data uses ``numpy.random.Generator``
(PCG64) seeded from a ``SeedSequence``.  Generation on a CUDA device gives
different (but equally valid and deterministic) bits than on the CPU; callers
that compare two consumers hand both the *same* generated tensors.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

KV_BLOCK = 16  # tokens per paged KV block

SEED_WEIGHTS, SEED_PROMPT, SEED_SPANS, SEED_SERVE, SEED_KV = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Shape:
    """Decoder shape.  ``loop_depth`` > 1 means one shared block applied that
    many times (``n_layers`` must then be 1)."""
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    dtype: str = "bf16"          # "bf16" or "f32"
    rope_theta: float = 10000.0
    rms_eps: float = 1e-5
    loop_depth: int = 1

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def cache_layers(self) -> int:
        return self.n_layers * self.loop_depth

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def replace(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


TINY = Shape("tiny", 1, 256, 4, 4, 64, 1024, 1024, dtype="f32")
LLAMA_1B = Shape("llama-1b", 16, 2048, 32, 8, 64, 8192, 32000)
LLAMA_7B = Shape("llama-7b", 32, 4096, 32, 8, 128, 14336, 32000)
LOOPED = Shape("looped-2b", 1, 2048, 16, 16, 128, 5632, 32000, loop_depth=8)
# one GPU's share of the 7B shape under 8-way tensor parallelism: one KV head
# with its four query heads, an eighth of the FFN columns and of the
# vocabulary (a vocabulary-split LM head); the residual stream stays d_model
# wide on every GPU
LLAMA_7B_TP8 = Shape("llama-7b-tp8-share", 32, 4096, 4, 1, 128, 1792, 4000)
SHAPES = {s.name: s for s in (TINY, LLAMA_1B, LLAMA_7B, LOOPED, LLAMA_7B_TP8)}


# ----------------------------------------------------------------------------
# weights
# ----------------------------------------------------------------------------

def _gen(seed: int, idx: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + idx) & 0x7FFFFFFFFFFFFFFF)
    return g


def _normal(shape, std, seed, idx, device, dtype):
    g = _gen(seed, idx, device)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(std)
    return t.to(dtype)


def make_weights(shape: Shape, seed: int = SEED_WEIGHTS, device="cpu",
                 std: float = 0.02, layers: Optional[Sequence[int]] = None) -> Dict:
    """Random-init weights in nn.Linear layout ``[out][in]``.

    Returns ``{"tok_embed", "final_norm", "lm_head", "layers": [ {attn_norm,
    w_qkv, w_o, ffn_norm, w_gate_up, w_down}, ... ]}``.  ``w_qkv`` stacks the
    q, k and v rows; ``w_gate_up`` stacks the gate rows then the up rows.
    Gains are ones.  ``layers`` restricts generation to a subset of layer
    indices (each layer's tensors depend only on the seed and its index, so a
    subset has the same bits as the full model).
    """
    dt = shape.torch_dtype
    d, F, V = shape.d_model, shape.ffn_dim, shape.vocab
    hq = shape.n_q_heads * shape.head_dim
    out = {
        "tok_embed": _normal((V, d), std, seed, 0, device, dt),
        "final_norm": torch.ones(d, device=device, dtype=dt),
        "lm_head": _normal((V, d), std, seed, 1, device, dt),
        "layers": [],
    }
    idxs = range(shape.n_layers) if layers is None else layers
    for li in idxs:
        base = 16 + 8 * li
        out["layers"].append({
            "attn_norm": torch.ones(d, device=device, dtype=dt),
            "w_qkv": _normal((shape.qkv_rows, d), std, seed, base + 0, device, dt),
            "w_o": _normal((d, hq), std, seed, base + 1, device, dt),
            "ffn_norm": torch.ones(d, device=device, dtype=dt),
            "w_gate_up": _normal((2 * F, d), std, seed, base + 2, device, dt),
            "w_down": _normal((d, F), std, seed, base + 3, device, dt),
        })
    return out


def weights_to_numpy(w: Dict) -> Dict:
    """Exact host copies as float32 numpy arrays (bf16 -> f32 widening is exact)."""
    conv = lambda t: t.detach().to("cpu", torch.float32).numpy()
    return {
        "tok_embed": conv(w["tok_embed"]),
        "final_norm": conv(w["final_norm"]),
        "lm_head": conv(w["lm_head"]),
        "layers": [{k: conv(v) for k, v in lw.items()} for lw in w["layers"]],
    }


# ----------------------------------------------------------------------------
# token data
# ----------------------------------------------------------------------------

def rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(list(key)))


def zipf_ids(r: np.random.Generator, n: int, vocab: int, a: float = 1.1) -> np.ndarray:
    """``n`` token ids drawn as Zipf(a) - 1, redrawn while >= vocab."""
    out = np.empty(n, dtype=np.int64)
    filled = 0
    while filled < n:
        z = r.zipf(a, size=2 * (n - filled) + 16) - 1
        z = z[z < vocab]
        take = min(len(z), n - filled)
        out[filled:filled + take] = z[:take]
        filled += take
    return out


@dataclasses.dataclass
class LinePrompt:
    tokens: np.ndarray          # int32 [L]
    line_starts: np.ndarray     # int64 start offset of every line slot (< L)
    dup_starts: np.ndarray      # starts of slots whose line occurs twice


def make_line_prompt(L: int, vocab: int, seed: int = SEED_PROMPT, line_len=80,
                     dup_frac: float = 0.7, line_len_range=None) -> LinePrompt:
    """Prompt of ``L`` tokens built from "lines" of Zipf(1.1) ids in which
    about ``dup_frac`` of the line slots hold a line that occurs twice.

    ``line_len_range=(lo, hi)`` draws each line length uniformly in [lo, hi]
    instead of the fixed ``line_len``.
    """
    r = rng(seed, L, vocab)
    lens: List[int] = []
    total = 0
    while total < L:
        n = line_len if line_len_range is None else int(r.integers(line_len_range[0], line_len_range[1] + 1))
        lens.append(n)
        total += n
    n_slots = len(lens)
    n_dup_slots = 2 * int(round(dup_frac * n_slots / 2))
    n_src = n_dup_slots // 2
    # source lines (each placed twice) followed by unique lines
    slot_src = list(range(n_src)) * 2 + list(range(n_src, n_src + n_slots - n_dup_slots))
    order = r.permutation(n_slots)
    slot_src = [slot_src[i] for i in order]
    src_len: Dict[int, int] = {}
    for s, n in zip(slot_src, lens):
        src_len.setdefault(s, n)
    src_tokens = {s: zipf_ids(r, n, vocab) for s, n in sorted(src_len.items())}
    parts, starts, dups = [], [], []
    counts = {s: slot_src.count(s) for s in set(slot_src)}
    pos = 0
    for s in slot_src:
        starts.append(pos)
        if counts[s] == 2:
            dups.append(pos)
        parts.append(src_tokens[s])
        pos += len(src_tokens[s])
    toks = np.concatenate(parts)[:L].astype(np.int32)
    starts = np.array([p for p in starts if p < L], dtype=np.int64)
    dups = np.array([p for p in dups if p < L], dtype=np.int64)
    return LinePrompt(toks, starts, dups)


def uniform_prompt(L: int, vocab: int, seed: int = SEED_PROMPT) -> np.ndarray:
    return rng(seed, L, vocab, 7).integers(0, vocab, size=L).astype(np.int32)


def pick_span(prompt: LinePrompt, N: int, seed: int = SEED_SPANS, which: int = 0) -> np.ndarray:
    """``N`` tokens copied verbatim from the prompt, starting at the first
    token of a duplicated line (crossing line boundaries when N exceeds a
    line)."""
    L = len(prompt.tokens)
    cands = prompt.dup_starts[prompt.dup_starts + N <= L]
    if len(cands) == 0:
        cands = np.array([max(0, L - N)])
    r = rng(seed, N, which)
    st = int(cands[r.integers(0, len(cands))])
    return prompt.tokens[st:st + N].copy()


def mask_words(vocab: int) -> int:
    return (vocab + 31) // 32


def pack_mask(allowed: np.ndarray) -> np.ndarray:
    """bool [N, V] -> uint32 [N, ceil(V/32)], bit v%32 of word v//32, LSB first."""
    N, V = allowed.shape
    W = mask_words(V)
    padded = np.zeros((N, W * 32), dtype=np.uint64)
    padded[:, :V] = allowed
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    return (padded.reshape(N, W, 32) * weights).sum(axis=2).astype(np.uint32)


def allowed_fraction_mask(N: int, vocab: int, n_allowed: int, seed: int = SEED_SPANS,
                          which: int = 0) -> np.ndarray:
    """Each position allows exactly ``n_allowed`` ids, chosen by a seeded permutation."""
    r = rng(seed, N, vocab, n_allowed, which)
    allowed = np.zeros((N, vocab), dtype=bool)
    for k in range(N):
        allowed[k, r.permutation(vocab)[:n_allowed]] = True
    return pack_mask(allowed)


def banned_ids_mask(N: int, vocab: int, n_banned: int, seed: int = SEED_SPANS,
                    which: int = 0) -> np.ndarray:
    """All ids allowed except ``n_banned`` distinct random ids per position."""
    r = rng(seed, N, vocab, n_banned, which, 1)
    allowed = np.ones((N, vocab), dtype=bool)
    for k in range(N):
        allowed[k, r.choice(vocab, size=n_banned, replace=False)] = False
    return pack_mask(allowed)


# ----------------------------------------------------------------------------
# KV caches
# ----------------------------------------------------------------------------

def kv_std(shape: Shape) -> float:
    """Spread of a K or V entry produced by a unit-RMS row times an N(0, 0.02)
    projection: 0.02 * sqrt(d_model)."""
    return 0.02 * math.sqrt(shape.d_model)


def random_kv_logical(shape: Shape, L: int, seed: int = SEED_KV, device="cpu"):
    """Random prefix cache in logical layout: K, V ``[cache_layers][Hkv][L][hd]``."""
    std = kv_std(shape)
    sz = (shape.cache_layers, shape.n_kv_heads, L, shape.head_dim)
    k = _normal(sz, std, seed, 0, device, shape.torch_dtype)
    v = _normal(sz, std, seed, 1, device, shape.torch_dtype)
    return k, v


def identity_block_table(n_blocks: int, device="cpu") -> torch.Tensor:
    return torch.arange(n_blocks, dtype=torch.int32, device=device)


def shuffled_block_table(n_blocks: int, pool_blocks: int, seed: int, device="cpu") -> torch.Tensor:
    """A block table that uses ``n_blocks`` distinct blocks of a pool, in a seeded random order."""
    r = rng(seed, n_blocks, pool_blocks, 11)
    return torch.from_numpy(r.permutation(pool_blocks)[:n_blocks].astype(np.int32)).to(device)


# ----------------------------------------------------------------------------
# batched serving schedule
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class ServeStep:
    L: np.ndarray        # int64 [B] valid cache length per sequence
    spans: List[np.ndarray]  # per sequence int32 [N_b]
    is_copy: np.ndarray  # bool [B]


def serve_step(n_seq: int, prompts: List[LinePrompt], rng_: np.random.Generator,
               L_range=(1024, 8192), p_copy: float = 0.106, p_lines: float = 0.25,
               cap: int = 512) -> ServeStep:
    """One step of the batched editing workload: each sequence either splices a
    copy span of Geometric(p_lines) duplicated lines (capped at ``cap`` tokens)
    or takes a single-token generation step."""
    Ls, spans, copy = [], [], []
    for b in range(n_seq):
        L = int(rng_.integers(L_range[0], L_range[1] + 1))
        pr = prompts[b]
        if rng_.random() < p_copy:
            n_lines = int(rng_.geometric(p_lines))
            cands = pr.dup_starts
            st = int(cands[rng_.integers(0, len(cands))])
            idx = int(np.searchsorted(pr.line_starts, st))
            end_idx = min(idx + n_lines, len(pr.line_starts))
            end = int(pr.line_starts[end_idx]) if end_idx < len(pr.line_starts) else len(pr.tokens)
            span = pr.tokens[st:min(end, st + cap)]
            copy.append(True)
        else:
            span = np.array([int(rng_.integers(0, 32000))], dtype=np.int32) % max(1, int(pr.tokens.max()) + 1)
            copy.append(False)
        spans.append(np.asarray(span, dtype=np.int32))
        Ls.append(L)
    return ServeStep(np.array(Ls, dtype=np.int64), spans, np.array(copy))
