"""CopyLoop's concurrent pipeline on a looped decoder -- TEST INFRASTRUCTURE.

CopyLoop (Du, Chung), §2:
* "Block Construction": a block is a fresh head followed by up to K tokens
  copied after the longest earlier match of the context's suffix (lengths
  four down to one); no match gives a single-token block.
* "Shallow Screening": at depth ds < D the copied tokens are checked against
  the predictions made one position earlier at that depth; the longest
  agreeing prefix survives, the rest is released at once, and the last
  survivor's shallow prediction becomes the head of the next block.
* "Concurrent Pipeline": surviving positions keep their state and go on
  towards depth D while new blocks enter; every position advances on its own
  depth's KV states, and causal order is kept (older blocks are deeper).
* "Full-Depth Verification": at depth D tokens are accepted in order; the
  first mismatch supplies the correct token and discards the rest of the
  block and every block built on it; a fully matched block adds the last
  position's prediction as the next token.
§A.1: the decoder starts from the prompt (its full-depth prediction is the
first token), admits blocks, prunes at the screening depth, commits at full
depth, and an admission limit can cut a block's copied tail (its head waits
if nothing fits).

Readings where the pages leave a step open (the plainest one the rest
supports):
* A block's head is verified as soon as the block before it has been read
  out at full depth: if it differs from that readout's next token, the
  block and everything younger are discarded and a correction block headed
  by the verified token takes its place.  A block therefore reaches depth D
  with its head already verified, and its full-depth readout checks only
  its copied tokens.
* The next token after a verified block is committed when it is known (the
  verified head of the following block, or the correction).
* Admission limit: the rows in flight never exceed ``max_rows``; a block
  admitted with r free rows keeps at most r - 1 copied tokens; with no free
  row its head waits (its tail is proposed when it is admitted).
* Every tick advances every block in flight by one depth; a block is read
  out after the tick that brings it to ds (screening) and to D
  (verification); blocks are processed oldest first.

The committed tokens equal greedy full-depth decoding: every committed token
is a full-depth prediction after a verified prefix.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

from .decoder import Config, KVCache, final_logits, splice_layer, splice_hidden, f64, _layer_weights
from .decision import masked_argmax, acceptance, VERIFY
from .suffix import suffix_match


def loop_step(cfg: Config, W, kv: KVCache, groups: Sequence[Dict], tokens: Sequence[int],
              state: np.ndarray) -> Dict[int, np.ndarray]:
    """One tick of the pipeline.  Each group ``{"pos", "rows", "depth",
    "state", "readout"}`` gets one more application of the shared block on
    cache index ``depth``; its rows start from the embedding of their tokens
    (depth 0) or from ``state`` and are written back to ``state``.  Returns
    the logits of every group with ``readout`` set (group index -> [rows, V])."""
    out = {}
    r0 = 0
    for gi, g in enumerate(groups):
        n = int(g["rows"])
        toks = np.asarray(tokens[r0:r0 + n], dtype=np.int64)
        rows = slice(int(g["state"]), int(g["state"]) + n)
        x = f64(W["tok_embed"])[toks] if g["depth"] == 0 else state[rows].copy()
        x = splice_layer(cfg, _layer_weights(W, int(g["depth"]), cfg), kv, int(g["depth"]), x, int(g["pos"]))
        state[rows] = x
        if g.get("readout"):
            out[gi] = final_logits(cfg, W, x)
        r0 += n
    return out


@dataclasses.dataclass
class _Block:
    pos: int
    toks: List[int]
    depth: int = 0
    slot: int = -1          # first state row (-1: waiting for admission)
    in_flight: bool = False


def copyloop_decode(cfg: Config, W, kv: KVCache, prompt: Sequence[int], n_new: int, ds: int, K: int,
                    max_rows: int, max_ngram: int = 4, min_ngram: int = 1):
    """Decode ``n_new`` tokens after ``prompt`` with context-copy blocks,
    shallow screening at ``ds`` and full-depth verification at
    ``cfg.loop_depth``, every block in flight advancing one depth per tick.
    ``kv`` must hold ``len(prompt) + n_new + D * (K + 1)`` positions per
    depth (blocks in flight run ahead of the committed tokens).
    Returns ``(tokens, stats)``."""
    D = cfg.loop_depth
    if not (1 <= ds < D):
        raise ValueError("screening depth must be in [1, D)")
    if max_rows < 1:
        raise ValueError("max_rows must be at least 1")
    L0 = len(prompt)
    # prefill: the prompt through all D depths; its last full-depth prediction is the first token
    x = splice_hidden(cfg, W, kv, 0, prompt)
    first = int(masked_argmax(final_logits(cfg, W, x[-1:]), None)[0])
    hist: List[int] = [int(t) for t in prompt]
    out: List[int] = [first]
    # rejected: copied rows refused at full depth; discarded: rows of younger
    # blocks dropped with them (or after a refused head)
    stats = dict(ticks=0, rows_run=0, blocks=0, proposed=0, screened_out=0, rejected=0, discarded=0)
    n_slots = D
    slot_rows = K + 1
    state = np.zeros((n_slots * slot_rows, cfg.d_model))
    free_slots = list(range(n_slots))
    blocks: List[_Block] = [_Block(L0, [first])]

    def rows_in_flight():
        return sum(len(b.toks) for b in blocks if b.in_flight)

    def admit_waiting():
        # the youngest entry may be a head waiting for room
        b = blocks[-1] if blocks else None
        if b is None or b.in_flight:
            return
        room = max_rows - rows_in_flight()
        if room < 1:
            return
        del hist[b.pos:]
        hist.append(b.toks[0])
        tail, _ = suffix_match(hist, max_ngram, min_ngram, K) if K > 0 else ([], -1)
        tail = [int(t) for t in tail][:room - 1]
        b.toks = b.toks[:1] + tail
        hist.extend(tail)
        b.slot = free_slots.pop(0)
        b.in_flight = True
        stats["blocks"] += 1
        stats["proposed"] += len(tail)

    def discard_from(i):
        for b in blocks[i:]:
            if b.in_flight:
                stats["discarded"] += len(b.toks)
                free_slots.append(b.slot)
        del blocks[i:]
        free_slots.sort()

    admit_waiting()
    while len(out) < n_new:
        groups = [dict(pos=b.pos, rows=len(b.toks), depth=b.depth, state=b.slot * slot_rows,
                       readout=int(b.depth + 1 in (ds, D))) for b in blocks if b.in_flight]
        live = [b for b in blocks if b.in_flight]
        tokens = [t for b in live for t in b.toks]
        logits = loop_step(cfg, W, kv, groups, tokens, state)
        stats["ticks"] += 1
        stats["rows_run"] += len(tokens)
        for b in live:
            b.depth += 1
        reads = {id(b): logits[i] for i, b in enumerate(live) if i in logits}
        i = 0
        while i < len(blocks):
            b = blocks[i]
            if not b.in_flight or id(b) not in reads:
                i += 1
                continue
            a = masked_argmax(reads[id(b)], None)
            if b.depth == D:
                # full-depth verification of the copied tokens (the head is verified already)
                acc = acceptance(a, b.toks, VERIFY)
                out.extend(b.toks[1:acc])
                nxt = int(a[acc - 1])
                stats["rejected"] += len(b.toks) - acc
                free_slots.append(b.slot)
                free_slots.sort()
                pos_next = b.pos + acc
                del blocks[i]
                if i < len(blocks) and acc == len(b.toks) and blocks[i].toks[0] == nxt:
                    out.append(nxt)                 # the next block's head is the verified token
                else:
                    discard_from(i)
                    del hist[pos_next:]
                    out.append(nxt)
                    blocks.append(_Block(pos_next, [nxt]))   # correction (or continuation) block
                continue                              # block i is now the next entry
            if b.depth == ds:
                # shallow screening: keep the longest prefix agreeing with the depth-ds predictions
                m = acceptance(a, b.toks, VERIFY)
                stats["screened_out"] += len(b.toks) - m
                b.toks = b.toks[:m]
                del hist[b.pos + m:]
                if i == len(blocks) - 1:
                    blocks.append(_Block(b.pos + m, [int(a[m - 1])]))  # seeded by the last survivor
            i += 1
        admit_waiting()
    stats["committed"] = len(out)
    return out[:n_new], stats


def greedy_decode(cfg: Config, W, kv: KVCache, prompt: Sequence[int], n_new: int) -> List[int]:
    """Plain full-depth greedy decoding: the prompt through all depths, then
    one token at a time through all depths (the comparator CopyLoop's
    speedups are quoted against)."""
    from .decoder import decode_step
    x = splice_hidden(cfg, W, kv, 0, prompt)
    out = [int(masked_argmax(final_logits(cfg, W, x[-1:]), None)[0])]
    L0 = len(prompt)
    while len(out) < n_new:
        lg = decode_step(cfg, W, kv, L0 + len(out) - 1, out[-1])[None]
        out.append(int(masked_argmax(lg, None)[0]))
    return out
