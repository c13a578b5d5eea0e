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


@dataclasses.dataclass
class _LBlock:
    pos: int
    toks: List[int]
    depth: int = 0
    slot: int = -1
    in_flight: bool = False
    line: Optional[int] = None   # None: before any live fork; 0 / 1: the first / second child's line of the fork


def copyloop_branch_decode(cfg: Config, W, kv: KVCache, prompt: Sequence[int], n_new: int, ds: int, d2: int, K: int,
                           max_rows: int, max_ngram: int = 4, min_ngram: int = 1):
    """CopyLoop decoding with branching at a second readout depth (CopyLoop
    §A.2, on top of the pipeline of ``copyloop_decode``): when a block is
    read out at depth ``d2`` (ds < d2 < D), the prediction at its last
    surviving row is compared with the prediction at depth ds that headed
    its child; if they differ, a second child headed by the d2 prediction is
    admitted (with its own copied tail, screened like any block).  The two
    children and their descendants form two lines over the same positions,
    each with its own KV states; blocks older than the fork belong to both
    (their K/V reach both lines).  When the parent is verified at full
    depth, the line whose head equals the verified next token is kept and
    the other removed; if neither matches (or the parent's own tail was
    refused), both are removed and a correction block takes their place.

    Readings where the pages leave a step open:
    * at most one fork is live at a time (a block reaching d2 while one is
      live does not fork), and a fork needs its parent's first child in
      flight and a free row for the second child's head (its copied tail is
      cut to the free rows, as at admission);
    * the second line's positions start from a copy of the KV states at the
      fork; positions older than the fork keep receiving the K/V their
      blocks write at later depths in both lines;
    * blocks of the two lines are processed in the list order (older line
      first); the line kept at resolution becomes the only line.
    Returns ``(tokens, stats)`` like ``copyloop_decode``, with the counters
    ``forks`` (second children admitted), ``forks_kept`` / ``forks_lost``
    (resolutions that kept the second / the first child's line),
    ``fork_rows_dropped`` (rows in flight of the line removed at such a
    resolution, also counted in ``discarded``), and
    ``fork_log``: per fork the tokens before its children and the two heads
    (the depth-ds and the depth-d2 prediction there)."""
    D = cfg.loop_depth
    if not (1 <= ds < d2 < D):
        raise ValueError("need 1 <= ds < d2 < loop_depth")
    if max_rows < 1:
        raise ValueError("max_rows must be at least 1")
    L0 = len(prompt)
    x = splice_hidden(cfg, W, kv, 0, prompt)
    first = int(masked_argmax(final_logits(cfg, W, x[-1:]), None)[0])
    hists: Dict[int, List[int]] = {0: [int(t) for t in prompt]}
    caches: Dict[int, KVCache] = {0: kv}
    out: List[int] = [first]
    stats = dict(ticks=0, rows_run=0, blocks=0, proposed=0, screened_out=0, rejected=0, discarded=0, forks=0,
                 forks_kept=0, forks_lost=0, fork_rows_dropped=0)
    slot_rows = K + 1
    n_slots = 2 * D
    state = np.zeros((n_slots * slot_rows, cfg.d_model))
    free_slots = list(range(n_slots))
    blocks: List[_LBlock] = [_LBlock(L0, [first])]
    fork: Dict = {}          # the live fork: {"parent": block}
    fork_log: List[Dict] = []  # every fork: the tokens before its children, the ds head, the d2 head

    def ln(b):
        return 1 if b.line == 1 else 0

    def rows_in_flight():
        return sum(len(b.toks) for b in blocks if b.in_flight)

    def admit(b, room):
        h = hists[ln(b)]
        del h[b.pos:]
        h.append(b.toks[0])
        tail, _ = suffix_match(h, max_ngram, min_ngram, K) if K > 0 else ([], -1)
        tail = [int(t) for t in tail][:room - 1]
        b.toks = b.toks[:1] + tail
        h.extend(tail)
        b.slot = free_slots.pop(0)
        b.in_flight = True
        stats["blocks"] += 1
        stats["proposed"] += len(tail)

    def admit_waiting():
        for b in list(blocks):
            if not b.in_flight:
                room = max_rows - rows_in_flight()
                if room < 1 or not free_slots:
                    return
                admit(b, room)

    def drop(pred):
        """remove the blocks matching pred (their rows in flight are discarded); returns the rows"""
        n = 0
        for b in blocks:
            if pred(b) and b.in_flight:
                n += len(b.toks)
                free_slots.append(b.slot)
        blocks[:] = [b for b in blocks if not pred(b)]
        free_slots.sort()
        stats["discarded"] += n
        return n

    def end_fork(keep):
        """keep the line `keep` (0 or 1) as the only one"""
        if keep == 1:
            for c in range(len(kv.k)):
                kv.k[c][...] = caches[1].k[c]
                kv.v[c][...] = caches[1].v[c]
            hists[0] = hists[1]
        caches.pop(1, None)
        hists.pop(1, None)
        for b in blocks:
            b.line = None
        fork.clear()

    admit_waiting()
    while len(out) < n_new:
        live = [b for b in blocks if b.in_flight]
        reads = {}
        for b in live:
            n = len(b.toks)
            rows = slice(b.slot * slot_rows, b.slot * slot_rows + n)
            xx = f64(W["tok_embed"])[np.asarray(b.toks, dtype=np.int64)] if b.depth == 0 else state[rows].copy()
            cache = caches[ln(b)]
            xx = splice_layer(cfg, _layer_weights(W, b.depth, cfg), cache, b.depth, xx, b.pos)
            if b.line is None and 1 in caches:   # older than the fork: its K/V belong to both lines
                caches[1].k[b.depth][:, b.pos:b.pos + n] = cache.k[b.depth][:, b.pos:b.pos + n]
                caches[1].v[b.depth][:, b.pos:b.pos + n] = cache.v[b.depth][:, b.pos:b.pos + n]
            state[rows] = xx
            if b.depth + 1 in (ds, d2, D):
                reads[id(b)] = final_logits(cfg, W, xx)
            b.depth += 1
        stats["ticks"] += 1
        stats["rows_run"] += sum(len(b.toks) for b in live)
        i = 0
        while i < len(blocks):
            b = blocks[i]
            if not b.in_flight or id(b) not in reads:
                i += 1
                continue
            a = masked_argmax(reads[id(b)], None)
            if b.depth == D:
                acc = acceptance(a, b.toks, VERIFY)
                out.extend(b.toks[1:acc])
                nxt = int(a[acc - 1])
                stats["rejected"] += len(b.toks) - acc
                free_slots.append(b.slot)
                free_slots.sort()
                pos_next = b.pos + acc
                del blocks[i]
                if fork.get("parent") is b:
                    keep = None
                    if acc == len(b.toks):
                        for line in (0, 1):
                            c = next((bb for bb in blocks if bb.line == line), None)
                            if c is not None and c.toks[0] == nxt:
                                keep = line
                                break
                    if keep is None:
                        drop(lambda bb: bb.line is not None)
                        end_fork(0)
                        del hists[0][pos_next:]
                        out.append(nxt)
                        blocks.append(_LBlock(pos_next, [nxt]))
                    else:
                        stats["fork_rows_dropped"] += drop(lambda bb, k=keep: bb.line == 1 - k)
                        stats["forks_kept" if keep == 1 else "forks_lost"] += 1
                        end_fork(keep)
                        out.append(nxt)
                    continue
                if i < len(blocks) and acc == len(b.toks) and blocks[i].toks[0] == nxt:
                    out.append(nxt)
                else:
                    drop(lambda bb, keep_ids={id(x) for x in blocks[:i]}: id(bb) not in keep_ids)
                    if fork:
                        end_fork(0)
                    del hists[0][pos_next:]
                    out.append(nxt)
                    blocks.append(_LBlock(pos_next, [nxt]))
                continue
            if b.depth == d2:
                child = blocks[i + 1] if i + 1 < len(blocks) else None
                if (not fork and b.line is None and child is not None and child.in_flight
                        and child.pos == b.pos + len(b.toks)):
                    h1 = int(a[len(b.toks) - 1])
                    room = max_rows - rows_in_flight()
                    if h1 != child.toks[0] and room >= 1 and free_slots:
                        fork["parent"] = b
                        for bb in blocks[i + 1:]:
                            bb.line = 0
                        caches[1] = kv.copy()
                        hists[1] = hists[0][:child.pos]
                        nb = _LBlock(child.pos, [h1], line=1)
                        blocks.append(nb)
                        admit(nb, room)
                        stats["forks"] += 1
                        fork_log.append({"prefix": list(hists[0][:child.pos]), "h0": int(child.toks[0]), "h1": h1})
            elif b.depth == ds:
                m = acceptance(a, b.toks, VERIFY)
                stats["screened_out"] += len(b.toks) - m
                b.toks = b.toks[:m]
                del hists[ln(b)][b.pos + m:]
                younger_same_line = any(bb.line == b.line for bb in blocks[i + 1:])
                if not younger_same_line:
                    nb = _LBlock(b.pos + m, [int(a[m - 1])], line=b.line)
                    # a line-0 block goes before the second line's blocks
                    j = next((k for k, bb in enumerate(blocks) if bb.line == 1), len(blocks)) \
                        if b.line == 0 else len(blocks)
                    blocks.insert(j, nb)
            i += 1
        admit_waiting()
    stats["committed"] = len(out)
    stats["fork_log"] = fork_log
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
