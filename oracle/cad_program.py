"""Copy-as-Decode program decoding -- TEST INFRASTRUCTURE.

Copy-as-Decode (Liu):
* §2.1: a program is ``<program> Op* </program>``, an op is
  ``<copy lines="i-j"/>`` or ``<gen> text </gen>``; the resolver (§2.2)
  expands copies to the document's lines i..j (1-indexed, inclusive).
* §2.3: masked model steps at decision points -- {<, </} at op boundaries,
  {copy, gen} for the op type, digits, '-' and the closing quote inside a
  copy's range; forced-template prefills for fixed literal sequences; free
  generation inside a gen body until the token encoding of ``</gen>``.
* Appendix "States.": AWAIT_OP ({<} before the first op, {<, </} after),
  AFTER_LT ({copy, gen}), COPY_LINES (digits, hyphen, digits, closing
  quote; the terminator force-prefilled), GEN_BODY (free), CLOSE
  (``</program>`` force-prefilled).
* Appendix "Forced prefills.": once the op type is chosen the rest of the
  tag is a fixed token sequence spliced in one forward: ``copy`` + `` lines``
  + ``="`` for a copy opener, ``gen`` + ``>`` for a gen opener, ``</`` +
  ``program`` + ``>`` for the terminator.
* Appendix "Token-sequence end-of-gen detector.": a rolling window over the
  last three emitted ids, matched against the three-token encoding of
  ``</gen>``.
* §2.4: a copy op's span is spliced into the cache in one forward.
* §5 "Token-level extension.": ``<copy tokens="a-b"/>`` copies document
  tokens a..b instead of lines.  §5 "Composition with speculative
  decoding.": inside a gen body, drafts (here: the continuation of the
  longest earlier match of the output's suffix in document + output) are
  verified by one forward, lossless.

Readings where the pages leave a step open (the plainest one the rest
supports):
* The prompt ends with ``<program>``; decoding starts in AWAIT_OP.
* Every action feeds a token sequence and the masked argmax of its last row
  is the next decision: a masked step feeds the last chosen token; a forced
  prefill feeds the chosen token followed by the rest of its template; a
  finished copy range feeds the closing quote, ``/>`` and the copied units
  in one forward (the terminator's forced prefill and the copy splice,
  back to back, are one splice).
* Range digits: no leading zero; the first number lies in [1, U] and the
  second in [first, U] (U = the document's line count, or token count for
  token-level copies); a digit is allowed while some number in range still
  starts with the digits so far, the hyphen (the quote) once the number
  itself is in range.
* A gen body runs until the window sees the ``</gen>`` ids (its last id is
  then fed by the next masked step) or reaches ``max_gen`` tokens, after
  which the chosen token and the three ``</gen>`` ids are force-prefilled.
  After ``max_ops`` ops only ``</`` is allowed at an op boundary.
* Gen-body drafts: up to ``draft_k`` tokens continuing the most recent
  earlier match (lengths 4 down to 1) of the stream's suffix in the
  document followed by the stream; verified with the acceptance rule, the
  accepted tokens plus the correction/bonus then pass through the window in
  order (an end-of-gen inside them ends the body there).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

from .decoder import Config, KVCache, splice, final_logits, splice_hidden
from .decision import masked_argmax, acceptance, VERIFY
from .suffix import suffix_match

AWAIT_OP, AFTER_LT, NUM_A, NUM_B, GEN_BODY, DONE = range(6)


@dataclasses.dataclass(frozen=True)
class Table:
    """Token ids of the program's structural literals (tokenizer-specific,
    resolved once at load).  ``kw`` is `` lines`` (or `` tokens`` for the
    token-level primitive)."""
    lt: int
    lt_slash: int
    gt: int
    copy: int
    gen: int
    program: int
    kw: int
    eq_quote: int
    quote: int
    slash_gt: int
    hyphen: int
    digits: Sequence[int]

    @property
    def eog(self):
        return (self.lt_slash, self.gen, self.gt)


def _can_extend(prefix: int, lo: int, hi: int) -> bool:
    """Some integer in [lo, hi] has ``prefix`` as its leading decimal digits."""
    k = 1
    while prefix * k <= hi:
        if prefix * k + (k - 1) >= lo:
            return True
        k *= 10
    return False


class Fsm:
    """The token-level grammar automaton: allowed ids per state and the
    transition on each chosen id."""

    def __init__(self, table: Table, units: int, max_ops: int, max_gen: int):
        self.t, self.U, self.max_ops, self.max_gen = table, units, max_ops, max_gen
        self.state, self.n_ops = AWAIT_OP, 0
        self.v = self.nd = self.a = 0
        self.win: List[int] = []
        self.gen_len = 0
        self.ops: List[Dict] = []

    def allowed(self) -> List[int]:
        t = self.t
        if self.state == AWAIT_OP:
            if self.n_ops >= self.max_ops:
                return [t.lt_slash]
            return [t.lt] if self.n_ops == 0 else [t.lt, t.lt_slash]
        if self.state == AFTER_LT:
            return [t.copy, t.gen]
        if self.state in (NUM_A, NUM_B):
            lo = 1 if self.state == NUM_A else self.a
            ids = [t.digits[d] for d in range(10)
                   if not (self.nd == 0 and d == 0) and _can_extend(self.v * 10 + d, lo, self.U)]
            if self.nd > 0 and lo <= self.v <= self.U:
                ids.append(t.hyphen if self.state == NUM_A else t.quote)
            return ids
        if self.state == GEN_BODY:
            return None  # free generation
        return []

    def mask(self, vocab: int) -> Optional[np.ndarray]:
        ids = self.allowed()
        if ids is None:
            return None
        allowed = np.zeros((1, (vocab + 31) // 32 * 32), dtype=bool)
        allowed[0, ids] = True
        return np.packbits(allowed, axis=1, bitorder="little").view("<u4")

    def choose(self, tok: int) -> List[int]:
        """Apply a chosen id.  Returns the token sequence to feed next: the
        id alone (a masked or free step), or a forced prefill; the empty list
        after the program's end."""
        t = self.t
        if self.state == AWAIT_OP:
            if tok == t.lt:
                self.state = AFTER_LT
                return [tok]
            self.state = DONE
            return [t.lt_slash, t.program, t.gt]
        if self.state == AFTER_LT:
            if tok == t.copy:
                self.state, self.v, self.nd = NUM_A, 0, 0
                return [t.copy, t.kw, t.eq_quote]
            self.state, self.win, self.gen_len = GEN_BODY, [], 0
            self.ops.append({"op": "gen", "body": []})
            return [t.gen, t.gt]
        if self.state in (NUM_A, NUM_B):
            if tok in t.digits:
                self.v, self.nd = self.v * 10 + list(t.digits).index(tok), self.nd + 1
                return [tok]
            if self.state == NUM_A:
                self.a, self.v, self.nd, self.state = self.v, 0, 0, NUM_B
                return [tok]
            self.ops.append({"op": "copy", "a": self.a, "b": self.v})
            self.n_ops += 1
            self.state = AWAIT_OP
            return None  # the host splices the closing quote, "/>" and the span
        if self.state == GEN_BODY:
            self.win = (self.win + [tok])[-3:]
            self.gen_len += 1
            self.ops[-1]["body"].append(tok)
            if tuple(self.win) == t.eog:
                del self.ops[-1]["body"][-3:]
                self.n_ops += 1
                self.state = AWAIT_OP
                return [tok]
            if self.gen_len >= self.max_gen:
                self.n_ops += 1
                self.state = AWAIT_OP
                return [tok, t.lt_slash, t.gen, t.gt]
            return [tok]
        raise ValueError("choice after the program's end")


def span_units(doc_lines: Sequence[Sequence[int]], a: int, b: int, unit: str) -> List[int]:
    """Resolver: the document's lines a..b (or tokens a..b), 1-indexed, inclusive."""
    if unit == "lines":
        return [int(x) for line in doc_lines[a - 1:b] for x in line]
    flat = [int(x) for line in doc_lines for x in line]
    return flat[a - 1:b]


def program_decode(cfg: Config, W, kv: KVCache, prompt: Sequence[int], doc_lines: Sequence[Sequence[int]],
                   table: Table, unit: str = "lines", max_ops: int = 8, max_gen: int = 16, draft_k: int = 0,
                   max_stream: int = 512):
    """Decode a program after ``prompt`` (which ends with ``<program>``).
    Returns the fed token stream (after the prompt), the ops, the resolved
    output (copies expanded, gen bodies as generated) and counters."""
    V = cfg.vocab
    U = len(doc_lines) if unit == "lines" else sum(len(x) for x in doc_lines)
    fsm = Fsm(table, U, max_ops, max_gen)
    doc_flat = [int(x) for line in doc_lines for x in line]
    L = len(prompt)
    lg = splice(cfg, W, kv, 0, prompt)[-1:]
    tok = int(masked_argmax(lg, fsm.mask(V))[0])
    stream: List[int] = []
    stats = dict(forwards=1, masked_steps=1, forced_prefills=0, copies=0, copied_tokens=0, drafts=0,
                 draft_tokens=0, draft_accepted=0)
    while fsm.state != DONE and len(stream) < max_stream:
        if fsm.state == GEN_BODY and draft_k > 0:
            # draft from document + stream, verify [tok, drafts] in one forward
            P = L + len(stream)
            draft, _ = suffix_match(doc_flat + stream + [tok], 4, 1, draft_k)
            seq = [tok] + [int(x) for x in draft]
            lg = splice(cfg, W, kv, P, seq)
            a = masked_argmax(lg, None)
            acc = acceptance(a, seq, VERIFY)
            stats["forwards"] += 1
            stats["drafts"] += 1
            stats["draft_tokens"] += len(seq) - 1
            # the accepted ids go through the automaton in order
            end = -1
            for i in range(acc):
                feed = fsm.choose(seq[i])
                if fsm.state != GEN_BODY:
                    end = i
                    break
            if end < 0:
                stream.extend(seq[:acc])
                stats["draft_accepted"] += acc - 1
                tok = int(a[acc - 1])
                continue
            # the body ended at seq[end]: seq[:end + 1] stay fed, the rest is stale
            stream.extend(seq[:end + 1])
            stats["draft_accepted"] += end
            row = lg[end:end + 1]
            if len(feed) > 1:  # length cap: the close is force-prefilled
                row = splice(cfg, W, kv, L + len(stream), feed[1:])[-1:]
                stream.extend(feed[1:])
                stats["forwards"] += 1
                stats["forced_prefills"] += 1
            stats["masked_steps"] += 1
            tok = int(masked_argmax(row, fsm.mask(V))[0])
            continue
        feed = fsm.choose(tok)
        if feed is None:
            op = fsm.ops[-1]
            feed = [table.quote, table.slash_gt] + span_units(doc_lines, op["a"], op["b"], unit)
            stats["copies"] += 1
            stats["copied_tokens"] += len(feed) - 2
        elif len(feed) > 1:
            stats["forced_prefills"] += 1
        lg = splice(cfg, W, kv, L + len(stream), feed)
        stream.extend(feed)
        stats["forwards"] += 1
        if fsm.state == DONE:
            break
        m = fsm.mask(V)
        if m is not None:
            stats["masked_steps"] += 1
        tok = int(masked_argmax(lg[-1:], m)[0])
    output: List[int] = []
    for op in fsm.ops:
        output += span_units(doc_lines, op["a"], op["b"], unit) if op["op"] == "copy" else op["body"]
    return stream, fsm.ops, output, stats
