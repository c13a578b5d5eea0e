"""Looped (shared-block) decoder with shallow screening and full-depth verification.

CopyLoop §2: a block ``[head, copied tail]`` runs through the shared block to
the screening depth ds; the copied tokens are checked against the
predecessor's shallow prediction and only the longest agreeing prefix
survives ("Shallow Screening"); survivors continue to the full depth D,
each depth attending over its own KV states ("Concurrent Pipeline"); at D
tokens are accepted sequentially up to the first mismatch ("Full-Depth
Verification").

Readings: the looped model is a D-deep stack whose D blocks share weights,
with one KV cache per depth; the readout at depth d is the final norm and LM
head applied after d applications; screening and verification use the same
acceptance rule; pruned rows never write deeper caches.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .decoder import Config, KVCache, final_logits, splice_hidden, f64
from .decision import masked_argmax, acceptance, VERIFY


def looped_splice(cfg: Config, W, kv: KVCache, L: int, span: Sequence[int], screen_depth: int,
                  mask: Optional[np.ndarray] = None) -> Dict:
    D = cfg.loop_depth
    N = len(span)
    if not (1 <= screen_depth <= D):
        raise ValueError("screen depth out of range")
    x = splice_hidden(cfg, W, kv, L, span, first=0, last=screen_depth)
    logits_s = final_logits(cfg, W, x)
    a_s = masked_argmax(logits_s, mask)
    m = acceptance(a_s, span, VERIFY)
    x = splice_hidden(cfg, W, kv, L, span, first=screen_depth, last=D, x=x, write_rows=m)
    logits_f = final_logits(cfg, W, x[:m])
    a_f = np.full(N, -1, dtype=np.int64)
    a_f[:m] = masked_argmax(logits_f, None if mask is None else mask[:m])
    acc = acceptance(a_f[:m], list(span)[:m], VERIFY)
    return {"screen_logits": logits_s, "screen_argmax": a_s, "survivors": m,
            "logits": logits_f, "argmax": a_f, "accepted": acc}
