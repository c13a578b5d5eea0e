"""Batched splice over independent sequences.

Copy-as-Decode §7 names integration of the splice with paged attention and
continuous batching as the next step; the method itself is unchanged: each
sequence commits its own span over its own cache.  The oracle is therefore
the per-sequence splice applied to every sequence in turn.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from .decoder import Config, KVCache, splice
from .decision import masked_argmax, acceptance


def batched_splice(cfg: Config, W, caches: List[KVCache], Ls: Sequence[int],
                   spans: Sequence[Sequence[int]], masks: Optional[Sequence[Optional[np.ndarray]]],
                   mode: int):
    logits, argmax, accepted = [], [], []
    for b, (kv, L, span) in enumerate(zip(caches, Ls, spans)):
        lg = splice(cfg, W, kv, int(L), span)
        m = None if masks is None else masks[b]
        a = masked_argmax(lg, m)
        logits.append(lg)
        argmax.append(a)
        accepted.append(acceptance(a, span, mode))
    return logits, argmax, np.array(accepted, dtype=np.int64)
