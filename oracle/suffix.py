"""Context-copy proposal by longest matching suffix.

CopyLoop §2 "Block Construction": a block is the model's fresh head token
followed by up to K tokens copied from just after the longest matching
earlier occurrence of the current suffix; suffix lengths are tried from four
down to one; with no match the block is the head alone.

Readings where the summary is silent: the history searched is the whole
token sequence so far (prompt, accepted output and the new head); the
occurrence must end before the last token (so at least one token follows it)
and may overlap the suffix; among occurrences of the same length the most
recent one wins; the proposal runs to at most K tokens or the end of the
history, whichever comes first.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np


def suffix_match(tokens: Sequence[int], max_ngram: int = 4, min_ngram: int = 1,
                 K: int = 8) -> Tuple[np.ndarray, int]:
    """Return ``(proposal, pos)``: the copied tokens (int32, 0..K of them) and
    the history index they start at (-1 when nothing matched)."""
    x = [int(t) for t in tokens]
    T = len(x)
    top = min(max_ngram, T - 1)
    for n in range(top, min_ngram - 1, -1):
        suffix = x[T - n:]
        p = T - 1 - n                      # latest start that leaves a follower
        while p >= 0:
            if x[p:p + n] == suffix:
                start = p + n
                end = min(start + K, T)
                return np.array(x[start:end], dtype=np.int32), start
            p -= 1
    return np.zeros(0, dtype=np.int32), -1
