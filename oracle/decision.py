"""Masked argmax and longest-agreeing-prefix acceptance.

* Masked argmax -- Copy-as-Decode §2.3 (argmax restricted to the allowed set
  at decision points) and the appendix paragraph on deterministic greedy
  decoding (apply the mask, then take the argmax).  Readings: the mask is a
  per-position bitmask of ``ceil(V/32)`` uint32 words, bit ``v % 32`` of word
  ``v // 32`` set = id ``v`` allowed; no mask = everything allowed; ties go
  to the lowest id; a row that allows nothing yields -1.
* Acceptance -- CopyLoop §2 "Shallow Screening" / "Full-Depth Verification":
  span position 0 (the head, or the first committed token) is always kept;
  position j >= 1 is kept while the prediction made at position j-1 equals
  the span token at j; the first mismatch stops the scan.  Copy-as-Decode
  Fig. 1 / §2.4: inside a copy op acceptance is 1 by construction, so the
  COMMIT mode accepts all N.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

COMMIT, VERIFY = 0, 1


def allowed_matrix(mask: Optional[np.ndarray], N: int, V: int) -> np.ndarray:
    """Unpack the bitmask into bool [N, V]."""
    if mask is None:
        return np.ones((N, V), dtype=bool)
    ids = np.arange(V)
    words = np.asarray(mask, dtype=np.uint32)[:, ids // 32].astype(np.int64)
    return ((words >> (ids % 32)) & 1) == 1


def masked_argmax(logits: np.ndarray, mask: Optional[np.ndarray]) -> np.ndarray:
    """``logits [N, V]``, ``mask [N, ceil(V/32)]`` uint32 or None -> int64 [N].

    Disallowed ids are set to -inf and ``np.argmax`` picks the first maximum,
    i.e. the lowest id among ties; a row with no allowed id gives -1."""
    N, V = logits.shape
    ok = allowed_matrix(mask, N, V)
    vals = np.where(ok, logits, -np.inf)
    out = np.argmax(vals, axis=1).astype(np.int64)
    out[~ok.any(axis=1)] = -1
    return out


def top2_margin(logits: np.ndarray, mask: Optional[np.ndarray]) -> np.ndarray:
    """Gap between the best and the second-best *allowed* logit of each row:
    0 when the maximum is tied between two allowed ids, inf when the row
    allows fewer than two ids (its masked argmax then has no rival).

    This decides which positions the parity tests grade bit-exactly: a
    masked argmax is only well defined against rounding when its margin is
    clear (the tolerance reading of the spec parity rule)."""
    N, V = logits.shape
    ok = allowed_matrix(mask, N, V)
    out = np.empty(N)
    for k in range(N):
        vals = logits[k][ok[k]]
        if len(vals) < 2:
            out[k] = np.inf
        else:
            top = np.partition(vals, len(vals) - 2)[-2:]
            out[k] = top.max() - top.min()
    return out


def acceptance(argmax: Sequence[int], span: Sequence[int], mode: int) -> int:
    """Number of span positions committed: N in COMMIT mode, the longest
    agreeing prefix in VERIFY mode.  The next token after the call is
    ``argmax[accepted - 1]``: the correction on a mismatch, the bonus token
    on a full match."""
    N = len(span)
    if N == 0:
        raise ValueError("empty span")
    if mode == COMMIT:
        return N
    acc = 1
    while acc < N and int(argmax[acc - 1]) == int(span[acc]):
        acc += 1
    return acc
