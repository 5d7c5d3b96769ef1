"""Oracle: Longformer token-level attention pattern.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Longformer: The Long-Document Transformer, §3.1 "Sliding Window": with window
size w every token attends to w/2 tokens on each side.  Here the per-side count
is the argument ``w1`` and the token itself is included, so token p sees keys q
with |p - q| <= w1, clipped at the sequence ends.

Same page, §3.1 "Global Attention": attention on pre-selected locations is made
symmetric: a global token attends to all tokens and all tokens attend to it.

So token p may attend to token q iff |p - q| <= w1, or p is global, or q is
global.  Forward and backward then follow ``oracle.attention`` on this mask.
"""

from __future__ import annotations

import numpy as np


def longformer_allowed(p: int, q: int, w1: int, global_tokens) -> bool:
    """Pairwise predicate, used by brute-force pins."""
    g = set(int(x) for x in global_tokens)
    return abs(p - q) <= w1 or p in g or q in g


def longformer_mask(n: int, w1: int, global_tokens):
    """Callable row-band mask(h, p0, p1) -> bool [p1-p0, n]; identical for every head."""
    gt = np.zeros(n, dtype=bool)
    gt[np.asarray(list(global_tokens), dtype=np.int64)] = True

    def rows(h: int, p0: int, p1: int) -> np.ndarray:
        p = np.arange(p0, p1)[:, None]
        q = np.arange(n)[None, :]
        return (np.abs(p - q) <= w1) | gt[p0:p1, None] | gt[None, :]

    return rows
