"""Oracle: BigBird-ETC attention pattern (added global tokens, blocked window).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Big Bird: Transformers for Longer Sequences, §2 "global tokens": in the ETC
construction extra global tokens (such as CLS) are added to the sequence; a global
token attends to every token and every token attends to it.  App. E, the BigBird-etc
column of the MLM table: block length b = 84, g = 256 global tokens, window of 3
blocks, no random tokens (the large model doubles b to 169; the QA tables use
g = 230 ... 430 with w = 507 = 3 * 169 tokens).  The Chinese walkthrough, §2.3,
describes ETC the same way (global tokens added, e.g. CLS).

Readings:
* The sequence holds the g added global tokens first, then the n ordinary tokens,
  so it has g + n positions; the tensors are [B, H, g + n, d].
* The ordinary tokens form ceil(n / b) blocks of b (App. D eq. (13) writes
  ceil(n/b)); when b does not divide n the last block is shorter.  No padding
  token exists: a short last block simply has fewer keys.
* The window is blocked as in the ITC pattern: an ordinary token in block k sees
  the ordinary tokens of blocks k - (w-1)/2 ... k + (w-1)/2 (w odd, clipped at the
  ends) and every global token.

So p may attend to q iff p < g, or q < g, or both are ordinary and their blocks
differ by at most (w-1)/2.  Forward and backward follow ``oracle.attention``.
"""

from __future__ import annotations

import numpy as np


def _check(g: int, n: int, b: int, w: int):
    if g < 0 or n < 1 or b < 1 or w < 1 or w % 2 == 0:
        raise ValueError("need g >= 0, n >= 1, b >= 1 and an odd w >= 1")


def etc_allowed(p: int, q: int, g: int, n: int, b: int, w: int) -> bool:
    """Pairwise predicate over the g + n positions, used by brute-force pins."""
    _check(g, n, b, w)
    if p < g or q < g:
        return True
    return abs((p - g) // b - (q - g) // b) <= (w - 1) // 2


def etc_mask(g: int, n: int, b: int, w: int):
    """Callable row-band mask(h, p0, p1) -> bool [p1-p0, g+n]; same for every head."""
    _check(g, n, b, w)
    total = g + n
    half = (w - 1) // 2
    blk = np.full(total, -1, dtype=np.int64)
    blk[g:] = np.arange(n) // b

    def rows(h: int, p0: int, p1: int) -> np.ndarray:
        bp = blk[p0:p1, None]
        bq = blk[None, :]
        glob = (bp < 0) | (bq < 0)
        return glob | (np.abs(bp - bq) <= half)

    return rows
