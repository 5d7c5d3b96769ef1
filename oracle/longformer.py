"""Oracle: Longformer token-level attention pattern.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Longformer: The Long-Document Transformer, §3.1 "Sliding Window": with window
size w every token attends to w/2 tokens on each side.  Here the per-side count
is the argument ``w1`` and the token itself is included, so token p sees keys q
with |p - q| <= w1, clipped at the sequence ends.

Same page, §3.1 "Dilated Sliding Window" and Fig. 2(c): the window may have gaps
of d tokens between the tokens it attends to.  Reading: with dilation d the
window still holds w1 tokens on each side, spaced d + 1 apart, so q is in p's
window iff p - q is a multiple of d + 1 and |p - q| <= w1 * (d + 1).  d = 0 is
the plain window (Table 12 lists dilation 0 for layers without dilation).  §3.1
allows a different dilation per head, so ``dilation`` may be one value per head.

Same page, §3.1 "Global Attention": attention on pre-selected locations is made
symmetric: a global token attends to all tokens and all tokens attend to it.

Same page, §4.1 and App. B "Character LM Hyperparameters": the kernel has an
autoregressive mode in which a token attends to a window of earlier tokens only.
Reading: with ``causal`` the window keeps its left half and the token itself,
0 <= p - q <= w1 * (d + 1); global tokens are not defined in that mode (a global
token would see later tokens), so a causal pattern with global tokens is rejected.

So token p may attend to token q iff q is in p's window, or p is global, or q is
global.  Forward and backward then follow ``oracle.attention`` on this mask.
"""

from __future__ import annotations

import numpy as np


def _check(global_tokens, causal: bool):
    g = [int(x) for x in global_tokens]
    if causal and g:
        raise ValueError("the causal window has no global tokens")
    return g


def in_window(p: int, q: int, w1: int, dilation: int = 0, causal: bool = False) -> bool:
    """Window membership of the pair (query p, key q) for one head."""
    s = dilation + 1
    delta = p - q
    if delta % s != 0:
        return False
    if causal:
        return 0 <= delta <= w1 * s
    return abs(delta) <= w1 * s


def longformer_allowed(p: int, q: int, w1: int, global_tokens, dilation: int = 0,
                       causal: bool = False) -> bool:
    """Pairwise predicate, used by brute-force pins."""
    g = set(_check(global_tokens, causal))
    return in_window(p, q, w1, dilation, causal) or p in g or q in g


def longformer_mask(n: int, w1: int, global_tokens, dilation=0, causal: bool = False):
    """Callable row-band mask(h, p0, p1) -> bool [p1-p0, n].

    ``dilation`` is one int for every head or a sequence indexed by head."""
    g = _check(global_tokens, causal)
    gt = np.zeros(n, dtype=bool)
    gt[np.asarray(g, dtype=np.int64)] = True
    per_head = not np.isscalar(dilation)

    def rows(h: int, p0: int, p1: int) -> np.ndarray:
        s = int(dilation[h] if per_head else dilation) + 1
        p = np.arange(p0, p1)[:, None]
        q = np.arange(n)[None, :]
        delta = p - q
        lo = 0 if causal else -w1 * s
        win = (delta % s == 0) & (delta >= lo) & (delta <= w1 * s)
        return win | gt[p0:p1, None] | gt[None, :]

    return rows


# --- separate global projections ---------------------------------------------------
#
# Same page, §3.1 "Linear Projections for Global Attention": one set of projections
# (Q_s, K_s, V_s) scores the sliding-window attention and another (Q_g, K_g, V_g) the
# global attention, the second set starting equal to the first.  Reading: the
# "global attention" is the attention of a global token, whose row covers every
# token; it uses Q_g for that token and K_g, V_g for all keys.  Every other row (its
# window and the global keys) uses Q_s, K_s, V_s.  Each row therefore belongs to one
# of two independent masked attentions, and O, lse and the gradients are those of
# the two problems with each row taken from its own.

def _rows_split(n: int, global_tokens):
    g = np.zeros(n, dtype=bool)
    g[np.asarray(list(global_tokens), dtype=np.int64)] = True
    return g


def longformer_gproj_fwd(q, k, v, qg, kg, vg, n: int, w1: int, global_tokens, scale: float,
                         dilation=0):
    """O and lse [B,H,n] with separate global projections (fp64)."""
    from . import attention as A
    g = _rows_split(n, global_tokens)
    o_s, l_s = A.attention_fwd(q, k, v, longformer_mask(n, w1, global_tokens, dilation), scale)
    full = np.ones((n, n), dtype=bool)
    o_g, l_g = A.attention_fwd(qg, kg, vg, full, scale)
    o = np.where(g[None, None, :, None], o_g, o_s)
    lse = np.where(g[None, None, :], l_g, l_s)
    return o, lse


def longformer_gproj_bwd(q, k, v, qg, kg, vg, dout, n: int, w1: int, global_tokens,
                         scale: float, dilation=0):
    """(dQ, dK, dV, dQ_g, dK_g, dV_g) for the loss <dout, O> of longformer_gproj_fwd:
    each problem sees the output gradient of its own rows only."""
    from . import attention as A
    g = _rows_split(n, global_tokens)
    dout = np.asarray(dout, dtype=np.float64)
    d_s = np.where(g[None, None, :, None], 0.0, dout)
    d_g = np.where(g[None, None, :, None], dout, 0.0)
    dq, dk, dv = A.attention_bwd(q, k, v, d_s, longformer_mask(n, w1, global_tokens, dilation),
                                 scale)
    full = np.ones((n, n), dtype=bool)
    dqg, dkg, dvg = A.attention_bwd(qg, kg, vg, d_g, full, scale)
    return dq, dk, dv, dqg, dkg, dvg
