"""Pins for the oracle's BigBird-ETC pattern (CPU only).

References independent of ``oracle.etc``: a per-block closed form of the attended
pairs, the ITC pattern of ``oracle.layout`` (written separately, from the block
definitions) in the case where the added tokens fill whole 64-blocks, torch's fp64
scaled-dot-product attention when the window covers every block, pure-Python
per-pair loops, the Q = 0 closed form over keys enumerated block by block, and
central finite differences for the backward.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import etc as E
from oracle import layout as L


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def block_sizes(n, b):
    nb = -(-n // b)
    return [min(b, n - b * j) for j in range(nb)]


def pairs_closed_form(g, n, b, w):
    """g full rows of g + n keys; an ordinary token of block k sees the g global
    tokens and the tokens of blocks max(0, k-h) .. min(nb-1, k+h)."""
    sz = block_sizes(n, b)
    nb, h = len(sz), (w - 1) // 2
    total = g * (g + n)
    for k in range(nb):
        win = sum(sz[max(0, k - h):min(nb - 1, k + h) + 1])
        total += sz[k] * (g + win)
    return total


@pytest.mark.parametrize("g,n,b,w", [
    (256, 4096, 84, 3),      # base ETC (App. E MLM table)
    (430, 4096, 169, 3),     # large ETC, WikiHop global count
    (230, 4096, 169, 3),
    (0, 1000, 84, 5),
    (7, 100, 13, 1),
])
def test_pair_count_closed_form(g, n, b, w):
    m = E.etc_mask(g, n, b, w)
    N = g + n
    counts = sum(int(m(0, p0, min(N, p0 + 512)).sum()) for p0 in range(0, N, 512))
    assert counts == pairs_closed_form(g, n, b, w)


@pytest.mark.parametrize("gm,nb,w", [(1, 8, 3), (2, 6, 5), (0, 5, 3), (3, 4, 1)])
def test_whole_64_blocks_of_added_tokens_equal_the_itc_pattern(gm, nb, w):
    """g = 64*gm added tokens, b = 64: ETC equals the ITC layout of the g + n tokens
    with global blocks 0..gm-1 and no random blocks (those blocks' rows are full, and
    every row sees them, so the window reaching into them changes nothing)."""
    g, n, b = 64 * gm, 64 * nb, 64
    lay = L.build_layout(g + n, b, 1, list(range(gm)), w, 0, 1)
    itc = L.token_mask(lay["rows"][0], gm + nb, b)
    etc = E.etc_mask(g, n, b, w)(0, 0, g + n)
    assert np.array_equal(itc, etc)


def test_window_over_every_block_is_full_attention():
    g, n, b, H, d = 5, 120, 17, 2, 8
    q, k, v = rnd(1, 1, H, g + n, d), rnd(2, 1, H, g + n, d), rnd(3, 1, H, g + n, d)
    o, _ = A.attention_fwd(q, k, v, E.etc_mask(g, n, b, 2 * (n // b) + 3), 0.3)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=0.3).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_brute_force_tiny():
    g, n, b, w, d = 3, 37, 5, 3, 3
    N = g + n
    q, k, v = rnd(4, 1, 1, N, d), rnd(5, 1, 1, N, d), rnd(6, 1, 1, N, d)
    o, lse = A.attention_fwd(q, k, v, E.etc_mask(g, n, b, w), 0.7)
    for p in range(N):
        keys = [t for t in range(N) if E.etc_allowed(p, t, g, n, b, w)]
        s = [0.7 * sum(q[0, 0, p, c] * k[0, 0, t, c] for c in range(d)) for t in keys]
        mx = max(s)
        z = sum(math.exp(x - mx) for x in s)
        ref = sum(math.exp(x - mx) / z * v[0, 0, t] for x, t in zip(s, keys))
        np.testing.assert_allclose(o[0, 0, p], ref, rtol=0, atol=1e-12)
        assert abs(lse[0, 0, p] - (mx + math.log(z))) < 1e-12


@pytest.mark.parametrize("g,n,b,w", [(10, 200, 23, 3), (0, 130, 64, 3), (64, 300, 84, 5)])
def test_zero_queries_closed_form(g, n, b, w):
    """Q = 0: each row is the mean of V over its keys, the keys listed block by block
    (global tokens, then the ordinary blocks of the window)."""
    N, dh = g + n, 4
    k, v = rnd(7, 1, 1, N, dh), rnd(8, 1, 1, N, dh)
    o, lse = A.attention_fwd(np.zeros((1, 1, N, dh)), k, v, E.etc_mask(g, n, b, w), 0.125)
    nb, h = -(-n // b), (w - 1) // 2
    for p in range(N):
        if p < g:
            keys = list(range(N))
        else:
            kb = (p - g) // b
            keys = list(range(g))
            for j in range(max(0, kb - h), min(nb - 1, kb + h) + 1):
                keys += list(range(g + b * j, min(g + n, g + b * (j + 1))))
        np.testing.assert_allclose(o[0, 0, p], v[0, 0, keys].mean(0), rtol=0, atol=1e-13)
        assert abs(lse[0, 0, p] - math.log(len(keys))) < 1e-13


def test_backward_finite_differences():
    g, n, b, w, H, d = 4, 45, 7, 3, 1, 5
    mask = E.etc_mask(g, n, b, w)
    q, k, v, do = (rnd(s, 1, H, g + n, d) for s in (9, 10, 11, 12))
    dq, dk, dv = A.attention_bwd(q, k, v, do, mask, 0.5)

    def loss(q_, k_, v_):
        o, _ = A.attention_fwd(q_, k_, v_, mask, 0.5)
        return float((o * do).sum())

    eps = 1e-5
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        e = rnd(20 + which, 1, H, g + n, d)
        plus, minus = [q, k, v], [q, k, v]
        plus[which] = plus[which] + eps * e
        minus[which] = minus[which] - eps * e
        fd = (loss(*plus) - loss(*minus)) / (2 * eps)
        an = float((grad * e).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, fd, an)


def test_bad_arguments_rejected():
    for args in ((-1, 10, 4, 3), (0, 0, 4, 3), (0, 10, 0, 3), (0, 10, 4, 2), (0, 10, 4, 0)):
        with pytest.raises(ValueError):
            E.etc_mask(*args)


def test_pins_catch_planted_mistakes():
    """A window of w blocks on each side, and block indices taken without removing
    the g added tokens, both fail the pins above."""
    g, n, b, w = 256, 4096, 84, 3
    blk = np.full(g + n, -1)
    blk[g:] = np.arange(n) // b
    N = g + n

    def count(rows):
        return sum(int(rows(p0, min(N, p0 + 512)).sum()) for p0 in range(0, N, 512))

    def wide(p0, p1):
        bp, bq = blk[p0:p1, None], blk[None, :]
        return (bp < 0) | (bq < 0) | (np.abs(bp - bq) <= w)
    assert count(wide) != pairs_closed_form(g, n, b, w)

    g3, n3, b3 = 10, 100, 16          # g not a whole block
    pos = np.arange(g3 + n3)
    bad_blk = np.where(pos < g3, -1, pos // b3)   # forgot to subtract g
    bp, bq = bad_blk[:, None], bad_blk[None, :]
    bad = (bp < 0) | (bq < 0) | (np.abs(bp - bq) <= 1)
    assert int(bad.sum()) != pairs_closed_form(g3, n3, b3, 3)
