"""Pins for the oracle's masked attention, forward and backward (CPU only).

References used here are independent of the oracle's code: PyTorch's fp64
scaled-dot-product attention and autograd (library routines), pure-Python per-pair
loops that test pattern membership with the predicates directly, closed forms
(Q = 0, V = 1), central finite differences, and the gradient-sum identities.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import layout as L
from oracle import longformer as LF


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def sdpa_full(q, k, v, scale):
    """Dense attention via torch's fp64 CPU routine: [B,H,n,d] -> [B,H,n,d]."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), scale=scale).numpy()


def bigbird_mask(n, b, heads, G, w, r, seed):
    lay = L.build_layout(n, b, heads, G, w, r, seed)
    nb = n // b
    return np.stack([L.token_mask(lay["rows"][h], nb, b) for h in range(heads)]), lay


# --- forward ------------------------------------------------------------------

def test_full_window_equals_full_attention():
    n, b, H, d = 256, 16, 2, 8
    q, k, v = rnd(1, 2, H, n, d), rnd(2, 2, H, n, d), rnd(3, 2, H, n, d)
    scale = 1 / math.sqrt(d)
    mask, _ = bigbird_mask(n, b, H, [0], 2 * (n // b) - 1, 3, 5)
    assert mask.all()
    o, lse = A.attention_fwd(q, k, v, mask, scale)
    np.testing.assert_allclose(o, sdpa_full(q, k, v, scale), rtol=0, atol=1e-12)
    s = scale * np.einsum("bhpd,bhqd->bhpq", q, k)
    ref_lse = np.log(np.exp(s).sum(-1))
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_all_global_equals_full_attention():
    n, b, H, d = 192, 32, 1, 16
    q, k, v = rnd(4, 1, H, n, d), rnd(5, 1, H, n, d), rnd(6, 1, H, n, d)
    mask, _ = bigbird_mask(n, b, H, list(range(n // b)), 1, 0, 0)
    o, _ = A.attention_fwd(q, k, v, mask, 0.3)
    np.testing.assert_allclose(o, sdpa_full(q, k, v, 0.3), rtol=0, atol=1e-12)


def test_global_rows_equal_full_rows():
    n, b, H, d = 1024, 64, 2, 64
    q, k, v = rnd(7, 1, H, n, d), rnd(8, 1, H, n, d), rnd(9, 1, H, n, d)
    G = [0, 15]
    mask, _ = bigbird_mask(n, b, H, G, 3, 3, 11)
    o, _ = A.attention_fwd(q, k, v, mask, 0.125)
    full = sdpa_full(q, k, v, 0.125)
    for g in G:
        rows = slice(g * b, (g + 1) * b)
        np.testing.assert_allclose(o[:, :, rows], full[:, :, rows], rtol=0, atol=1e-12)
    # non-global rows differ from full attention (the pattern is sparse)
    assert np.abs(o[:, :, 5 * b:6 * b] - full[:, :, 5 * b:6 * b]).max() > 1e-3


def test_probability_rows_sum_to_one_and_vanish_off_pattern():
    n, b, d = 16384, 64, 64
    lay = L.build_layout(n, b, 1, [0, 255], 3, 3, 0x5EED)
    q, k = rnd(10, 512, d), rnd(11, n, d)
    rows = np.r_[0:128, 4096:4224, n - 256:n]      # global, interior and last blocks
    qm = np.concatenate([q[:128], q[128:256], q[256:512]])
    mrows = np.zeros((len(rows), n), dtype=bool)
    for t, p in enumerate(rows):
        mrows[t] = np.isin(np.arange(n) // b, lay["rows"][0][p // b])
    P, _ = A.attention_probs(qm, k, mrows, 1 / 8)
    np.testing.assert_allclose(P.sum(1), 1.0, rtol=0, atol=1e-12)
    assert (P[~mrows] == 0).all()
    assert (P[mrows] > 0).all()


def brute_force_bigbird(q, k, v, scale, b, G, w, r, seed, h):
    """Per-pair loop: key q_ is allowed for query p iff block(q_) is global, or
    block(p) is global, or |block(p) - block(q_)| <= (w-1)/2, or block(q_) is one of
    the random blocks drawn for block(p)."""
    n, d = q.shape
    nb = n // b
    out = np.zeros((n, d))
    lse = np.zeros(n)
    for p in range(n):
        bp = p // b
        rset = set(L.random_blocks(h, bp, nb, G, w, r, seed)) if bp not in G else set()
        scores = []
        for qq in range(n):
            bq = qq // b
            ok = (bq in G) or (bp in G) or abs(bp - bq) <= (w - 1) // 2 or (bq in rset)
            if ok:
                scores.append((qq, scale * sum(q[p, c] * k[qq, c] for c in range(d))))
        m = max(s for _, s in scores)
        z = sum(math.exp(s - m) for _, s in scores)
        for qq, s in scores:
            out[p] += math.exp(s - m) / z * v[qq]
        lse[p] = m + math.log(z)
    return out, lse


@pytest.mark.parametrize("b,G,w,r", [(4, [0], 3, 2), (2, [1, 5], 1, 3), (1, [], 3, 4),
                                     (4, [3], 5, 1)])
def test_brute_force_tiny(b, G, w, r):
    nb = 8 if b > 1 else 16
    n, d, H, seed = nb * b, 4, 2, 77
    q, k, v = rnd(12, 1, H, n, d), rnd(13, 1, H, n, d), rnd(14, 1, H, n, d)
    mask, _ = bigbird_mask(n, b, H, G, w, r, seed)
    o, lse = A.attention_fwd(q, k, v, mask, 0.7)
    for h in range(H):
        bo, bl = brute_force_bigbird(q[0, h], k[0, h], v[0, h], 0.7, b, G, w, r, seed, h)
        np.testing.assert_allclose(o[0, h], bo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, h], bl, rtol=0, atol=1e-12)


def test_zero_queries_closed_form():
    """Q = 0: every allowed key scores 0, so O is the mean of the allowed values and
    LSE = ln(number of allowed keys) = ln(b * |N(i)|)."""
    n, b, H, d = 2048, 64, 2, 64
    nb = n // b
    G = [0, nb - 1]
    mask, lay = bigbird_mask(n, b, H, G, 3, 3, 3)
    q = np.zeros((1, H, n, d))
    k, v = rnd(15, 1, H, n, d), rnd(16, 1, H, n, d)
    o, lse = A.attention_fwd(q, k, v, mask, 0.125)
    for h in range(H):
        for i in range(nb):
            keys = lay["rows"][h][i]
            idx = np.concatenate([np.arange(j * b, (j + 1) * b) for j in keys])
            np.testing.assert_allclose(o[0, h, i * b:(i + 1) * b],
                                       np.broadcast_to(v[0, h, idx].mean(0), (b, d)),
                                       rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse[0, h, i * b:(i + 1) * b],
                                       math.log(b * len(keys)), rtol=0, atol=1e-13)


def test_unit_values_give_unit_output():
    n, b, H, d = 1024, 64, 1, 64
    mask, _ = bigbird_mask(n, b, H, [0, 15], 3, 3, 4)
    q, k = rnd(17, 1, H, n, d), rnd(18, 1, H, n, d)
    o, _ = A.attention_fwd(q, k, np.ones((1, H, n, d)), mask, 0.125)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-13)


def test_row_sampler_matches_full_forward():
    n, b, H, d = 1024, 64, 2, 64
    mask, _ = bigbird_mask(n, b, H, [0, 15], 3, 3, 4)
    q, k, v = rnd(19, 2, H, n, d), rnd(20, 2, H, n, d), rnd(21, 2, H, n, d)
    o, lse = A.attention_fwd(q, k, v, mask, 0.125, row_chunk=300)
    rows = [0, 63, 64, 500, 1023]
    ro, rl = A.attention_fwd_rows(q, k, v, mask, 0.125, 1, 1, rows)
    np.testing.assert_allclose(ro, o[1, 1, rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(rl, lse[1, 1, rows], rtol=0, atol=1e-13)


# --- backward -----------------------------------------------------------------

def loss(q, k, v, dout, mask, scale):
    o, _ = A.attention_fwd(q, k, v, mask, scale)
    return float((o * dout).sum())


def test_backward_finite_differences():
    n, b, H, d = 64, 8, 2, 8
    mask, _ = bigbird_mask(n, b, H, [0], 3, 2, 9)
    q, k, v, do = (rnd(s, 1, H, n, d) for s in (22, 23, 24, 25))
    scale = 0.4
    dq, dk, dv = A.attention_bwd(q, k, v, do, mask, scale)
    eps = 1e-5
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for t in range(3):
            e = rnd(100 + 10 * which + t, 1, H, n, d)
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which] = args_p[which] + eps * e
            args_m[which] = args_m[which] - eps * e
            fd = (loss(*args_p, do, mask, scale) - loss(*args_m, do, mask, scale)) / (2 * eps)
            an = float((grad * e).sum())
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, fd, an)


def test_backward_full_pattern_matches_autograd():
    n, b, H, d = 128, 16, 2, 16
    mask, _ = bigbird_mask(n, b, H, [], 2 * (n // b) - 1, 0, 0)
    assert mask.all()
    q, k, v, do = (rnd(s, 2, H, n, d) for s in (26, 27, 28, 29))
    scale = 0.25
    dq, dk, dv = A.attention_bwd(q, k, v, do, mask, scale)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.softmax(scale * tq @ tk.transpose(-1, -2), dim=-1) @ tv
    o.backward(torch.tensor(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)


def test_backward_sum_identities():
    """Rows of P sum to 1, so the dV rows sum to the dO rows; rows of dS sum to 0,
    so the dK rows sum to zero."""
    n, b, H, d = 1024, 64, 2, 64
    mask, _ = bigbird_mask(n, b, H, [0, 15], 3, 3, 31)
    q, k, v, do = (rnd(s, 1, H, n, d) for s in (30, 31, 32, 33))
    dq, dk, dv = A.attention_bwd(q, k, v, do, mask, 0.125, row_chunk=256)
    np.testing.assert_allclose(dv.sum(2), do.sum(2), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dk.sum(2), 0.0, rtol=0, atol=1e-10)


def test_backward_row_chunking_is_invisible():
    n, b, H, d = 512, 64, 1, 32
    mask, _ = bigbird_mask(n, b, H, [0, 7], 3, 3, 2)
    q, k, v, do = (rnd(s, 1, H, n, d) for s in (34, 35, 36, 37))
    a = A.attention_bwd(q, k, v, do, mask, 0.2, row_chunk=512)
    c = A.attention_bwd(q, k, v, do, mask, 0.2, row_chunk=100)
    for x, y in zip(a, c):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-12)


# --- planted mistakes: each pin above catches a plausible slip -----------------

def test_pins_catch_planted_mistakes():
    n, b, H, d = 64, 8, 1, 8
    q, k, v = rnd(40, 1, H, n, d), rnd(41, 1, H, n, d), rnd(42, 1, H, n, d)
    G, w, r, seed = [1], 3, 2, 5
    mask, _ = bigbird_mask(n, b, H, G, w, r, seed)
    bo, _ = brute_force_bigbird(q[0, 0], k[0, 0], v[0, 0], 0.5, b, G, w, r, seed, 0)

    # transposed mask
    o_t, _ = A.attention_fwd(q, k, v, mask.transpose(0, 2, 1), 0.5)
    assert np.abs(o_t[0, 0] - bo).max() > 1e-3
    # dropped scale
    o_s, _ = A.attention_fwd(q, k, v, mask, 1.0)
    assert np.abs(o_s[0, 0] - bo).max() > 1e-3
    # wrong Fisher-Yates modulus (u mod m instead of u mod (m - t))
    def bad_random(h, i, nb_, G_, w_, r_, seed_):
        excl = set(G_) | set(L.window_blocks(i, nb_, w_))
        cand = [j for j in range(nb_) if j not in excl]
        m = len(cand)
        for t in range(min(r_, m)):
            u = L.splitmix64(seed_, (h * nb_ + i) * r_ + t + 1)
            s = (t + u % m) % m
            cand[t], cand[s] = cand[s], cand[t]
        return cand[:min(r_, m)]
    from conftest import read_golden
    seed0, nb0, w0, r0, rand0, _ = read_golden("layout_row0.txt")[0]
    assert bad_random(0, 0, int(nb0), [], int(w0), int(r0), int(seed0)) != \
        [int(x) for x in rand0.split(",")]
    # flipped sign in the softmax gradient
    dq, dk, dv = A.attention_bwd(q, k, v, v, mask, 0.5)
    bad = -dq
    e = rnd(43, 1, H, n, d)
    eps = 1e-5
    fd = (loss(q + eps * e, k, v, v, mask, 0.5) - loss(q - eps * e, k, v, v, mask, 0.5)) / (2 * eps)
    assert abs(fd - float((dq * e).sum())) < 1e-7
    assert abs(fd - float((bad * e).sum())) > 1e-4


# --- Longformer ----------------------------------------------------------------

def test_longformer_full_window_is_full_attention():
    n, H, d = 200, 2, 16
    q, k, v = rnd(50, 1, H, n, d), rnd(51, 1, H, n, d), rnd(52, 1, H, n, d)
    o, _ = A.attention_fwd(q, k, v, LF.longformer_mask(n, n, []), 0.25)
    np.testing.assert_allclose(o, sdpa_full(q, k, v, 0.25), rtol=0, atol=1e-12)


def test_longformer_global_rows_are_full_rows():
    n, H, d = 1024, 2, 64
    q, k, v = rnd(53, 1, H, n, d), rnd(54, 1, H, n, d), rnd(55, 1, H, n, d)
    G = list(range(0, 16)) + [500, 777]
    o, _ = A.attention_fwd(q, k, v, LF.longformer_mask(n, 64, G), 0.125)
    full = sdpa_full(q, k, v, 0.125)
    np.testing.assert_allclose(o[:, :, G], full[:, :, G], rtol=0, atol=1e-12)


def test_longformer_brute_force_tiny():
    n, H, d, w1 = 40, 1, 3, 4
    G = [0, 17]
    q, k, v = rnd(56, 1, H, n, d), rnd(57, 1, H, n, d), rnd(58, 1, H, n, d)
    o, lse = A.attention_fwd(q, k, v, LF.longformer_mask(n, w1, G), 0.9)
    for p in range(n):
        keys = [t for t in range(n) if LF.longformer_allowed(p, t, w1, G)]
        s = [0.9 * sum(q[0, 0, p, c] * k[0, 0, t, c] for c in range(d)) for t in keys]
        m = max(s)
        z = sum(math.exp(x - m) for x in s)
        ref = sum(math.exp(x - m) / z * v[0, 0, t] for x, t in zip(s, keys))
        np.testing.assert_allclose(o[0, 0, p], ref, rtol=0, atol=1e-12)
        assert abs(lse[0, 0, p] - (m + math.log(z))) < 1e-12


def test_longformer_pair_count_closed_form():
    """n = 4096, 256 per side, global tokens 0..63: 64 full rows; rows 64..319 see
    p + 257 keys; rows 320..3839 see 513 + 64; rows 3840..4095 see 4416 - p."""
    n, w1 = 4096, 256
    f = LF.longformer_mask(n, w1, range(64))
    counts = np.concatenate([f(0, p0, p0 + 512).sum(1) for p0 in range(0, n, 512)])
    p = np.arange(n)
    expect = np.where(p < 64, n, np.where(p < 320, p + 257, np.where(p < 3840, 577, 4416 - p)))
    assert (counts == expect).all()
    assert counts.sum() == 2_522_816


def test_longformer_zero_queries_closed_form():
    n, H, d, w1 = 512, 1, 64, 32
    G = [0, 1, 2, 300]
    k, v = rnd(59, 1, H, n, d), rnd(60, 1, H, n, d)
    o, lse = A.attention_fwd(np.zeros((1, H, n, d)), k, v, LF.longformer_mask(n, w1, G), 0.125)
    for p in range(n):
        keys = sorted({t for t in range(max(0, p - w1), min(n, p + w1 + 1))} | set(G)) \
            if p not in G else list(range(n))
        np.testing.assert_allclose(o[0, 0, p], v[0, 0, keys].mean(0), rtol=0, atol=1e-13)
        assert abs(lse[0, 0, p] - math.log(len(keys))) < 1e-13


def test_longformer_backward_finite_differences():
    """The backward the Longformer GPU gradient is checked against, pinned by central
    differences of the forward on a tiny band + scattered-global pattern."""
    n, H, d, w1 = 48, 1, 6, 3
    G = [0, 29]
    mask = LF.longformer_mask(n, w1, G)
    q, k, v, do = (rnd(s, 1, H, n, d) for s in (61, 62, 63, 64))
    scale = 0.5
    dq, dk, dv = A.attention_bwd(q, k, v, do, mask, scale)

    def loss(q_, k_, v_):
        o, _ = A.attention_fwd(q_, k_, v_, mask, scale)
        return float((o * do).sum())

    eps = 1e-5
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for t in range(3):
            e = rnd(200 + 10 * which + t, 1, H, n, d)
            plus, minus = [q, k, v], [q, k, v]
            plus[which] = plus[which] + eps * e
            minus[which] = minus[which] - eps * e
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            an = float((grad * e).sum())
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, fd, an)


def test_longformer_backward_full_window_matches_autograd():
    n, H, d = 96, 2, 16
    q, k, v, do = (rnd(s, 1, H, n, d) for s in (65, 66, 67, 68))
    dq, dk, dv = A.attention_bwd(q, k, v, do, LF.longformer_mask(n, n, [5]), 0.25)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.softmax(0.25 * tq @ tk.transpose(-1, -2), dim=-1) @ tv
    o.backward(torch.tensor(do))
    for a, b in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(a, b.grad.numpy(), rtol=0, atol=1e-12)
