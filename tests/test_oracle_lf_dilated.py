"""Pins for the oracle's dilated and causal Longformer patterns (CPU only).

The window of §3.1 "Dilated Sliding Window" (Fig. 2(c)) is pinned by its shape:
sorted keys of a row step by d + 1 and hold min(w1, p // (d+1)) tokens before p
and min(w1, (n-1-p) // (d+1)) after it (floor division, not the oracle's modulus
test).  The receptive field statement of §3.1 is pinned through boolean matrix
powers.  Whole-class windows reduce to torch's fp64 scaled-dot-product attention
(with ``is_causal`` for the autoregressive mode) on each residue class, forward
and backward (autograd).  Q = 0 gives uniform rows over the keys enumerated as
{p + k (d+1)} together with the global tokens.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import longformer as LF


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def mask_matrix(mask, n, h=0):
    return np.asarray(mask(h, 0, n), dtype=bool)


def window_shape_ok(m, n, w1, d, causal):
    """True iff every row of m is the window of Fig. 2(c): keys spaced d + 1 apart
    around p, with the closed-form number of keys before and after p."""
    s = d + 1
    for p in range(n):
        keys = np.flatnonzero(m[p])
        if p not in keys:
            return False
        if len(keys) > 1 and not (np.diff(keys) == s).all():
            return False
        before = int((keys < p).sum())
        after = int((keys > p).sum())
        if before != min(w1, p // s):
            return False
        if after != (0 if causal else min(w1, (n - 1 - p) // s)):
            return False
    return True


@pytest.mark.parametrize("d", [0, 1, 2, 3])
@pytest.mark.parametrize("causal", [False, True])
def test_dilated_window_shape(d, causal):
    n, w1 = 150, 7
    assert window_shape_ok(mask_matrix(LF.longformer_mask(n, w1, [], d, causal), n),
                           n, w1, d, causal)


@pytest.mark.parametrize("d,causal", [(1, False), (3, False), (2, True)])
def test_receptive_field_grows_with_layers_dilation_and_window(d, causal):
    """§3.1: a stack of l layers of windows with w1 tokens per side and gaps of d
    reaches l * w1 * (d + 1) tokens on each side (one side when causal), and with
    d > 0 only tokens of the same residue modulo d + 1."""
    n, w1, layers = 400, 4, 3
    s = d + 1
    m = mask_matrix(LF.longformer_mask(n, w1, [], d, causal), n).astype(np.int64)
    reach = np.eye(n, dtype=np.int64)
    for _ in range(layers):
        reach = (m @ reach > 0).astype(np.int64)   # row p: tokens reachable from p
    p = 200
    r = np.flatnonzero(reach[p])
    span = layers * w1 * s
    assert r.min() == p - span
    assert r.max() == (p if causal else p + span)
    assert ((r - p) % s == 0).all()
    assert len(r) == (layers * w1 + 1 if causal else 2 * layers * w1 + 1)


def sdpa(q, k, v, scale, causal):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), scale=scale, is_causal=causal).numpy()


@pytest.mark.parametrize("d,causal", [(0, True), (1, False), (2, False), (3, True), (2, True)])
def test_whole_class_window_is_attention_within_each_residue_class(d, causal):
    """w1 >= n: each residue class modulo d + 1 attends to itself in full (or
    causally), and to nothing else."""
    n, H, dh, s = 121, 2, 8, d + 1
    q, k, v = rnd(70, 1, H, n, dh), rnd(71, 1, H, n, dh), rnd(72, 1, H, n, dh)
    o, _ = A.attention_fwd(q, k, v, LF.longformer_mask(n, n, [], d, causal), 0.3)
    for c in range(s):
        ref = sdpa(q[:, :, c::s], k[:, :, c::s], v[:, :, c::s], 0.3, causal)
        np.testing.assert_allclose(o[:, :, c::s], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("d,causal", [(0, True), (2, False), (1, True)])
def test_whole_class_backward_matches_autograd(d, causal):
    n, H, dh, s = 70, 1, 8, d + 1
    q, k, v, do = (rnd(sd, 1, H, n, dh) for sd in (73, 74, 75, 76))
    dq, dk, dv = A.attention_bwd(q, k, v, do, LF.longformer_mask(n, n, [], d, causal), 0.4)
    for c in range(s):
        tq, tk, tv = (torch.tensor(np.ascontiguousarray(x[:, :, c::s]), requires_grad=True)
                      for x in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.4,
                                                             is_causal=causal)
        o.backward(torch.tensor(np.ascontiguousarray(do[:, :, c::s])))
        for a, b in ((dq, tq), (dk, tk), (dv, tv)):
            np.testing.assert_allclose(a[:, :, c::s], b.grad.numpy(), rtol=0, atol=1e-12)


def test_causal_first_token_sees_itself_only():
    n, dh = 64, 8
    q, k, v = rnd(77, 1, 1, n, dh), rnd(78, 1, 1, n, dh), rnd(79, 1, 1, n, dh)
    for d in (0, 2):
        o, lse = A.attention_fwd(q, k, v, LF.longformer_mask(n, 5, [], d, True), 0.5)
        np.testing.assert_array_equal(o[0, 0, :d + 1], v[0, 0, :d + 1])
        assert abs(lse[0, 0, 0] - 0.5 * float(q[0, 0, 0] @ k[0, 0, 0])) < 1e-13


@pytest.mark.parametrize("d,G", [(1, [0, 3, 50]), (3, [10, 11, 12, 199]), (2, [])])
def test_dilated_zero_queries_closed_form(d, G):
    n, dh, w1, s = 200, 4, 6, d + 1
    k, v = rnd(80, 1, 1, n, dh), rnd(81, 1, 1, n, dh)
    o, lse = A.attention_fwd(np.zeros((1, 1, n, dh)), k, v,
                             LF.longformer_mask(n, w1, G, d), 0.125)
    for p in range(n):
        if p in G:
            keys = list(range(n))
        else:
            win = {p + j * s for j in range(-w1, w1 + 1)}
            keys = sorted({t for t in win if 0 <= t < n} | set(G))
        np.testing.assert_allclose(o[0, 0, p], v[0, 0, keys].mean(0), rtol=0, atol=1e-13)
        assert abs(lse[0, 0, p] - math.log(len(keys))) < 1e-13


def test_per_head_dilation_selects_each_heads_window():
    n, H, dh, w1 = 96, 3, 8, 5
    dil = [0, 2, 1]
    q, k, v = rnd(82, 1, H, n, dh), rnd(83, 1, H, n, dh), rnd(84, 1, H, n, dh)
    o, _ = A.attention_fwd(q, k, v, LF.longformer_mask(n, w1, [7], dil), 0.25)
    for h, d in enumerate(dil):
        m = mask_matrix(LF.longformer_mask(n, w1, [7], d), n)
        oh, _ = A.attention_fwd(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], m, 0.25)
        np.testing.assert_array_equal(o[:, h], oh[:, 0])
    # and the windows differ between heads
    assert not np.array_equal(mask_matrix(LF.longformer_mask(n, w1, [], dil), n, 0),
                              mask_matrix(LF.longformer_mask(n, w1, [], dil), n, 1))


def test_dilated_backward_finite_differences():
    n, H, dh, w1 = 40, 1, 5, 3
    for d, G, causal in ((2, [0, 17], False), (1, [], True)):
        mask = LF.longformer_mask(n, w1, G, d, causal)
        q, k, v, do = (rnd(sd, 1, H, n, dh) for sd in (85, 86, 87, 88))
        dq, dk, dv = A.attention_bwd(q, k, v, do, mask, 0.5)

        def loss(q_, k_, v_):
            o, _ = A.attention_fwd(q_, k_, v_, mask, 0.5)
            return float((o * do).sum())

        eps = 1e-5
        for which, grad in ((0, dq), (1, dk), (2, dv)):
            e = rnd(300 + which, 1, H, n, dh)
            plus, minus = [q, k, v], [q, k, v]
            plus[which] = plus[which] + eps * e
            minus[which] = minus[which] - eps * e
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            an = float((grad * e).sum())
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (d, causal, which, fd, an)


def test_causal_pattern_rejects_global_tokens():
    with pytest.raises(ValueError):
        LF.longformer_mask(128, 8, [0], 0, True)
    with pytest.raises(ValueError):
        LF.longformer_allowed(3, 1, 8, [0], 0, True)


def test_pins_catch_planted_dilation_mistakes():
    """A window spaced d apart instead of d + 1, one that drops the token itself,
    and a causal window on the wrong side all fail the pins above."""
    n, w1, d = 150, 7, 2
    p = np.arange(n)[:, None]
    q = np.arange(n)[None, :]
    delta = p - q
    wrong_stride = (delta % d == 0) & (np.abs(delta) <= w1 * d)
    assert not window_shape_ok(wrong_stride, n, w1, d, False)
    s = d + 1
    no_self = (delta % s == 0) & (np.abs(delta) <= w1 * s) & (delta != 0)
    assert not window_shape_ok(no_self, n, w1, d, False)
    wrong_side = (delta % s == 0) & (delta <= 0) & (delta >= -w1 * s)
    assert not window_shape_ok(wrong_side, n, w1, d, True)
    # the same wrong side against the library's causal attention
    H, dh = 1, 8
    qq, kk, vv = rnd(89, 1, H, n, dh), rnd(90, 1, H, n, dh), rnd(91, 1, H, n, dh)
    full_wrong = delta <= 0
    o, _ = A.attention_fwd(qq, kk, vv, full_wrong, 0.3)
    assert np.abs(o - sdpa(qq, kk, vv, 0.3, True)).max() > 1e-3


def test_plain_reading_unchanged_at_zero_dilation():
    """d = 0, not causal: the pattern of §3.1 already pinned elsewhere, the same
    boolean matrix as the predicate gives pair by pair."""
    n, w1, G = 90, 6, [4, 50]
    m = mask_matrix(LF.longformer_mask(n, w1, G, 0, False), n)
    for p in range(n):
        for t in range(n):
            assert m[p, t] == (abs(p - t) <= w1 or p in G or t in G)


# --- separate global projections (§3.1) --------------------------------------------

def gproj_torch(q, k, v, qg, kg, vg, n, w1, G, scale):
    """Independent torch formulation: two score matrices, rows chosen by a mask."""
    t = lambda x: torch.tensor(np.ascontiguousarray(x), requires_grad=True)
    tq, tk, tv, tqg, tkg, tvg = (t(x) for x in (q, k, v, qg, kg, vg))
    idx = torch.arange(n)
    win = (idx[:, None] - idx[None, :]).abs() <= w1
    gl = torch.zeros(n, dtype=torch.bool)
    gl[list(G)] = True
    allowed = win | gl[:, None] | gl[None, :]
    s_s = (tq @ tk.transpose(-1, -2)) * scale
    s_s = s_s.masked_fill(~allowed, float("-inf"))
    o_s = torch.softmax(s_s, dim=-1) @ tv
    o_g = torch.softmax((tqg @ tkg.transpose(-1, -2)) * scale, dim=-1) @ tvg
    o = torch.where(gl[None, None, :, None], o_g, o_s)
    return o, (tq, tk, tv, tqg, tkg, tvg)


def test_gproj_equal_projections_reduce_to_one_set():
    """The global projections start equal to the window ones (§3.1): then the output
    is the single-projection Longformer attention."""
    n, H, dh, w1, G = 96, 2, 8, 5, [0, 40, 95]
    q, k, v = rnd(92, 1, H, n, dh), rnd(93, 1, H, n, dh), rnd(94, 1, H, n, dh)
    o, lse = LF.longformer_gproj_fwd(q, k, v, q, k, v, n, w1, G, 0.3)
    o1, l1 = A.attention_fwd(q, k, v, LF.longformer_mask(n, w1, G), 0.3)
    np.testing.assert_allclose(o, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, l1, rtol=0, atol=1e-13)


def test_gproj_forward_and_backward_match_torch_autograd():
    n, H, dh, w1, G = 80, 2, 8, 4, [3, 17, 79]
    xs = [rnd(95 + i, 1, H, n, dh) for i in range(7)]
    q, k, v, qg, kg, vg, do = xs
    o, _ = LF.longformer_gproj_fwd(q, k, v, qg, kg, vg, n, w1, G, 0.4)
    grads = LF.longformer_gproj_bwd(q, k, v, qg, kg, vg, do, n, w1, G, 0.4)
    to, leaves = gproj_torch(q, k, v, qg, kg, vg, n, w1, G, 0.4)
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=0, atol=1e-12)
    to.backward(torch.tensor(do))
    for a, b in zip(grads, leaves):
        np.testing.assert_allclose(a, b.grad.numpy(), rtol=0, atol=1e-12)
    # the window projections get nothing from global rows and vice versa
    gl = np.zeros(n, dtype=bool)
    gl[G] = True
    assert np.all(grads[0][:, :, gl] == 0) and np.all(grads[3][:, :, ~gl] == 0)


def test_gproj_global_rows_ignore_window_projections():
    """Changing Q_s, K_s, V_s leaves the rows of global tokens unchanged, and changing
    Q_g, K_g, V_g leaves the other rows unchanged."""
    n, H, dh, w1, G = 64, 1, 4, 3, [0, 30]
    xs = [rnd(110 + i, 1, H, n, dh) for i in range(6)]
    o, _ = LF.longformer_gproj_fwd(*xs, n, w1, G, 0.5)
    o2, _ = LF.longformer_gproj_fwd(*[x + 1.0 for x in xs[:3]], *xs[3:], n, w1, G, 0.5)
    o3, _ = LF.longformer_gproj_fwd(*xs[:3], *[x - 0.5 for x in xs[3:]], n, w1, G, 0.5)
    gl = np.zeros(n, dtype=bool)
    gl[G] = True
    np.testing.assert_array_equal(o[:, :, gl], o2[:, :, gl])
    np.testing.assert_array_equal(o[:, :, ~gl], o3[:, :, ~gl])
    assert np.abs(o[:, :, ~gl] - o2[:, :, ~gl]).max() > 1e-3
    assert np.abs(o[:, :, gl] - o3[:, :, gl]).max() > 1e-3
