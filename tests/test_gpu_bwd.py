"""GPU block-sparse backward vs the fp64 oracle's exact gradient."""

import math

import numpy as np
import pytest
import torch

from block_sparse_long_bsattn_amd import _lib as B
from block_sparse_long_bsattn_amd import inputs as I
from oracle import attention as OA
from gpu_util import BF16_TOL, max_abs, qkv, say, to_f64
from test_gpu_fwd import oracle_mask

pytestmark = pytest.mark.gpu


def run_bwd(n, heads, bsz, G, w, r, seed):
    shape = (bsz, heads, n, 64)
    (q, k, v, do), (qr, kr, vr, dor) = qkv(shape, "bf16",
                                          (I.SEED_Q, I.SEED_K, I.SEED_V, I.SEED_DO))
    h = B.bsattn_layout_build(n, 64, heads, G, w, r, seed)
    try:
        o = torch.empty_like(q)
        lse = torch.empty((bsz, heads, n), dtype=torch.float32, device="cuda")
        wsf = torch.empty(max(1, B.bsattn_fwd_workspace(h, bsz)), dtype=torch.uint8, device="cuda")
        wsb = torch.empty(max(1, B.bsattn_bwd_workspace(h, bsz)), dtype=torch.uint8, device="cuda")
        B.bsattn_fwd(h, q, k, v, o, lse, wsf)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        B.bsattn_bwd(h, q, k, v, o, lse, do, dq, dk, dv, wsb)
        torch.cuda.synchronize()
    finally:
        B.bsattn_layout_destroy(h)
    return (qr, kr, vr, dor), (to_f64(dq), to_f64(dk), to_f64(dv))


@pytest.mark.parametrize("case", [
    (1024, 2, 2, [0, 15], 3, 3),      # split global rows and columns
    (768, 2, 1, [0, 11], 3, 3),       # ragged last segment
    (512, 1, 2, [0, 7], 3, 3),        # unsplit
    (640, 2, 1, [], 3, 4),            # no global blocks
    (64, 1, 2, [0], 1, 3),            # single block
    (576, 2, 1, [4], 5, 2),           # interior global block, wider window
    (1536, 1, 1, [0, 5, 23], 3, 20),  # many random blocks
    (6400, 1, 1, [0, 99], 3, 3),      # 100 blocks: dK/dV order from 2-word bitmaps
    (9600, 1, 1, [0, 149], 3, 5),     # 150 blocks: 4-word bitmaps
])
def test_bwd_full_compare(case):
    n, heads, bsz, G, w, r = case
    say(f"bwd full-compare n={n} H={heads} B={bsz} G={G} w={w} r={r}")
    (qr, kr, vr, dor), got = run_bwd(n, heads, bsz, G, w, r, 21)
    mask, _ = oracle_mask(n, heads, G, w, r, 21)
    ref = OA.attention_bwd(qr, kr, vr, dor, mask, 1 / 8.0)
    errs = [max_abs(a, b) for a, b in zip(got, ref)]
    say(f"   max-abs dQ {errs[0]:.3e} dK {errs[1]:.3e} dV {errs[2]:.3e}")
    assert max(errs) <= BF16_TOL


def test_bwd_full_size_sampled():
    """batch 4, 12 heads, n = 4096, G = {0, 63}, w = 3, r = 3 (the training-step
    workload, run as the benchmark runs it: the forward writes the rounding residual
    of O and the backward takes it): the whole job runs on the GPU.  Three (batch, head) slices are
    compared in full with the oracle (O, lse, dQ, dK, dV); in every one of the 48
    slices, sampled rows of O, lse and dQ, and dK, dV of two non-global key blocks
    (the oracle run on exactly the query rows that attend to them, so those
    gradients are exact); and per slice the sum identities (dV rows sum to the dO
    rows, dK rows to zero), which cover the global columns."""
    n, heads, bsz, G = 4096, 12, 4, [0, 63]
    say("fwd+bwd full-size n=4096 H=12 B=4")
    shape = (bsz, heads, n, 64)
    (q, k, v, do), (qr, kr, vr, dor) = qkv(shape, "bf16",
                                          (I.SEED_Q, I.SEED_K, I.SEED_V, I.SEED_DO))
    h = B.bsattn_layout_build(n, 64, heads, G, 3, 3, I.SEED_LAYOUT)
    try:
        o = torch.empty_like(q)
        lse = torch.empty((bsz, heads, n), dtype=torch.float32, device="cuda")
        wsf = torch.empty(max(1, B.bsattn_fwd_workspace(h, bsz)), dtype=torch.uint8, device="cuda")
        wsb = torch.empty(max(1, B.bsattn_bwd_workspace(h, bsz)), dtype=torch.uint8, device="cuda")
        o_lo = torch.empty_like(q)
        B.bsattn_fwd(h, q, k, v, o, lse, wsf, o_lo=o_lo)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        B.bsattn_bwd(h, q, k, v, o, lse, do, dq, dk, dv, wsb, o_lo=o_lo)
        torch.cuda.synchronize()
    finally:
        B.bsattn_layout_destroy(h)
    o, lse, dq, dk, dv = (to_f64(t) for t in (o, lse, dq, dk, dv))
    mask, lay = oracle_mask(n, heads, G, 3, 3, I.SEED_LAYOUT)
    worst = 0.0
    for bi, hh in ((0, 0), (1, 5), (3, 11)):
        sl = (slice(bi, bi + 1), slice(hh, hh + 1))
        mh = lambda _h, p0, p1, hh=hh: mask(hh, p0, p1)
        ro, rl = OA.attention_fwd(qr[sl], kr[sl], vr[sl], mh, 1 / 8.0, row_chunk=1024)
        worst = max(worst, max_abs(o[bi, hh], ro[0, 0]), max_abs(lse[bi, hh], rl[0, 0]))
        ref = OA.attention_bwd(qr[sl], kr[sl], vr[sl], dor[sl], mh, 1 / 8.0, row_chunk=1024)
        for a, b in zip((dq, dk, dv), ref):
            worst = max(worst, max_abs(a[bi, hh], b[0, 0]))
    say(f"   three whole slices: worst max-abs {worst:.3e}")
    rng = np.random.default_rng(4096)
    cp, cs = lay["csc_ptr"], lay["csc_idx"]
    nb = lay["nb"]
    worst_s = worst_id = 0.0
    for bi in range(bsz):
        for hh in range(heads):
            sub = (slice(bi, bi + 1), slice(hh, hh + 1))
            rows = np.unique(np.r_[0, 63, 64, 65, n - 65, n - 1, rng.integers(0, n, 6)])
            ro, rl = OA.attention_fwd_rows(qr, kr, vr, mask, 1 / 8.0, bi, hh, rows)
            worst_s = max(worst_s, max_abs(o[bi, hh, rows], ro), max_abs(lse[bi, hh, rows], rl))

            def rows_mask(_h, p0, p1, sel, hh=hh):
                return np.concatenate([mask(hh, int(p), int(p) + 1) for p in sel[p0:p1]])
            rdq, _, _ = OA.attention_bwd(qr[sub][:, :, rows], kr[sub], vr[sub],
                                         dor[sub][:, :, rows],
                                         lambda _h, p0, p1: rows_mask(_h, p0, p1, rows),
                                         1 / 8.0)
            worst_s = max(worst_s, max_abs(dq[bi, hh, rows], rdq[0, 0]))
            cols = [j for j in rng.choice(nb, 6, replace=False) if j not in G][:2]
            base = hh * nb
            for j in cols:
                qblks = cs[cp[base + j]:cp[base + j + 1]]
                sel = (np.asarray(qblks)[:, None] * 64 + np.arange(64)).ravel()
                _, rdk, rdv = OA.attention_bwd(qr[sub][:, :, sel], kr[sub], vr[sub],
                                               dor[sub][:, :, sel],
                                               lambda _h, p0, p1, sel=sel: rows_mask(_h, p0, p1, sel),
                                               1 / 8.0, row_chunk=1024)
                kr_ = slice(64 * j, 64 * j + 64)
                worst_s = max(worst_s, max_abs(dk[bi, hh, kr_], rdk[0, 0, kr_]),
                              max_abs(dv[bi, hh, kr_], rdv[0, 0, kr_]))
            worst_id = max(worst_id, max_abs(dv[bi, hh].sum(0), dor[bi, hh].sum(0)),
                           float(np.max(np.abs(dk[bi, hh].sum(0)))))
    say(f"   every slice, sampled: worst max-abs {worst_s:.3e}; sum identities {worst_id:.3e}")
    assert worst <= BF16_TOL
    assert worst_s <= BF16_TOL
    assert worst_id <= 1.0      # sums over 4096 rows of bf16-rounded values


def test_fwd_bwd_max_blocks_sampled():
    """The largest layout (4096 blocks, n = 262,144), 1 head, forward and backward:
    sampled rows of O, lse and dQ (the two global rows among them), and dK, dV of two
    non-global key blocks (the oracle run on exactly the query rows that see them)."""
    n, G, seed = 64 * 4096, [0, 4095], 92
    say(f"fwd+bwd max blocks n={n}")
    shape = (1, 1, n, 64)
    (q, k, v, do), (qr, kr, vr, dor) = qkv(shape, "bf16",
                                          (I.SEED_Q, I.SEED_K, I.SEED_V, I.SEED_DO))
    h = B.bsattn_layout_build(n, 64, 1, G, 3, 3, seed)
    try:
        o = torch.empty_like(q)
        lse = torch.empty((1, 1, n), dtype=torch.float32, device="cuda")
        wsf = torch.empty(max(1, B.bsattn_fwd_workspace(h, 1)), dtype=torch.uint8, device="cuda")
        wsb = torch.empty(max(1, B.bsattn_bwd_workspace(h, 1)), dtype=torch.uint8, device="cuda")
        o_lo = torch.empty_like(q)
        B.bsattn_fwd(h, q, k, v, o, lse, wsf, o_lo=o_lo)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        B.bsattn_bwd(h, q, k, v, o, lse, do, dq, dk, dv, wsb, o_lo=o_lo)
        torch.cuda.synchronize()
    finally:
        B.bsattn_layout_destroy(h)
    o, lse, dq, dk, dv = (to_f64(t) for t in (o, lse, dq, dk, dv))
    mask, lay = oracle_mask(n, 1, G, 3, 3, seed)
    rng = np.random.default_rng(262144)
    rows = np.unique(np.r_[0, 63, 64, n - 65, n - 64, n - 1, rng.integers(0, n, 6)])
    ro, rl = OA.attention_fwd_rows(qr, kr, vr, mask, 1 / 8.0, 0, 0, rows)
    worst = max(max_abs(o[0, 0, rows], ro), max_abs(lse[0, 0, rows], rl))

    def rows_mask(p0, p1, sel):
        return np.concatenate([mask(0, int(p), int(p) + 1) for p in sel[p0:p1]])
    rdq, _, _ = OA.attention_bwd(qr[:, :, rows], kr, vr, dor[:, :, rows],
                                 lambda _h, p0, p1: rows_mask(p0, p1, rows), 1 / 8.0)
    worst = max(worst, max_abs(dq[0, 0, rows], rdq[0, 0]))
    cp, cs = lay["csc_ptr"], lay["csc_idx"]
    for j in (1234, 3000):
        sel = (np.asarray(cs[cp[j]:cp[j + 1]])[:, None] * 64 + np.arange(64)).ravel()
        _, rdk, rdv = OA.attention_bwd(qr[:, :, sel], kr, vr, dor[:, :, sel],
                                       lambda _h, p0, p1, sel=sel: rows_mask(p0, p1, sel),
                                       1 / 8.0, row_chunk=128)
        kr_ = slice(64 * j, 64 * j + 64)
        worst = max(worst, max_abs(dk[0, 0, kr_], rdk[0, 0, kr_]),
                    max_abs(dv[0, 0, kr_], rdv[0, 0, kr_]))
    say(f"   sampled rows and two key blocks: worst max-abs {worst:.3e}")
    assert worst <= BF16_TOL
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()


def test_bwd_gradient_sum_identities():
    """Rows of P sum to 1 and rows of dS to 0, so per (batch, head) the dV rows sum
    to the dO rows and the dK rows sum to zero."""
    n, heads, bsz = 2048, 2, 2
    (qr, kr, vr, dor), (dq, dk, dv) = run_bwd(n, heads, bsz, [0, 31], 3, 3, 8)
    e_v = max_abs(dv.sum(2), dor.sum(2))
    e_k = float(np.max(np.abs(dk.sum(2))))
    say(f"   sum identities: dV {e_v:.3e} dK {e_k:.3e}")
    assert e_v <= 0.5 and e_k <= 0.5      # sums over 2048 rows of bf16-rounded values


def test_bwd_deterministic():
    _, a = run_bwd(1024, 2, 2, [0, 15], 3, 3, 4)
    _, b = run_bwd(1024, 2, 2, [0, 15], 3, 3, 4)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("redraw", [False, True])
def test_fwd_bwd_layout_over_512_blocks_sampled(redraw):
    """n = 64 * 600 (a layout built by the two-kernel path, whose work-item records
    come from a kernel of their own), 2 heads, G = {0, 7, 599}, as built or redrawn
    with another seed.  Forward on sampled rows; dQ, dK and dV of three non-global
    key blocks per head, with the oracle run on exactly the query rows that attend
    to them (the only rows with a non-zero probability there), so those gradients
    are exact; the sum identities over all rows cover the global columns."""
    n, heads, bsz, G = 64 * 600, 2, 1, [0, 7, 599]
    seed = 32 if redraw else 31
    say(f"fwd+bwd n=38400 H=2 (more than 512 blocks), redraw={redraw}")
    shape = (bsz, heads, n, 64)
    (q, k, v, do), (qr, kr, vr, dor) = qkv(shape, "bf16",
                                          (I.SEED_Q, I.SEED_K, I.SEED_V, I.SEED_DO))
    h = B.bsattn_layout_build(n, 64, heads, G, 3, 3, 31)
    try:
        if redraw:
            B.bsattn_layout_rebuild(h, seed)
        o = torch.empty_like(q)
        lse = torch.empty((bsz, heads, n), dtype=torch.float32, device="cuda")
        wsf = torch.empty(max(1, B.bsattn_fwd_workspace(h, bsz)), dtype=torch.uint8, device="cuda")
        wsb = torch.empty(max(1, B.bsattn_bwd_workspace(h, bsz)), dtype=torch.uint8, device="cuda")
        B.bsattn_fwd(h, q, k, v, o, lse, wsf)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        B.bsattn_bwd(h, q, k, v, o, lse, do, dq, dk, dv, wsb)
        torch.cuda.synchronize()
    finally:
        B.bsattn_layout_destroy(h)
    o, lse, dq, dk, dv = (to_f64(t) for t in (o, lse, dq, dk, dv))
    mask, lay = oracle_mask(n, heads, G, 3, 3, seed)
    rng = np.random.default_rng(600)
    worst = 0.0
    for hh in range(heads):
        rows = np.unique(np.r_[0, 7 * 64 + 5, 599 * 64 + 63, 64, n - 65, rng.integers(0, n, 6)])
        ro, rl = OA.attention_fwd_rows(qr, kr, vr, mask, 1 / 8.0, 0, hh, rows)
        worst = max(worst, max_abs(o[0, hh, rows], ro), max_abs(lse[0, hh, rows], rl))
        cp, cs = lay["csc_ptr"], lay["csc_idx"]
        base = hh * lay["nb"]
        cols = [j for j in rng.choice(lay["nb"], 8, replace=False) if j not in G][:3]
        qblks = np.unique(np.concatenate([cs[cp[base + j]:cp[base + j + 1]] for j in cols]))
        sel = (qblks[:, None] * 64 + np.arange(64)).ravel()
        sub = (slice(0, 1), slice(hh, hh + 1))

        def sub_mask(_h, p0, p1, hh=hh, sel=sel):
            return np.concatenate([mask(hh, int(p), int(p) + 1) for p in sel[p0:p1]])
        rdq, rdk, rdv = OA.attention_bwd(qr[sub][:, :, sel], kr[sub], vr[sub], dor[sub][:, :, sel],
                                         sub_mask, 1 / 8.0, row_chunk=1024)
        worst = max(worst, max_abs(dq[0, hh, sel], rdq[0, 0]))
        for j in cols:
            kr_ = slice(64 * j, 64 * j + 64)
            worst = max(worst, max_abs(dk[0, hh, kr_], rdk[0, 0, kr_]),
                        max_abs(dv[0, hh, kr_], rdv[0, 0, kr_]))
    e_v = max_abs(dv.sum(2), dor.sum(2))
    e_k = float(np.max(np.abs(dk.sum(2))))
    say(f"   worst max-abs {worst:.3e}; sum identities dV {e_v:.3e} dK {e_k:.3e}")
    assert worst <= BF16_TOL
    assert e_v <= 2.0 and e_k <= 2.0      # sums over 38400 rows of bf16-rounded values


def test_fwd_bwd_after_rebuild():
    """A layout redrawn with a new seed (bsattn_layout_rebuild rewrites the lists, the
    dK/dV order and the per-row and per-column work-item records): forward and
    backward match the oracle on the new seed's pattern."""
    n, heads, bsz, G = 1024, 2, 2, [0, 15]
    say("fwd+bwd after layout_rebuild n=1024 H=2 B=2")
    shape = (bsz, heads, n, 64)
    (q, k, v, do), (qr, kr, vr, dor) = qkv(shape, "bf16",
                                          (I.SEED_Q, I.SEED_K, I.SEED_V, I.SEED_DO))
    h = B.bsattn_layout_build(n, 64, heads, G, 3, 3, 3)
    try:
        B.bsattn_layout_rebuild(h, 0xABCDEF)
        o = torch.empty_like(q)
        lse = torch.empty((bsz, heads, n), dtype=torch.float32, device="cuda")
        wsf = torch.empty(max(1, B.bsattn_fwd_workspace(h, bsz)), dtype=torch.uint8, device="cuda")
        wsb = torch.empty(max(1, B.bsattn_bwd_workspace(h, bsz)), dtype=torch.uint8, device="cuda")
        B.bsattn_fwd(h, q, k, v, o, lse, wsf)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        B.bsattn_bwd(h, q, k, v, o, lse, do, dq, dk, dv, wsb)
        torch.cuda.synchronize()
    finally:
        B.bsattn_layout_destroy(h)
    mask, _ = oracle_mask(n, heads, G, 3, 3, 0xABCDEF)
    ro, rl = OA.attention_fwd(qr, kr, vr, mask, 1 / 8.0)
    ref = OA.attention_bwd(qr, kr, vr, dor, mask, 1 / 8.0)
    errs = [max_abs(to_f64(o), ro), max_abs(to_f64(lse), rl)] + \
        [max_abs(to_f64(a), b) for a, b in zip((dq, dk, dv), ref)]
    say("   max-abs O {:.3e} lse {:.3e} dQ {:.3e} dK {:.3e} dV {:.3e}".format(*errs))
    assert max(errs) <= BF16_TOL
