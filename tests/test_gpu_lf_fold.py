"""GPU Longformer forward and backward past 16 segments per global row and per
global key column, where the partials are folded in two levels (runs of 8 to 64
consecutive partials first, over many work-groups, then the owning work-group's
merge of at most 8), against the fp64 oracle.

The oracle runs on row bands: a non-global row of [p0, p1) can only see keys in
[p0 - w1, p1 + w1) and the global keys, so the oracle gets exactly those columns
(the others are masked and contribute nothing); each global row gets every key.
dK and dV sum the bands' contributions.
"""

import numpy as np
import pytest
import torch

from block_sparse_long_bsattn_amd import _lib as B
from block_sparse_long_bsattn_amd import inputs as I
from oracle import attention as OA
from oracle import longformer as OLF
from gpu_util import BF16_TOL, max_abs, qkv, say, to_f64

pytestmark = pytest.mark.gpu


def banded_oracle(refs, n, w1, G, scale, band=512):
    qr, kr, vr, dor = refs
    bsz, heads, _, d = qr.shape
    mask = OLF.longformer_mask(n, w1, G)
    gset = np.zeros(n, dtype=bool)
    gset[G] = True
    o, dq, dk, dv = (np.zeros((bsz, heads, n, d)) for _ in range(4))
    lse = np.zeros((bsz, heads, n))
    for h in range(heads):
        hs = slice(h, h + 1)
        # (rows, columns, mask rows over those columns)
        parts = [(np.asarray(G), np.arange(n),
                  np.concatenate([mask(h, p, p + 1) for p in G]))]
        for p0 in range(0, n, band):
            p1 = min(n, p0 + band)
            rows = np.arange(p0, p1)[~gset[p0:p1]]
            cols = np.union1d(np.arange(max(0, p0 - w1), min(n, p1 + w1)), G)
            parts.append((rows, cols, mask(h, p0, p1)[rows - p0][:, cols]))
        for rows, cols, sub in parts:
            if len(rows) == 0:
                continue
            m = lambda _h, a, b, sub=sub: sub[a:b]
            args = (qr[:, hs][:, :, rows], kr[:, hs][:, :, cols], vr[:, hs][:, :, cols])
            ro, rl = OA.attention_fwd(*args, m, scale, row_chunk=1024)
            rdq, rdk, rdv = OA.attention_bwd(*args, dor[:, hs][:, :, rows], m, scale,
                                             row_chunk=1024)
            o[:, h, rows], lse[:, h, rows], dq[:, h, rows] = ro[:, 0], rl[:, 0], rdq[:, 0]
            dk[:, h, cols] += rdk[:, 0]
            dv[:, h, cols] += rdv[:, 0]
    return o, lse, dq, dk, dv


def run(n, heads, d, w1, G):
    scale = d ** -0.5
    (q, k, v, do), refs = qkv((1, heads, n, d), "bf16", (I.SEED_Q, I.SEED_K, I.SEED_V, I.SEED_DO))
    plan = B.lfattn_plan_build(n, w1, G)
    try:
        wsf_n = B.lfattn_fwd_workspace(plan, 1, heads, d)
        wsf = torch.empty(wsf_n, dtype=torch.uint8, device="cuda")
        wsb = torch.empty(B.lfattn_bwd_workspace(plan, 1, heads, d), dtype=torch.uint8,
                          device="cuda")
        o = torch.full_like(q, float("nan"))
        lse = torch.full((1, heads, n), float("nan"), dtype=torch.float32, device="cuda")
        grads = [torch.full_like(q, float("nan")) for _ in range(3)]
        outs = []
        for _ in range(2):   # the second call must give the same bits
            B.lfattn_fwd(plan, q, k, v, o, lse, wsf, scale=scale)
            B.lfattn_bwd(plan, q, k, v, o, lse, do, *grads, wsb, scale=scale)
            torch.cuda.synchronize()
            outs.append([t.clone() for t in [o, lse] + grads])
    finally:
        B.lfattn_plan_destroy(plan)
    same = all(torch.equal(a, b) for a, b in zip(*outs))
    return refs, [to_f64(t) for t in outs[1]], same, wsf_n


@pytest.mark.parametrize("case", [
    # n (257 or 513 tiles, the last one 64 tokens past a power of two of tiles), heads,
    # d, global tokens, segments of a global row, fold run length
    (16448, 2, 64, list(range(64)) + [100, 5000, 16000], 33, 8),   # two global tiles
    (16448, 1, 128, list(range(64)), 33, 8),
    (32832, 1, 64, list(range(64)), 65, 16),
])
def test_lf_folded_partials(case):
    n, heads, d, G, nseg, chunk = case
    w1, ngt = 256, (len(G) + 63) // 64
    say(f"lf folded partials n={n} H={heads} d={d} |G|={len(G)}")
    refs, got, same, wsf = run(n, heads, d, w1, G)
    nfold = -(-nseg // chunk)
    rec = 64 * d + 3 * 64
    # the forward's workspace holds the nseg partial records and the nfold folds
    assert wsf == heads * ngt * (nseg + nfold) * rec * 4
    want = banded_oracle(refs, n, w1, G, d ** -0.5)
    errs = {nm: max_abs(a, b) for nm, a, b in zip(("O", "lse", "dQ", "dK", "dV"), got, want)}
    say("   max-abs " + "  ".join(f"{a} {b:.2e}" for a, b in errs.items()) +
        f"  repeat-identical {same}")
    assert max(errs.values()) <= BF16_TOL
    assert same


def test_lf_folded_rows_sampled():
    """n = 66,048 (1032 tiles), 1 head: 129 segments per global row, folded in runs of
    32 (two load batches per run); the 64 global rows (O, lse, dQ: every partial fold)
    and a few window rows compared with the oracle."""
    n, w1, G = 66048, 256, list(range(64))
    say(f"lf folded rows sampled n={n}")
    refs, got, same, wsf = run(n, 1, 64, w1, G)
    assert wsf == (129 + 5) * (64 * 64 + 3 * 64) * 4
    qr, kr, vr, dor = refs
    mask = OLF.longformer_mask(n, w1, G)
    rng = np.random.default_rng(66048)
    rows = np.unique(np.r_[np.arange(64), 64, n - 1, rng.integers(64, n, 6)])
    ro, rl = OA.attention_fwd_rows(qr, kr, vr, mask, 1 / 8.0, 0, 0, rows)
    sub = np.concatenate([mask(0, int(p), int(p) + 1) for p in rows])
    rdq, _, _ = OA.attention_bwd(qr[:, :, rows], kr, vr, dor[:, :, rows],
                                 lambda _h, a, b: sub[a:b], 1 / 8.0)
    o, lse, dq = got[0][0, 0, rows], got[1][0, 0, rows], got[2][0, 0, rows]
    worst = max(max_abs(o, ro), max_abs(lse, rl), max_abs(dq, rdq[0, 0]))
    say(f"   sampled rows: worst max-abs {worst:.3e}  repeat-identical {same}")
    assert worst <= BF16_TOL and same
    assert all(np.isfinite(t).all() for t in got)
