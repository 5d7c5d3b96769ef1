"""GPU block-sparse forward and backward with more than 16 segments per global row
and column, where the fp32 partials are folded in two levels (runs of 8 consecutive
partials first, over many work-groups, then the owning work-group's merge of at
most 8), against the fp64 oracle on every output.

The oracle runs block row by block row: the queries of block i only see the keys
of the blocks in row i of the layout ("Big Bird", App. D), so the oracle gets
exactly those columns (the others are masked and contribute nothing); a global
block row gets every key.  dK and dV sum the block rows' contributions.
"""

import numpy as np
import pytest
import torch

from block_sparse_long_bsattn_amd import _lib as B
from block_sparse_long_bsattn_amd import inputs as I
from oracle import attention as OA
from oracle import layout as OL
from gpu_util import BF16_TOL, max_abs, qkv, say, to_f64

pytestmark = pytest.mark.gpu


def blockwise_oracle(refs, n, G, w, r, seed, scale):
    qr, kr, vr, dor = refs
    bsz, heads, _, d = qr.shape
    lay = OL.build_layout(n, 64, heads, G, w, r, seed)
    nb = lay["nb"]
    o, dq, dk, dv = (np.zeros((bsz, heads, n, d)) for _ in range(4))
    lse = np.zeros((bsz, heads, n))
    for h in range(heads):
        mask = OL.token_mask(lay["rows"][h], nb, 64, n)
        hs = slice(h, h + 1)
        for i in range(nb):
            rows = np.arange(64 * i, min(n, 64 * i + 64))
            cols = np.concatenate([np.arange(64 * j, min(n, 64 * j + 64))
                                   for j in sorted(lay["rows"][h][i])])
            sub = mask[rows][:, cols]
            m = lambda _h, a, b, sub=sub: sub[a:b]
            args = (qr[:, hs][:, :, rows], kr[:, hs][:, :, cols], vr[:, hs][:, :, cols])
            ro, rl = OA.attention_fwd(*args, m, scale)
            rdq, rdk, rdv = OA.attention_bwd(*args, dor[:, hs][:, :, rows], m, scale)
            o[:, h, rows], lse[:, h, rows], dq[:, h, rows] = ro[:, 0], rl[:, 0], rdq[:, 0]
            dk[:, h, cols] += rdk[:, 0]
            dv[:, h, cols] += rdv[:, 0]
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("case", [
    # n, heads, d, global blocks, segments of a global row
    (16428, 2, 64, [0, 100, 256], 33),   # 257 blocks, the last (global) holds 44 tokens
    (16448, 1, 128, [0, 256], 33),
])
def test_bs_folded_partials(case):
    n, heads, d, G, nseg = case
    w, r, seed, scale = 3, 3, 0xF01D, d ** -0.5
    say(f"bs folded partials n={n} H={heads} d={d} G={G}")
    (q, k, v, do), refs = qkv((1, heads, n, d), "bf16", (I.SEED_Q, I.SEED_K, I.SEED_V, I.SEED_DO))
    lay = B.bsattn_layout_build(n, 64, heads, G, w, r, seed)
    try:
        wsf = torch.empty(B.bsattn_fwd_workspace(lay, 1, d), dtype=torch.uint8, device="cuda")
        wsb_n = B.bsattn_bwd_workspace(lay, 1, d)
        wsb = torch.empty(wsb_n, dtype=torch.uint8, device="cuda")
        o, o_lo = torch.full_like(q, float("nan")), torch.full_like(q, float("nan"))
        lse = torch.full((1, heads, n), float("nan"), dtype=torch.float32, device="cuda")
        grads = [torch.full_like(q, float("nan")) for _ in range(3)]
        outs = []
        for _ in range(2):   # the second call must give the same bits
            B.bsattn_fwd(lay, q, k, v, o, lse, wsf, scale=scale, o_lo=o_lo)
            B.bsattn_bwd(lay, q, k, v, o, lse, do, *grads, wsb, scale=scale, o_lo=o_lo)
            torch.cuda.synchronize()
            outs.append([t.clone() for t in [o, lse] + grads])
    finally:
        B.bsattn_layout_destroy(lay)
    same = all(torch.equal(a, b) for a, b in zip(*outs))
    # the backward's workspace: D, then the dQ, dK, dV partial tiles of the nseg
    # segments of each global row and column, and their ceil(nseg / 8) folds
    up = lambda x: (x + 255) // 256 * 256
    assert wsb_n == up(heads * n * 4) + heads * len(G) * (nseg + -(-nseg // 8)) * 3 * 64 * d * 4
    got = [to_f64(t) for t in outs[1]]
    want = blockwise_oracle(refs, n, G, w, r, seed, scale)
    errs = {nm: max_abs(a, b) for nm, a, b in zip(("O", "lse", "dQ", "dK", "dV"), got, want)}
    say("   max-abs " + "  ".join(f"{a} {b:.2e}" for a, b in errs.items()) +
        f"  repeat-identical {same}")
    assert max(errs.values()) <= BF16_TOL
    assert same
