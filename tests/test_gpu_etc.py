"""GPU BigBird-ETC (added global tokens, blocked window) and sequences that end
inside a 64-token tile, forward and backward, against the fp64 oracle."""

import pytest
import torch

from block_sparse_long_bsattn_amd import _lib as B
from block_sparse_long_bsattn_amd import inputs as I
from oracle import attention as OA
from oracle import etc as OE
from oracle import longformer as OLF
from gpu_util import BF16_TOL, max_abs, qkv, say, to_f64

pytestmark = pytest.mark.gpu

SEEDS = (I.SEED_Q, I.SEED_K, I.SEED_V, I.SEED_DO)


def run(plan, N, heads, bsz):
    shape = (bsz, heads, N, 64)
    (q, k, v, do), refs = qkv(shape, "bf16", SEEDS)
    try:
        o = torch.empty_like(q)
        lse = torch.empty((bsz, heads, N), dtype=torch.float32, device="cuda")
        wsf = torch.empty(max(1, B.lfattn_fwd_workspace(plan, bsz, heads)), dtype=torch.uint8,
                          device="cuda")
        wsb = torch.empty(max(1, B.lfattn_bwd_workspace(plan, bsz, heads)), dtype=torch.uint8,
                          device="cuda")
        B.lfattn_fwd(plan, q, k, v, o, lse, wsf)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        B.lfattn_bwd(plan, q, k, v, o, lse, do, dq, dk, dv, wsb)
        torch.cuda.synchronize()
        first = [t.clone() for t in (o, lse, dq, dk, dv)]
        B.lfattn_fwd(plan, q, k, v, o, lse, wsf)
        B.lfattn_bwd(plan, q, k, v, o, lse, do, dq, dk, dv, wsb)
        torch.cuda.synchronize()
        same = all(torch.equal(a, b) for a, b in zip(first, (o, lse, dq, dk, dv)))
    finally:
        B.lfattn_plan_destroy(plan)
    return refs, [to_f64(t) for t in first], same


def compare(refs, got, mask, heads=None):
    qr, kr, vr, dor = refs
    if heads is not None:
        sl = (slice(None), slice(heads[0], heads[1]))
        qr, kr, vr, dor = (x[sl] for x in (qr, kr, vr, dor))
        got = [x[sl] for x in got]
    ro, rl = OA.attention_fwd(qr, kr, vr, mask, 1 / 8.0)
    rdq, rdk, rdv = OA.attention_bwd(qr, kr, vr, dor, mask, 1 / 8.0)
    errs = {}
    for name, a, b in zip(("O", "lse", "dQ", "dK", "dV"), got, (ro, rl, rdq, rdk, rdv)):
        errs[name] = max_abs(a, b)
    say("   max-abs " + "  ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    return max(errs.values())


@pytest.mark.parametrize("case", [
    (16, 200, 23, 3, 2, 1),      # ragged everywhere: 216 tokens, blocks of 23
    (256, 1000, 84, 3, 2, 1),    # base ETC block length, 1256 tokens
    (0, 1024, 64, 3, 1, 2),      # no added tokens: the blocked window alone
    (43, 800, 169, 3, 2, 1),     # large ETC block length, tokens not a multiple of 64
    (5, 120, 17, 11, 1, 1),      # window over every block: full attention
    (64, 300, 84, 5, 1, 1),      # a whole tile of global tokens, w = 5
    (7, 57, 13, 1, 1, 1),        # own block only, one partial tile
])
def test_etc_full_compare(case):
    g, n, b, w, heads, bsz = case
    say(f"etc full-compare g={g} n={n} b={b} w={w} H={heads} B={bsz}")
    refs, got, same = run(B.lfattn_plan_build_etc(g, n, b, w), g + n, heads, bsz)
    assert compare(refs, got, OE.etc_mask(g, n, b, w)) <= BF16_TOL
    assert same


@pytest.mark.parametrize("cfg", [
    (256, 4096, 84, 3, 12),      # BigBird-etc base (App. E MLM table)
    (430, 4096, 169, 3, 16),     # BigBird-etc large, WikiHop global count
])
def test_etc_full_size(cfg):
    """The whole job on the GPU; two heads compared in full with the oracle."""
    g, n, b, w, heads = cfg
    say(f"etc full-size g={g} n={n} b={b} w={w} H={heads}")
    refs, got, same = run(B.lfattn_plan_build_etc(g, n, b, w), g + n, heads, 1)
    worst = 0.0
    for h in (0, heads - 1):
        worst = max(worst, compare(refs, got, OE.etc_mask(g, n, b, w), heads=(h, h + 1)))
    assert worst <= BF16_TOL and same


def test_etc_base_batch4_long_segments():
    """BigBird-etc base at batch 4 (the benchmark shape): enough work per work-group
    slot that the global rows run in segments of 32 key tiles and the columns of the
    global keys in segments of 16 query tiles (read off the backward's workspace
    size); two (batch, head) slices compared in full with the oracle."""
    g, n, b, w, heads, bsz = 256, 4096, 84, 3, 12, 4
    N, nt, tile = g + n, (g + n + 63) // 64, 64 * 64 * 4
    plan = B.lfattn_plan_build_etc(g, n, b, w)
    try:
        ws = B.lfattn_bwd_workspace(plan, bsz, heads)
    finally:
        B.lfattn_plan_destroy(plan)
    up = lambda x: (x + 255) // 256 * 256
    rows, cols = bsz * heads * 4 * -(-nt // 32), bsz * heads * 4 * -(-nt // 16)
    assert ws == up(up(up(bsz * heads * N * 4) + rows * tile) + cols * 2 * tile)
    say(f"etc base batch 4: row segments of 32 tiles, column segments of 16 (workspace {ws})")
    refs, got, same = run(B.lfattn_plan_build_etc(g, n, b, w), N, heads, bsz)
    worst = 0.0
    for bi, h in ((0, 0), (3, 11)):
        sl = (slice(bi, bi + 1), slice(None))
        worst = max(worst, compare([x[sl] for x in refs], [x[sl] for x in got],
                                   OE.etc_mask(g, n, b, w), heads=(h, h + 1)))
    assert worst <= BF16_TOL and same


@pytest.mark.parametrize("case", [
    (1000, 70, [3, 999], [0], False),      # sliding window, ends 40 tokens into a tile
    (700, 33, [], [0, 2], True),           # causal, dilated, ragged
    (63, 5, [0], [1], False),              # shorter than one tile
])
def test_lf_ragged_length(case):
    n, w1, G, dil, causal = case
    say(f"lf ragged n={n} w1={w1} G={G} dil={dil} causal={causal}")
    plan = B.lfattn_plan_build_dilated(n, w1, G, len(dil), dil, causal)
    refs, got, same = run(plan, n, len(dil), 1)
    assert compare(refs, got, OLF.longformer_mask(n, w1, G, dil, causal)) <= BF16_TOL
    assert same
