"""GPU Longformer forward and backward with per-head dilation and the causal
window, against the fp64 oracle."""

import numpy as np
import pytest
import torch

from block_sparse_long_bsattn_amd import _lib as B
from block_sparse_long_bsattn_amd import inputs as I
from oracle import attention as OA
from oracle import longformer as OLF
from gpu_util import BF16_TOL, max_abs, qkv, say, to_f64

pytestmark = pytest.mark.gpu

SEEDS = (I.SEED_Q, I.SEED_K, I.SEED_V, I.SEED_DO)


def run(n, bsz, w1, G, dil, causal, bwd=True, plain_plan=False):
    heads = len(dil)
    shape = (bsz, heads, n, 64)
    (q, k, v, do), refs = qkv(shape, "bf16", SEEDS)
    if plain_plan:
        plan = B.lfattn_plan_build(n, w1, G)
    else:
        plan = B.lfattn_plan_build_dilated(n, w1, G, heads, dil, causal)
    try:
        o = torch.empty_like(q)
        lse = torch.empty((bsz, heads, n), dtype=torch.float32, device="cuda")
        wsf = torch.empty(max(1, B.lfattn_fwd_workspace(plan, bsz, heads)), dtype=torch.uint8,
                          device="cuda")
        B.lfattn_fwd(plan, q, k, v, o, lse, wsf)
        out = [o, lse]
        if bwd:
            wsb = torch.empty(max(1, B.lfattn_bwd_workspace(plan, bsz, heads)),
                              dtype=torch.uint8, device="cuda")
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            B.lfattn_bwd(plan, q, k, v, o, lse, do, dq, dk, dv, wsb)
            out += [dq, dk, dv]
        torch.cuda.synchronize()
    finally:
        B.lfattn_plan_destroy(plan)
    return refs, [t.clone() for t in out]


def report(names, got, ref):
    errs = []
    for name, a, b in zip(names, got, ref):
        e = max_abs(a, b)
        errs.append(e)
        i = np.unravel_index(np.argmax(np.abs(a - b)), a.shape)
        say(f"   {name}: max-abs {e:.3e} at {tuple(int(x) for x in i)} "
            f"(got {a[i]:.5f} ref {b[i]:.5f})")
    return max(errs)


@pytest.mark.parametrize("case", [
    (1024, 1, 64, [], [0, 1, 2, 3], False),            # one stride per head
    (1024, 2, 100, [5, 300, 301, 777], [1, 2], False),  # globals, ragged classes (s = 3)
    (1024, 1, 64, [], [0, 1, 2], True),                # causal
    (512, 1, 0, [], [0, 3], True),                     # causal, the token itself only
    (960, 1, 37, [0, 100, 959], [5], False),           # 160-token classes: ragged tiles
    (2048, 1, 2000, [], [0, 2], True),                 # window past the start: full causal
    (64, 1, 5, [10, 20], [1, 4], False),               # a single tile
    (1024, 1, 16, [], [63, 200], False),               # classes of 16 and 5 tokens
    (768, 1, 40, list(range(64)), [0, 1], False),      # a natural tile of globals, dilated
])
def test_lf_dilated_full_compare(case):
    n, bsz, w1, G, dil, causal = case
    say(f"lf dilated full-compare n={n} B={bsz} w1={w1} |G|={len(G)} dil={dil} causal={causal}")
    (qr, kr, vr, dor), got = run(n, bsz, w1, G, dil, causal)
    mask = OLF.longformer_mask(n, w1, G, dil, causal)
    ro, rl = OA.attention_fwd(qr, kr, vr, mask, 1 / 8.0)
    rdq, rdk, rdv = OA.attention_bwd(qr, kr, vr, dor, mask, 1 / 8.0)
    worst = report(("O", "lse", "dQ", "dK", "dV"), [to_f64(t) for t in got],
                   (ro, rl, rdq, rdk, rdv))
    assert worst <= BF16_TOL


def test_zero_dilation_plan_matches_plain_plan_bitwise():
    """A per-head plan with dilation 0 everywhere walks the same tiles in the same
    order as the plan for any head count: identical bits."""
    n, G = 1024, [0, 1, 2, 600]
    _, a = run(n, 2, 90, G, [0, 0, 0], False)
    _, b = run(n, 2, 90, G, [0, 0, 0], False, plain_plan=True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("a0", [0, 11008, 23040 - 64])
def test_lf_causal_dilated_full_size_windows(a0):
    """Batch 1, 8 heads, n = 23040, 256 earlier tokens, dilation 3 on two heads
    (the character-LM shape of Table 12 at its last-phase length).  The whole job
    runs on the GPU; tokens [a0, a0 + 64) are then checked in full on every head,
    forward and backward, against the oracle on the sub-sequence that holds every
    query and key their values depend on (the pattern depends on p - q only, so
    those values are the same there)."""
    n, w1, dil = 23040, 256, [3, 3, 0, 0, 0, 0, 0, 0]
    say(f"lf causal dilated full-size n={n} H=8 w1={w1} dil={dil} window at {a0}")
    (qr, kr, vr, dor), got = run(n, 1, w1, [], dil, True)
    got = [to_f64(t) for t in got]
    span = w1 * (max(dil) + 1)
    x0, x1 = max(0, a0 - span), min(n, a0 + 64 + span)
    sub = slice(x0, x1)
    mask = OLF.longformer_mask(x1 - x0, w1, [], dil, True)
    ro, rl = OA.attention_fwd(qr[:, :, sub], kr[:, :, sub], vr[:, :, sub], mask, 1 / 8.0)
    rdq, rdk, rdv = OA.attention_bwd(qr[:, :, sub], kr[:, :, sub], vr[:, :, sub],
                                     dor[:, :, sub], mask, 1 / 8.0)
    r = slice(a0 - x0, a0 - x0 + 64)
    g = slice(a0, a0 + 64)
    worst = report(("O", "lse", "dQ", "dK", "dV"),
                   [got[0][:, :, g], got[1][:, :, g], got[2][:, :, g], got[3][:, :, g],
                    got[4][:, :, g]],
                   (ro[:, :, r], rl[:, :, r], rdq[:, :, r], rdk[:, :, r], rdv[:, :, r]))
    assert worst <= BF16_TOL


def test_lf_dilated_rejects_bad_arguments():
    with pytest.raises(B.BsattnError):
        B.lfattn_plan_build_dilated(512, 8, [0], 2, [0, 1], causal=True)
    with pytest.raises(ValueError):
        B.lfattn_plan_build_dilated(512, 8, [], 2, [0])
    plan = B.lfattn_plan_build_dilated(512, 8, [], 2, [0, 1], causal=True)
    try:
        assert B.lfattn_fwd_workspace(plan, 1, 3) == 0
        (q, k, v), _ = qkv((1, 3, 512, 64), "bf16", (1, 2, 3))
        o = torch.empty_like(q)
        lse = torch.empty((1, 3, 512), dtype=torch.float32, device="cuda")
        with pytest.raises(Exception):
            B.lfattn_fwd(plan, q, k, v, o, lse, None)
    finally:
        B.lfattn_plan_destroy(plan)
