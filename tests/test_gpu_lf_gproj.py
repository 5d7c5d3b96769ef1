"""GPU Longformer with separate global projections (Q_g, K_g, V_g for the rows of
global tokens), forward and backward, against the fp64 oracle."""

import pytest
import torch

from block_sparse_long_bsattn_amd import _lib as B
from oracle import longformer as OLF
from gpu_util import BF16_TOL, max_abs, qkv, say, to_f64

pytestmark = pytest.mark.gpu

SEEDS = (101, 102, 103, 104, 105, 106, 107)   # q, k, v, qg, kg, vg, dout


def run(plan, n, heads, bsz, same_sets=False):
    shape = (bsz, heads, n, 64)
    dev, refs = qkv(shape, "bf16", SEEDS)
    q, k, v, qg, kg, vg, do = dev
    if same_sets:
        qg, kg, vg = q, k, v
        refs = refs[:3] + refs[:3] + refs[6:]
    try:
        o = torch.empty_like(q)
        lse = torch.empty((bsz, heads, n), dtype=torch.float32, device="cuda")
        wsf = torch.empty(max(1, B.lfattn_fwd_workspace(plan, bsz, heads)), dtype=torch.uint8,
                          device="cuda")
        wsb = torch.empty(max(1, B.lfattn_bwd_workspace(plan, bsz, heads)), dtype=torch.uint8,
                          device="cuda")
        B.lfattn_fwd_gproj(plan, q, k, v, qg, kg, vg, o, lse, wsf)
        grads = [torch.full_like(q, float("nan")) for _ in range(6)]   # every element written
        B.lfattn_bwd_gproj(plan, q, k, v, qg, kg, vg, o, lse, do, *grads, wsb)
        torch.cuda.synchronize()
        out = [o.clone(), lse.clone()] + [g.clone() for g in grads]
        if same_sets:
            o1, l1 = torch.empty_like(o), torch.empty_like(lse)
            B.lfattn_fwd(plan, q, k, v, o1, l1, wsf)
            torch.cuda.synchronize()
            out += [o1, l1]
    finally:
        B.lfattn_plan_destroy(plan)
    return refs, out


def compare(refs, got, n, w1, G, dil=0, heads=None):
    q, k, v, qg, kg, vg, do = refs
    got = [to_f64(t) for t in got[:8]]
    if heads is not None:
        sl = (slice(None), slice(heads[0], heads[1]))
        q, k, v, qg, kg, vg, do = (x[sl] for x in (q, k, v, qg, kg, vg, do))
        got = [x[sl] for x in got]
    ro, rl = OLF.longformer_gproj_fwd(q, k, v, qg, kg, vg, n, w1, G, 1 / 8.0, dil)
    rg = OLF.longformer_gproj_bwd(q, k, v, qg, kg, vg, do, n, w1, G, 1 / 8.0, dil)
    names = ("O", "lse", "dQ", "dK", "dV", "dQg", "dKg", "dVg")
    errs = {nm: max_abs(a, b) for nm, a, b in zip(names, got, (ro, rl) + tuple(rg))}
    say("   max-abs " + "  ".join(f"{a} {b:.2e}" for a, b in errs.items()))
    return max(errs.values())


@pytest.mark.parametrize("case", [
    (1024, 2, 1, 64, list(range(16))),          # prefix globals
    (1024, 1, 2, 100, [5, 300, 301, 777]),      # scattered globals
    (768, 1, 1, 40, list(range(64))),           # one tile entirely global
    (1000, 1, 1, 70, [3, 999]),                 # sequence ends inside a tile
    (512, 1, 1, 30, []),                        # no global tokens: dQg, dKg, dVg = 0
])
def test_gproj_full_compare(case):
    n, heads, bsz, w1, G = case
    say(f"gproj full-compare n={n} H={heads} B={bsz} w1={w1} |G|={len(G)}")
    plan = B.lfattn_plan_build(n, w1, G)
    refs, got = run(plan, n, heads, bsz)
    assert compare(refs, got, n, w1, G) <= BF16_TOL


def test_gproj_with_dilation():
    n, w1, G, dil = 1024, 50, [0, 5, 600], [1, 2]
    say(f"gproj dilated n={n} w1={w1} G={G} dil={dil}")
    plan = B.lfattn_plan_build_dilated(n, w1, G, 2, dil)
    refs, got = run(plan, n, 2, 1)
    worst = 0.0
    for h, d in enumerate(dil):
        worst = max(worst, compare(refs, got, n, w1, G, d, heads=(h, h + 1)))
    assert worst <= BF16_TOL


def test_gproj_equal_sets_forward_is_lfattn_fwd():
    """Equal projection sets (the page's initialisation): the forward is lfattn_fwd's,
    bit for bit, and the gradients still match the oracle."""
    n, w1, G = 1024, 64, [0, 1, 2, 500]
    plan = B.lfattn_plan_build(n, w1, G)
    refs, got = run(plan, n, 2, 1, same_sets=True)
    assert torch.equal(got[0], got[8]) and torch.equal(got[1], got[9])
    assert compare(refs, got, n, w1, G) <= BF16_TOL


def test_gproj_full_size_sampled():
    """batch 1, 12 heads, n = 4096, 256 per side, globals 0..63; heads 0 and 11."""
    n, heads, w1, G = 4096, 12, 256, list(range(64))
    say("gproj full-size n=4096 H=12 w1=256 G=0..63")
    plan = B.lfattn_plan_build(n, w1, G)
    refs, got = run(plan, n, heads, 1)
    worst = max(compare(refs, got, n, w1, G, heads=(h, h + 1)) for h in (0, 11))
    assert worst <= BF16_TOL


def test_gproj_rejects_aliased_outputs():
    n = 256
    plan = B.lfattn_plan_build(n, 16, [0])
    try:
        dev, _ = qkv((1, 1, n, 64), "bf16", SEEDS)
        q, k, v, qg, kg, vg, do = dev
        o = torch.empty_like(q)
        lse = torch.empty((1, 1, n), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(1, B.lfattn_bwd_workspace(plan, 1, 1)), dtype=torch.uint8,
                         device="cuda")
        g = torch.empty_like(q)
        with pytest.raises(B.BsattnError):
            B.lfattn_bwd_gproj(plan, q, k, v, qg, kg, vg, o, lse, do, g, torch.empty_like(q),
                               torch.empty_like(q), g, torch.empty_like(q),
                               torch.empty_like(q), ws)
    finally:
        B.lfattn_plan_destroy(plan)
