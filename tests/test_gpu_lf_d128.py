"""GPU token-level kernels (Longformer windows and globals, dilated and causal
windows, BigBird-ETC, separate global projections) at head dimension d = 128,
bf16, against the fp64 oracle.

Every configuration on the pages has d = 64 ("Longformer", App. B Table 12; "Big
Bird", App. E tables); d = 128 is built as a second instance of the same kernels.
Scores use scale = 1/sqrt(128), so that their spread matches the d = 64 cases,
and the bound is the same max-abs 2e-2 over every output of every slice.
"""

import math

import pytest
import torch

from block_sparse_long_bsattn_amd import _lib as B
from block_sparse_long_bsattn_amd import inputs as I
from oracle import attention as OA
from oracle import etc as OE
from oracle import longformer as OLF
from gpu_util import BF16_TOL, max_abs, qkv, say, to_f64

pytestmark = pytest.mark.gpu

D = 128
SCALE = 1 / math.sqrt(D)
SEEDS = (I.SEED_Q, I.SEED_K, I.SEED_V, I.SEED_DO)


def run(plan, N, heads, bsz, bwd=True):
    """Forward (and backward) through the plan; returns the fp64 inputs and outputs."""
    (q, k, v, do), refs = qkv((bsz, heads, N, D), "bf16", SEEDS)
    try:
        o = torch.full_like(q, float("nan"))
        olo = torch.full_like(q, float("nan"))
        lse = torch.full((bsz, heads, N), float("nan"), dtype=torch.float32, device="cuda")
        wsf = torch.empty(max(1, B.lfattn_fwd_workspace(plan, bsz, heads, D)),
                          dtype=torch.uint8, device="cuda")
        B.lfattn_fwd(plan, q, k, v, o, lse, wsf, scale=SCALE, o_lo=olo)
        out = [o, lse]
        if bwd:
            wsb = torch.empty(max(1, B.lfattn_bwd_workspace(plan, bsz, heads, D)),
                              dtype=torch.uint8, device="cuda")
            grads = [torch.full_like(q, float("nan")) for _ in range(3)]
            B.lfattn_bwd(plan, q, k, v, o, lse, do, *grads, wsb, scale=SCALE, o_lo=olo)
            out += grads
        torch.cuda.synchronize()
    finally:
        B.lfattn_plan_destroy(plan)
    return refs, [to_f64(t) for t in out]


def compare(refs, got, mask, heads=None):
    qr, kr, vr, dor = refs
    if heads is not None:
        sl = (slice(None), slice(heads[0], heads[1]))
        qr, kr, vr, dor = (x[sl] for x in (qr, kr, vr, dor))
        got = [x[sl] for x in got]
    ro, rl = OA.attention_fwd(qr, kr, vr, mask, SCALE)
    want = [ro, rl]
    if len(got) > 2:
        want += list(OA.attention_bwd(qr, kr, vr, dor, mask, SCALE))
    names = ("O", "lse", "dQ", "dK", "dV")
    errs = {nm: max_abs(a, b) for nm, a, b in zip(names, got, want)}
    say("   max-abs " + "  ".join(f"{a} {b:.2e}" for a, b in errs.items()))
    return max(errs.values())


LF_CASES = [
    # n, heads, bsz, w1, global tokens
    (1024, 2, 1, 100, list(range(16))),     # prefix globals
    (1000, 1, 2, 70, [3, 999]),             # sequence ends inside a tile
    (768, 1, 1, 40, list(range(64))),       # one tile entirely global
    (512, 1, 1, 30, []),                    # window only
    (2048, 1, 1, 256, [5, 300, 301, 777]),  # the page's window, scattered globals
]


@pytest.mark.parametrize("case", LF_CASES)
def test_lf_d128_forward(case):
    n, heads, bsz, w1, G = case
    say(f"lf d128 fwd n={n} H={heads} B={bsz} w1={w1} |G|={len(G)}")
    refs, got = run(B.lfattn_plan_build(n, w1, G), n, heads, bsz, bwd=False)
    assert compare(refs, got, OLF.longformer_mask(n, w1, G)) <= BF16_TOL


def test_lf_d128_dilated_causal_forward():
    n, w1, dil = 900, 50, [0, 2]
    say(f"lf d128 fwd dilated causal n={n} w1={w1} dilation={dil}")
    plan = B.lfattn_plan_build_dilated(n, w1, [], 2, dil, True)
    refs, got = run(plan, n, 2, 1, bwd=False)
    assert compare(refs, got, OLF.longformer_mask(n, w1, [], dil, True)) <= BF16_TOL


@pytest.mark.parametrize("case", [(64, 300, 84, 5), (16, 200, 23, 3)])
def test_etc_d128_forward(case):
    g, n, b, w = case
    say(f"etc d128 fwd g={g} n={n} b={b} w={w}")
    refs, got = run(B.lfattn_plan_build_etc(g, n, b, w), g + n, 2, 1, bwd=False)
    assert compare(refs, got, OE.etc_mask(g, n, b, w)) <= BF16_TOL


def test_lf_d128_gproj_forward():
    n, w1, G = 1024, 64, list(range(16))
    say(f"lf d128 gproj fwd n={n} w1={w1} |G|={len(G)}")
    dev, refs = qkv((1, 2, n, D), "bf16", (101, 102, 103, 104, 105, 106))
    q, k, v, qg, kg, vg = dev
    plan = B.lfattn_plan_build(n, w1, G)
    try:
        o = torch.full_like(q, float("nan"))
        lse = torch.full((1, 2, n), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(1, B.lfattn_fwd_workspace(plan, 1, 2, D)), dtype=torch.uint8,
                         device="cuda")
        B.lfattn_fwd_gproj(plan, q, k, v, qg, kg, vg, o, lse, ws, scale=SCALE)
        torch.cuda.synchronize()
    finally:
        B.lfattn_plan_destroy(plan)
    ro, rl = OLF.longformer_gproj_fwd(*refs, n, w1, G, SCALE)
    errs = (max_abs(to_f64(o), ro), max_abs(to_f64(lse), rl))
    say(f"   max-abs O {errs[0]:.2e} lse {errs[1]:.2e}")
    assert max(errs) <= BF16_TOL


def test_lf_d128_full_size_forward():
    """The Longformer workload's shape (12 heads, n = 4096, 256 each side, 64
    global tokens) at d = 128; two heads compared in full."""
    n, heads, w1, G = 4096, 12, 256, list(range(64))
    say(f"lf d128 fwd full size n={n} H={heads} w1={w1}")
    refs, got = run(B.lfattn_plan_build(n, w1, G), n, heads, 1, bwd=False)
    assert compare(refs, got, OLF.longformer_mask(n, w1, G), heads=(3, 5)) <= BF16_TOL


@pytest.mark.parametrize("case", LF_CASES[:4])
def test_lf_d128_forward_backward(case):
    n, heads, bsz, w1, G = case
    say(f"lf d128 fwd+bwd n={n} H={heads} B={bsz} w1={w1} |G|={len(G)}")
    refs, got = run(B.lfattn_plan_build(n, w1, G), n, heads, bsz)
    assert compare(refs, got, OLF.longformer_mask(n, w1, G)) <= BF16_TOL


def test_lf_d128_dilated_causal_backward():
    n, w1, dil = 900, 50, [0, 2]
    say(f"lf d128 fwd+bwd dilated causal n={n} w1={w1} dilation={dil}")
    plan = B.lfattn_plan_build_dilated(n, w1, [], 2, dil, True)
    refs, got = run(plan, n, 2, 1)
    assert compare(refs, got, OLF.longformer_mask(n, w1, [], dil, True)) <= BF16_TOL


def test_lf_d128_dilated_with_globals_backward():
    n, w1, dil, G = 700, 40, [1, 3], [0, 2, 650]
    say(f"lf d128 fwd+bwd dilated n={n} w1={w1} dilation={dil} G={G}")
    plan = B.lfattn_plan_build_dilated(n, w1, G, 2, dil, False)
    refs, got = run(plan, n, 2, 1)
    assert compare(refs, got, OLF.longformer_mask(n, w1, G, dil, False)) <= BF16_TOL


@pytest.mark.parametrize("case", [(64, 300, 84, 5), (16, 200, 23, 3)])
def test_etc_d128_backward(case):
    g, n, b, w = case
    say(f"etc d128 fwd+bwd g={g} n={n} b={b} w={w}")
    refs, got = run(B.lfattn_plan_build_etc(g, n, b, w), g + n, 2, 1)
    assert compare(refs, got, OE.etc_mask(g, n, b, w)) <= BF16_TOL


def test_lf_d128_gproj_backward():
    n, w1, G = 1024, 64, [5, 300, 301, 777]
    say(f"lf d128 gproj fwd+bwd n={n} w1={w1} G={G}")
    dev, refs = qkv((1, 2, n, D), "bf16", (101, 102, 103, 104, 105, 106, 107))
    q, k, v, qg, kg, vg, do = dev
    plan = B.lfattn_plan_build(n, w1, G)
    try:
        o = torch.full_like(q, float("nan"))
        lse = torch.full((1, 2, n), float("nan"), dtype=torch.float32, device="cuda")
        wsf = torch.empty(max(1, B.lfattn_fwd_workspace(plan, 1, 2, D)), dtype=torch.uint8,
                          device="cuda")
        wsb = torch.empty(max(1, B.lfattn_bwd_workspace(plan, 1, 2, D)), dtype=torch.uint8,
                          device="cuda")
        B.lfattn_fwd_gproj(plan, q, k, v, qg, kg, vg, o, lse, wsf, scale=SCALE)
        grads = [torch.full_like(q, float("nan")) for _ in range(6)]
        B.lfattn_bwd_gproj(plan, q, k, v, qg, kg, vg, o, lse, do, *grads, wsb, scale=SCALE)
        torch.cuda.synchronize()
    finally:
        B.lfattn_plan_destroy(plan)
    qr, kr, vr, qgr, kgr, vgr, dor = refs
    ro, rl = OLF.longformer_gproj_fwd(qr, kr, vr, qgr, kgr, vgr, n, w1, G, SCALE)
    rg = OLF.longformer_gproj_bwd(qr, kr, vr, qgr, kgr, vgr, dor, n, w1, G, SCALE)
    names = ("O", "lse", "dQ", "dK", "dV", "dQg", "dKg", "dVg")
    got = [to_f64(t) for t in [o, lse] + grads]
    errs = {nm: max_abs(a, b) for nm, a, b in zip(names, got, (ro, rl) + tuple(rg))}
    say("   max-abs " + "  ".join(f"{a} {b:.2e}" for a, b in errs.items()))
    assert max(errs.values()) <= BF16_TOL


def test_lf_d128_full_size_backward():
    """The Longformer workload's shape at d = 128, forward and backward; two heads
    compared in full."""
    n, heads, w1, G = 4096, 12, 256, list(range(64))
    say(f"lf d128 fwd+bwd full size n={n} H={heads} w1={w1}")
    refs, got = run(B.lfattn_plan_build(n, w1, G), n, heads, 1)
    assert compare(refs, got, OLF.longformer_mask(n, w1, G), heads=(7, 9)) <= BF16_TOL
