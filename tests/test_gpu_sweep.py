"""Seeded random configurations, forward and backward, full compare against the fp64
oracle (bf16 inputs, max-abs 2e-2 on O, lse, dQ, dK, dV).

The fixed-shape tests pick one case per code path; this sweep draws the pattern
parameters instead, so that combinations nobody wrote down (a global block next to
the window's edge, r beyond the free blocks of some rows, a ragged last block that
is also global, several dilations and a causal window with a ragged last tile) are
exercised too.  Every draw comes from one numpy generator with a fixed seed, and
each case prints its parameters before it runs.
"""

import numpy as np
import pytest
import torch

from block_sparse_long_bsattn_amd import _lib as B
from block_sparse_long_bsattn_amd import inputs as I
from oracle import attention as OA
from oracle import layout as OL
from oracle import longformer as OLF
from gpu_util import BF16_TOL, max_abs, qkv, say, to_f64

pytestmark = pytest.mark.gpu

SEEDS = (I.SEED_Q, I.SEED_K, I.SEED_V, I.SEED_DO)


def bigbird_cases(count=12, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        n = int(rng.integers(1, 17)) * 64 - int(rng.choice([0, 0, rng.integers(1, 64)]))
        nb = (n + 63) // 64
        g = int(rng.integers(0, min(nb, 4) + 1))
        G = sorted(int(x) for x in rng.choice(nb, g, replace=False))
        w = int(rng.choice([1, 3, 5, 7]))
        r = int(rng.integers(0, 6))
        heads = int(rng.integers(1, 4))
        bsz = int(rng.integers(1, 3))
        out.append((n, heads, bsz, G, w, r, int(rng.integers(0, 1 << 30))))
    return out


def longformer_cases(count=10, seed=7):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        n = int(rng.integers(1, 17)) * 64 - int(rng.choice([0, rng.integers(1, 64)]))
        heads = int(rng.integers(1, 4))
        w1 = int(rng.integers(0, 300))
        dil = [int(x) for x in rng.integers(0, 4, heads)]
        causal = bool(rng.integers(0, 2))
        G = [] if causal else sorted(int(x) for x in rng.choice(n, int(rng.integers(0, 9)),
                                                                 replace=False))
        out.append((n, heads, w1, G, dil, causal))
    return out


def full_check(refs, got, mask, scale):
    qr, kr, vr, dor = refs
    ro, rl = OA.attention_fwd(qr, kr, vr, mask, scale)
    rdq, rdk, rdv = OA.attention_bwd(qr, kr, vr, dor, mask, scale)
    errs = [max_abs(a, b) for a, b in zip(got, (ro, rl, rdq, rdk, rdv))]
    say("   max-abs O {:.2e} lse {:.2e} dQ {:.2e} dK {:.2e} dV {:.2e}".format(*errs))
    assert max(errs) <= BF16_TOL


@pytest.mark.parametrize("case", bigbird_cases())
def test_bigbird_random_pattern(case):
    n, heads, bsz, G, w, r, lseed = case
    say(f"bigbird sweep n={n} H={heads} B={bsz} G={G} w={w} r={r} seed={lseed}")
    shape = (bsz, heads, n, 64)
    (q, k, v, do), refs = qkv(shape, "bf16", SEEDS)
    h = B.bsattn_layout_build(n, 64, heads, G, w, r, lseed)
    try:
        o, olo = torch.empty_like(q), torch.empty_like(q)
        lse = torch.empty((bsz, heads, n), dtype=torch.float32, device="cuda")
        wsf = torch.empty(max(1, B.bsattn_fwd_workspace(h, bsz)), dtype=torch.uint8,
                          device="cuda")
        wsb = torch.empty(max(1, B.bsattn_bwd_workspace(h, bsz)), dtype=torch.uint8,
                          device="cuda")
        B.bsattn_fwd(h, q, k, v, o, lse, wsf, o_lo=olo)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        B.bsattn_bwd(h, q, k, v, o, lse, do, dq, dk, dv, wsb, o_lo=olo)
        torch.cuda.synchronize()
    finally:
        B.bsattn_layout_destroy(h)
    lay = OL.build_layout(n, 64, heads, G, w, r, lseed)
    masks = [OL.token_mask(lay["rows"][hh], lay["nb"], 64, n) for hh in range(heads)]
    full_check(refs, [to_f64(t) for t in (o, lse, dq, dk, dv)],
               lambda hh, p0, p1: masks[hh][p0:p1], 1 / 8.0)


@pytest.mark.parametrize("case", longformer_cases())
def test_longformer_random_pattern(case):
    n, heads, w1, G, dil, causal = case
    say(f"longformer sweep n={n} H={heads} w1={w1} G={G} dilation={dil} causal={causal}")
    shape = (1, heads, n, 64)
    (q, k, v, do), refs = qkv(shape, "bf16", SEEDS)
    plan = B.lfattn_plan_build_dilated(n, w1, G, heads, dil, causal)
    try:
        o, olo = torch.empty_like(q), torch.empty_like(q)
        lse = torch.empty((1, heads, n), dtype=torch.float32, device="cuda")
        wsf = torch.empty(max(1, B.lfattn_fwd_workspace(plan, 1, heads)), dtype=torch.uint8,
                          device="cuda")
        wsb = torch.empty(max(1, B.lfattn_bwd_workspace(plan, 1, heads)), dtype=torch.uint8,
                          device="cuda")
        B.lfattn_fwd(plan, q, k, v, o, lse, wsf, o_lo=olo)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        B.lfattn_bwd(plan, q, k, v, o, lse, do, dq, dk, dv, wsb, o_lo=olo)
        torch.cuda.synchronize()
    finally:
        B.lfattn_plan_destroy(plan)
    full_check(refs, [to_f64(t) for t in (o, lse, dq, dk, dv)],
               OLF.longformer_mask(n, w1, G, dil, causal), 1 / 8.0)
