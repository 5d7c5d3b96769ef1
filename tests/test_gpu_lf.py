"""GPU Longformer forward vs the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

from block_sparse_long_bsattn_amd import _lib as B
from oracle import attention as OA
from oracle import longformer as OLF
from gpu_util import BF16_TOL, max_abs, qkv, say, to_f64

pytestmark = pytest.mark.gpu


def run_lf(n, heads, bsz, w1, G):
    shape = (bsz, heads, n, 64)
    (q, k, v), (qr, kr, vr) = qkv(shape, "bf16")
    plan = B.lfattn_plan_build(n, w1, G)
    try:
        o = torch.empty_like(q)
        lse = torch.empty((bsz, heads, n), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(1, B.lfattn_fwd_workspace(plan, bsz, heads)), dtype=torch.uint8,
                         device="cuda")
        B.lfattn_fwd(plan, q, k, v, o, lse, ws)
        torch.cuda.synchronize()
    finally:
        B.lfattn_plan_destroy(plan)
    return (qr, kr, vr), to_f64(o), to_f64(lse)


@pytest.mark.parametrize("case", [
    (1024, 2, 2, 64, list(range(16))),          # prefix globals, window on tile edges
    (1024, 2, 1, 100, [5, 300, 301, 777]),      # scattered globals, ragged window
    (1024, 1, 1, 0, [0]),                       # the token itself only
    (1024, 2, 1, 200, []),                      # no global tokens
    (768, 1, 1, 2000, [3]),                     # window longer than the sequence
    (2048, 1, 1, 256, list(range(0, 2048, 15))),  # 137 globals: 3 packed tiles
    (640, 1, 2, 31, list(range(64))),           # one tile entirely global
    (64, 1, 1, 5, [10, 20]),                    # a single tile
])
def test_lf_full_compare(case):
    n, heads, bsz, w1, G = case
    say(f"lf full-compare n={n} H={heads} B={bsz} w1={w1} |G|={len(G)}")
    (qr, kr, vr), o, lse = run_lf(n, heads, bsz, w1, G)
    ro, rl = OA.attention_fwd(qr, kr, vr, OLF.longformer_mask(n, w1, G), 1 / 8.0)
    eo, el = max_abs(o, ro), max_abs(lse, rl)
    say(f"   max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= BF16_TOL and el <= BF16_TOL


def test_lf_full_size_sampled():
    """batch 1, 12 heads, n = 4096, 256 tokens per side, global tokens 0..63."""
    n, heads, w1, G = 4096, 12, 256, list(range(64))
    say("lf full-size n=4096 H=12 w1=256 G=0..63")
    (qr, kr, vr), o, lse = run_lf(n, heads, 1, w1, G)
    mask = OLF.longformer_mask(n, w1, G)
    worst = 0.0
    for h in (0, 7):
        sl = (slice(0, 1), slice(h, h + 1))
        ro, rl = OA.attention_fwd(qr[sl], kr[sl], vr[sl], mask, 1 / 8.0, row_chunk=1024)
        worst = max(worst, max_abs(o[0, h], ro[0, 0]), max_abs(lse[0, h], rl[0, 0]))
    rng = np.random.default_rng(5)
    for h in range(heads):
        rows = np.unique(np.r_[0, 63, 64, 319, 320, 3839, 3840, 4095, rng.integers(0, n, 8)])
        ro, rl = OA.attention_fwd_rows(qr, kr, vr, mask, 1 / 8.0, 0, h, rows)
        worst = max(worst, max_abs(o[0, h, rows], ro), max_abs(lse[0, h, rows], rl))
    say(f"   worst max-abs {worst:.3e}")
    assert worst <= BF16_TOL


def test_lf_zero_queries_closed_form():
    n, w1, G = 2048, 100, [0, 1, 2, 999, 1500]
    shape = (1, 1, n, 64)
    (q, k, v), (qr, kr, vr) = qkv(shape, "bf16")
    q.zero_()
    plan = B.lfattn_plan_build(n, w1, G)
    try:
        o = torch.empty_like(q)
        lse = torch.empty((1, 1, n), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(1, B.lfattn_fwd_workspace(plan, 1, 1)), dtype=torch.uint8, device="cuda")
        B.lfattn_fwd(plan, q, k, v, o, lse, ws)
        torch.cuda.synchronize()
    finally:
        B.lfattn_plan_destroy(plan)
    o, lse = to_f64(o), to_f64(lse)
    gs = set(G)
    worst_o = worst_l = 0.0
    for p in range(0, n, 7):
        keys = list(range(n)) if p in gs else sorted(set(range(max(0, p - w1), min(n, p + w1 + 1))) | gs)
        worst_o = max(worst_o, max_abs(o[0, 0, p], vr[0, 0, keys].mean(0)))
        worst_l = max(worst_l, abs(lse[0, 0, p] - math.log(len(keys))))
    say(f"   Q=0: max|dO|={worst_o:.3e} max|dlse|={worst_l:.3e}")
    assert worst_o <= 2e-3 and worst_l <= 1e-5
