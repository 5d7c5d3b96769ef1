"""Compute calls inside a captured HIP graph: none of them allocates, copies or
clears memory, so a captured step replays the eager results bit for bit.  Every
replay is checked, with eager work and synchronisations between replays."""

import pytest
import torch

from block_sparse_long_bsattn_amd import _lib as B
from block_sparse_long_bsattn_amd import inputs as I
from gpu_util import qkv, say

pytestmark = pytest.mark.gpu

SEEDS = (I.SEED_Q, I.SEED_K, I.SEED_V, I.SEED_DO)


def capture_and_replay(step, outputs, replays=3):
    """Run step eagerly, then capture it on a side stream and replay it; returns
    whether every replay reproduced the eager outputs."""
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step()                      # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.synchronize()
    same = []
    junk = torch.randn(1 << 16, device="cuda")
    for rep in range(replays):
        for t in outputs:           # clobber the outputs eagerly between replays
            t.fill_(float("nan") if t.is_floating_point() else 0)
        junk.mul_(1.0001)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same.append(all(torch.equal(a, b) for a, b in zip(outputs, ref)))
        say(f"   replay {rep}: bitwise equal to eager = {same[-1]}")
    return all(same)


def test_blocksparse_step_replays_bitwise():
    n, heads, bsz = 1024, 2, 2
    (q, k, v, do), _ = qkv((bsz, heads, n, 64), "bf16", SEEDS)
    lay = B.bsattn_layout_build(n, 64, heads, [0, 15], 3, 3, 7)
    try:
        o = torch.empty_like(q)
        lse = torch.empty((bsz, heads, n), dtype=torch.float32, device="cuda")
        wsf = torch.empty(max(16, B.bsattn_fwd_workspace(lay, bsz)), dtype=torch.uint8,
                          device="cuda")
        wsb = torch.empty(max(16, B.bsattn_bwd_workspace(lay, bsz)), dtype=torch.uint8,
                          device="cuda")
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))

        def step():
            B.bsattn_layout_rebuild(lay, 11)
            B.bsattn_fwd(lay, q, k, v, o, lse, wsf)
            B.bsattn_bwd(lay, q, k, v, o, lse, do, dq, dk, dv, wsb)

        say("graph: block-sparse rebuild + fwd + bwd")
        assert capture_and_replay(step, [o, lse, dq, dk, dv])
    finally:
        B.bsattn_layout_destroy(lay)


def test_longformer_step_replays_bitwise():
    n, heads, bsz = 1024, 2, 1
    (q, k, v, do), _ = qkv((bsz, heads, n, 64), "bf16", SEEDS)
    plan = B.lfattn_plan_build_dilated(n, 70, [0, 5, 600], heads, [0, 1])
    try:
        o = torch.empty_like(q)
        lse = torch.empty((bsz, heads, n), dtype=torch.float32, device="cuda")
        wsf = torch.empty(max(16, B.lfattn_fwd_workspace(plan, bsz, heads)), dtype=torch.uint8,
                          device="cuda")
        wsb = torch.empty(max(16, B.lfattn_bwd_workspace(plan, bsz, heads)), dtype=torch.uint8,
                          device="cuda")
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))

        def step():
            B.lfattn_fwd(plan, q, k, v, o, lse, wsf)
            B.lfattn_bwd(plan, q, k, v, o, lse, do, dq, dk, dv, wsb)

        say("graph: Longformer (dilated, globals) fwd + bwd")
        assert capture_and_replay(step, [o, lse, dq, dk, dv])
    finally:
        B.lfattn_plan_destroy(plan)


def test_blocksparse_d128_noalloc_step_replays_bitwise():
    """Head dimension 128, the forward writing the O residual and the backward
    without a workspace (its static scratch): the step a graph-capturing caller that
    cannot allocate would record."""
    n, heads, bsz, d = 768, 2, 1, 128
    (q, k, v, do), _ = qkv((bsz, heads, n, d), "bf16", SEEDS)
    lay = B.bsattn_layout_build(n, 64, heads, [0, 11], 3, 3, 9)
    try:
        o, olo = torch.empty_like(q), torch.empty_like(q)
        lse = torch.empty((bsz, heads, n), dtype=torch.float32, device="cuda")
        wsf = torch.empty(max(16, B.bsattn_fwd_workspace(lay, bsz, d)), dtype=torch.uint8,
                          device="cuda")
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))

        def step():
            B.bsattn_layout_rebuild(lay, 13)
            B.bsattn_fwd(lay, q, k, v, o, lse, wsf, o_lo=olo)
            B.bsattn_bwd_noalloc(lay, q, k, v, o, lse, do, dq, dk, dv, o_lo=olo)

        say("graph: block-sparse d=128 rebuild + fwd + no-allocation bwd")
        assert capture_and_replay(step, [o, olo, lse, dq, dk, dv])
    finally:
        B.bsattn_layout_destroy(lay)
