"""GPU Longformer backward vs the fp64 oracle's exact gradient."""

import numpy as np
import pytest
import torch

from block_sparse_long_bsattn_amd import _lib as B
from block_sparse_long_bsattn_amd import inputs as I
from oracle import attention as OA
from oracle import longformer as OLF
from gpu_util import BF16_TOL, max_abs, qkv, say, to_f64

pytestmark = pytest.mark.gpu


def run_lf_bwd(n, heads, bsz, w1, G, seeds=(I.SEED_Q, I.SEED_K, I.SEED_V, I.SEED_DO)):
    shape = (bsz, heads, n, 64)
    (q, k, v, do), refs = qkv(shape, "bf16", seeds)
    plan = B.lfattn_plan_build(n, w1, G)
    try:
        o = torch.empty_like(q)
        lse = torch.empty((bsz, heads, n), dtype=torch.float32, device="cuda")
        wsf = torch.empty(max(1, B.lfattn_fwd_workspace(plan, bsz, heads)), dtype=torch.uint8,
                          device="cuda")
        wsb = torch.empty(max(1, B.lfattn_bwd_workspace(plan, bsz, heads)), dtype=torch.uint8,
                          device="cuda")
        B.lfattn_fwd(plan, q, k, v, o, lse, wsf)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        B.lfattn_bwd(plan, q, k, v, o, lse, do, dq, dk, dv, wsb)
        torch.cuda.synchronize()
        out = (dq.clone(), dk.clone(), dv.clone())
        # a second call on the same buffers must give the same bits
        B.lfattn_bwd(plan, q, k, v, o, lse, do, dq, dk, dv, wsb)
        torch.cuda.synchronize()
        same = all(torch.equal(a, b) for a, b in zip(out, (dq, dk, dv)))
    finally:
        B.lfattn_plan_destroy(plan)
    return refs, tuple(to_f64(t) for t in out), same


# w1 = 0 with a global token (every row puts ~1/2 of its mass on that token, whose dK
# and dV sum n such terms, reaching 40-60) is compared on random inputs in
# test_gpu_edge.py, against 2e-2 plus half a bf16 ulp of the exact value, and with
# Q = 0 against the closed form below.
@pytest.mark.parametrize("case", [
    (1024, 2, 2, 64, list(range(16))),          # prefix globals, window on tile edges
    (1024, 2, 1, 100, [5, 300, 301, 777]),      # scattered globals, ragged window
    (1024, 1, 1, 0, []),                        # the token itself only (P = 1)
    (1024, 2, 1, 200, []),                      # no global tokens
    (768, 1, 1, 2000, [3]),                     # window longer than the sequence
    (2048, 1, 1, 256, list(range(0, 2048, 15))),  # 137 globals: 3 global tiles
    (640, 1, 2, 31, list(range(64))),           # one tile entirely global
    (64, 1, 1, 5, [10, 20]),                    # a single tile
])
def test_lf_bwd_full_compare(case):
    n, heads, bsz, w1, G = case
    say(f"lf bwd full-compare n={n} H={heads} B={bsz} w1={w1} |G|={len(G)}")
    (qr, kr, vr, dor), got, same = run_lf_bwd(n, heads, bsz, w1, G)
    ref = OA.attention_bwd(qr, kr, vr, dor, OLF.longformer_mask(n, w1, G), 1 / 8.0)
    errs = [max_abs(a, b) for a, b in zip(got, ref)]
    say(f"   max-abs dQ {errs[0]:.3e} dK {errs[1]:.3e} dV {errs[2]:.3e}  repeat-identical {same}")
    for name, a, b in zip("QKV", got, ref):
        i = np.unravel_index(np.argmax(np.abs(a - b)), a.shape)
        say(f"   d{name} worst at {tuple(int(x) for x in i)}: got {a[i]:.5f} ref {b[i]:.5f}; "
            f"max |ref| {np.max(np.abs(b)):.3f}")
    assert max(errs) <= BF16_TOL
    assert same


def test_lf_bwd_full_size_sampled():
    """batch 1, 12 heads, n = 4096, 256 tokens per side, global tokens 0..63: the whole
    job runs on the GPU; two heads are compared in full with the oracle."""
    n, heads, w1, G = 4096, 12, 256, list(range(64))
    say("lf bwd full-size n=4096 H=12 w1=256 G=0..63")
    (qr, kr, vr, dor), got, same = run_lf_bwd(n, heads, 1, w1, G)
    mask = OLF.longformer_mask(n, w1, G)
    worst = 0.0
    for h in (0, 11):
        sl = (slice(0, 1), slice(h, h + 1))
        ref = OA.attention_bwd(qr[sl], kr[sl], vr[sl], dor[sl], mask, 1 / 8.0, row_chunk=1024)
        worst = max(worst, *(max_abs(a[0, h], b[0, 0]) for a, b in zip(got, ref)))
    say(f"   worst max-abs {worst:.3e}  repeat-identical {same}")
    assert worst <= BF16_TOL and same


def test_lf_long_row_segments():
    """Batch 4, 12 heads, n = 4096, 256 per side, global tokens 0..63: enough work per
    work-group slot that the global rows run in segments of 32 key tiles (two per row,
    read off the forward's workspace size) instead of 8.  Forward and backward of two
    (batch, head) slices compared in full with the oracle."""
    n, heads, bsz, w1, G = 4096, 12, 4, 256, list(range(64))
    plan = B.lfattn_plan_build(n, w1, G)
    try:
        rec = 64 * 64 + 3 * 64    # floats of one partial record of a 64-row global tile
        nseg = B.lfattn_fwd_workspace(plan, bsz, heads) // (bsz * heads * 1 * rec * 4)
    finally:
        B.lfattn_plan_destroy(plan)
    say(f"lf long row segments n={n} H={heads} B={bsz}: {nseg} segments per global row")
    assert nseg == 2
    (q, k, v, do), refs = qkv((bsz, heads, n, 64), "bf16",
                             (I.SEED_Q, I.SEED_K, I.SEED_V, I.SEED_DO))
    plan = B.lfattn_plan_build(n, w1, G)
    try:
        o = torch.empty_like(q)
        lse = torch.empty((bsz, heads, n), dtype=torch.float32, device="cuda")
        wsf = torch.empty(B.lfattn_fwd_workspace(plan, bsz, heads), dtype=torch.uint8,
                          device="cuda")
        wsb = torch.empty(B.lfattn_bwd_workspace(plan, bsz, heads), dtype=torch.uint8,
                          device="cuda")
        B.lfattn_fwd(plan, q, k, v, o, lse, wsf)
        grads = [torch.empty_like(q) for _ in range(3)]
        B.lfattn_bwd(plan, q, k, v, o, lse, do, *grads, wsb)
        torch.cuda.synchronize()
    finally:
        B.lfattn_plan_destroy(plan)
    got = [to_f64(t) for t in [o, lse] + grads]
    qr, kr, vr, dor = refs
    mask = OLF.longformer_mask(n, w1, G)
    worst = 0.0
    for b, h in ((0, 5), (3, 11)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ro, rl = OA.attention_fwd(qr[sl], kr[sl], vr[sl], mask, 1 / 8.0)
        rg = OA.attention_bwd(qr[sl], kr[sl], vr[sl], dor[sl], mask, 1 / 8.0, row_chunk=1024)
        for a, r in zip(got, (ro, rl) + tuple(rg)):
            worst = max(worst, max_abs(a[sl], r))
    say(f"   worst max-abs {worst:.3e}")
    assert worst <= BF16_TOL


def test_lf_bwd_sum_identities():
    """Rows of P sum to one and rows of dS to zero, so per (batch, head) the dV rows
    sum to the dO rows and the dK rows sum to zero (bf16 outputs: loose bound)."""
    n, w1, G = 2048, 150, [0, 1, 700, 2047]
    (qr, kr, vr, dor), (dq, dk, dv), _ = run_lf_bwd(n, 2, 1, w1, G)
    e_v = max_abs(dv.sum(2), dor.sum(2))
    e_k = float(np.max(np.abs(dk.sum(2))))
    say(f"   |sum dV - sum dO| {e_v:.3e}  |sum dK| {e_k:.3e}")
    assert e_v <= 0.5 and e_k <= 0.5


def test_lf_bwd_rejects_bad_arguments():
    n = 512
    plan = B.lfattn_plan_build(n, 64, [0])
    try:
        shape = (1, 1, n, 64)
        (q, k, v, do), _ = qkv(shape, "bf16", (1, 2, 3, 4))
        o = torch.empty_like(q)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        with pytest.raises(ValueError):
            B.lfattn_bwd(plan, q, k, v, o, None, do, dq, dk, dv, None)
        lse = torch.empty((1, 1, n), dtype=torch.float32, device="cuda")
        small = torch.empty(16, dtype=torch.uint8, device="cuda")
        with pytest.raises(Exception):
            B.lfattn_bwd(plan, q, k, v, o, lse, do, dq, dk, dv, small)
    finally:
        B.lfattn_plan_destroy(plan)


def test_lf_bwd_zero_queries_closed_form():
    """Q = 0 makes every row's probabilities uniform over its keys.  With w1 = 0 they
    are exact in bf16: 1/2 (a token and the global token 0) and 1/1024 (the global
    row), or 1 without global tokens.  Then dV[q] = sum over the rows p that see q of
    dO[p] / |N(p)| and dK = 0 exactly.  With token 0 global this is the extreme
    fan-in case: every row puts half its mass on token 0."""
    n = 1024
    for G in ([0], []):
        w1 = 0
        shape = (1, 1, n, 64)
        (q, k, v, do), (qr, kr, vr, dor) = qkv(shape, "bf16",
                                              (I.SEED_Q, I.SEED_K, I.SEED_V, I.SEED_DO))
        q.zero_()
        plan = B.lfattn_plan_build(n, w1, G)
        try:
            o = torch.empty_like(q)
            lse = torch.empty((1, 1, n), dtype=torch.float32, device="cuda")
            wsf = torch.empty(max(1, B.lfattn_fwd_workspace(plan, 1, 1)), dtype=torch.uint8,
                              device="cuda")
            wsb = torch.empty(max(1, B.lfattn_bwd_workspace(plan, 1, 1)), dtype=torch.uint8,
                              device="cuda")
            B.lfattn_fwd(plan, q, k, v, o, lse, wsf)
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            B.lfattn_bwd(plan, q, k, v, o, lse, do, dq, dk, dv, wsb)
            torch.cuda.synchronize()
        finally:
            B.lfattn_plan_destroy(plan)
        dk, dv = to_f64(dk), to_f64(dv)
        ref = np.zeros((n, 64))
        for p in range(n):
            keys = list(range(n)) if p in G else sorted({p} | set(G))
            ref[keys] += dor[0, 0, p] / len(keys)
        # bound: fp32 accumulation plus half a bf16 ulp of the output
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        err = np.abs(dv[0, 0] - ref)
        say(f"   G={G}: max|dV - ref| {err.max():.3e} (max |ref| {np.abs(ref).max():.2f}), "
            f"max|dK| {np.abs(dk).max():.1e}")
        assert np.all(err <= 0.5 * ulp + 1e-3)
        assert np.abs(dk).max() == 0.0
