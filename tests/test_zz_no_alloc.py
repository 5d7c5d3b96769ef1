"""bsattn_bwd_noalloc (the backward with the library's static device scratch, for
callers that cannot allocate) against bsattn_bwd with a caller workspace: same
kernels, so the outputs must be identical bit for bit.  Two calls in a row, the
second on a smaller problem (the scratch keeps the first call's contents), and a
problem whose scratch need exceeds the static array is rejected."""

import ctypes

import numpy as np
import pytest
import torch

from block_sparse_long_bsattn_amd import _lib as B
from block_sparse_long_bsattn_amd import inputs as I
from gpu_util import qkv, say

pytestmark = pytest.mark.gpu


def one_case(n, heads, bsz, G, seed):
    say(f"bwd_noalloc vs bwd: n={n} H={heads} B={bsz} G={G}")
    shape = (bsz, heads, n, 64)
    (q, k, v, do), _ = qkv(shape, "bf16", (I.SEED_Q, I.SEED_K, I.SEED_V, I.SEED_DO))
    h = B.bsattn_layout_build(n, 64, heads, G, 3, 3, seed)
    try:
        need = B.bsattn_bwd_workspace(h, bsz)
        assert need <= B.BSATTN_BWD_NOALLOC_SCRATCH_BYTES
        o = torch.empty_like(q)
        o_lo = torch.empty_like(q)
        lse = torch.empty((bsz, heads, n), dtype=torch.float32, device="cuda")
        wsf = torch.empty(max(16, B.bsattn_fwd_workspace(h, bsz)), dtype=torch.uint8, device="cuda")
        wsb = torch.empty(max(16, need), dtype=torch.uint8, device="cuda")
        B.bsattn_fwd(h, q, k, v, o, lse, wsf, o_lo=o_lo)
        ref = [torch.empty_like(q) for _ in range(3)]
        B.bsattn_bwd(h, q, k, v, o, lse, do, *ref, wsb, o_lo=o_lo)
        got = [torch.full_like(q, float("nan")) for _ in range(3)]
        # straight through the C ABI
        lib = B.load()
        st = lib.bsattn_bwd_noalloc(h, bsz, 64, B.BSATTN_BF16, ctypes.c_float(0.125),
                                    q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    o_lo.data_ptr(), lse.data_ptr(), do.data_ptr(),
                                    got[0].data_ptr(), got[1].data_ptr(), got[2].data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
        assert st == B.BSATTN_OK, B.bsattn_last_error()
        torch.cuda.synchronize()
    finally:
        B.bsattn_layout_destroy(h)
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        same = torch.equal(a, b)
        say(f"   {name} bitwise equal: {same}")
        assert same


def test_bwd_noalloc_matches_bwd_twice():
    # the headline training shape, then a smaller one with split global rows
    one_case(4096, 12, 4, [0, 63], I.SEED_LAYOUT)
    one_case(1024, 2, 1, [0, 15], 7)


def test_bwd_noalloc_rejects_oversize():
    """B = 32, 16 heads, n = 16384 needs ~235 MB of scratch: EINVAL before any launch
    (the tensor pointers are never dereferenced)."""
    h = B.bsattn_layout_build(16384, 64, 16, [0, 255], 3, 3, 1)
    try:
        assert B.bsattn_bwd_workspace(h, 32) > B.BSATTN_BWD_NOALLOC_SCRATCH_BYTES
        dummy = torch.empty(64, dtype=torch.bfloat16, device="cuda")
        p = dummy.data_ptr()
        st = B.load().bsattn_bwd_noalloc(h, 32, 64, B.BSATTN_BF16, ctypes.c_float(0.125),
                                         p, p, p, p, None, p, p, p, p, p, None)
        assert st == B.BSATTN_EINVAL
        assert "scratch" in B.bsattn_last_error()
    finally:
        B.bsattn_layout_destroy(h)
