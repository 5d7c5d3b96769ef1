"""GPU layout builder vs the oracle: bit-exact CSR and CSC."""

import numpy as np
import pytest

from block_sparse_long_bsattn_amd import _lib as B
from oracle import layout as OL
from gpu_util import say

pytestmark = pytest.mark.gpu

CONFIG_PATTERNS = [
    # n, heads, G, w, r   (the five workload patterns; Longformer has no block layout)
    (512, 1, [0, 7], 3, 3),
    (4096, 12, [0, 63], 3, 3),
    (16384, 16, [0, 255], 3, 3),
]


def compare(n, heads, G, w, r, seed):
    say(f"layout n={n} heads={heads} G={G[:6]}{'...' if len(G) > 6 else ''} w={w} r={r} seed={seed}")
    h = B.bsattn_layout_build(n, 64, heads, G, w, r, seed)
    try:
        rp, ci, cp, cs = B.bsattn_layout_to_host(h)
        nb, hh, nnz = B.bsattn_layout_info(h)
    finally:
        B.bsattn_layout_destroy(h)
    ref = OL.build_layout(n, 64, heads, G, w, r, seed)
    assert (nb, hh, nnz) == ((n + 63) // 64, heads, len(ref["col_idx"]))
    # every head stores nnz / heads pairs
    assert all(ref["row_ptr"][(x + 1) * nb] - ref["row_ptr"][x * nb] == nnz // heads
               for x in range(heads))
    np.testing.assert_array_equal(rp, ref["row_ptr"])
    np.testing.assert_array_equal(ci, ref["col_idx"])
    np.testing.assert_array_equal(cp, ref["csc_ptr"])
    np.testing.assert_array_equal(cs, ref["csc_idx"])


@pytest.mark.parametrize("cfg", CONFIG_PATTERNS)
def test_layout_configs_bit_exact(cfg):
    n, heads, G, w, r = cfg
    compare(n, heads, G, w, r, 0x5EED)


def test_layout_random_sweep_bit_exact():
    rng = np.random.default_rng(2024)
    for case in range(24):
        nb = int(rng.integers(1, 160))
        heads = int(rng.integers(1, 4))
        g = int(rng.integers(0, min(nb, 6) + 1))
        G = sorted(rng.choice(nb, size=g, replace=False).tolist())
        w = int(rng.choice([1, 3, 5, 7, 9, 2 * nb + 1]))
        r = int(rng.integers(0, 12))
        seed = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        compare(nb * 64, heads, G, w, r, seed)


def test_layout_edge_cases_bit_exact():
    compare(64, 1, [0], 1, 3, 1)                 # single block, global
    compare(64, 2, [], 1, 3, 1)                  # single block, nothing to draw
    compare(640, 2, list(range(10)), 3, 3, 5)    # every block global
    compare(640, 2, [], 1, 0, 5)                 # window only
    compare(1024, 2, [0], 1, 64, 5)              # r beyond the candidates
    compare(64 * 300, 1, [0, 299], 3, 3, 2**64 - 1)   # largest seed
    compare(64 * 600, 2, [0, 7, 599], 3, 3, 99)      # more than 512 blocks: two-kernel path
    compare(64 * 600, 1, [1, 300], 5, 12, 98)        # ... with more than 8 random blocks
    compare(64 * 40, 3, [2], 3, 9, 97)               # more than 8 random blocks
    compare(64 * 600, 1, list(range(0, 600, 50)), 3, 3, 96)   # > 512 blocks, > 8 global
    compare(64 * 100, 2, list(range(3, 100, 9)), 5, 4, 95)    # > 8 global blocks
    compare(64 * 512, 1, [0, 511], 3, 3, 94)         # 512 blocks: largest one-kernel layout


def test_layout_max_blocks_bit_exact():
    """The largest layout the library builds: n/b = 4096 blocks (n = 262,144)."""
    compare(64 * 4096, 1, [0, 4095], 3, 3, 93)


def test_layout_rebuild_matches_new_seed():
    n, heads, G, w, r = 4096, 3, [0, 63], 3, 3
    h = B.bsattn_layout_build(n, 64, heads, G, w, r, 11)
    try:
        B.bsattn_layout_rebuild(h, 12345)
        rp, ci, cp, cs = B.bsattn_layout_to_host(h)
    finally:
        B.bsattn_layout_destroy(h)
    ref = OL.build_layout(n, 64, heads, G, w, r, 12345)
    np.testing.assert_array_equal(ci, ref["col_idx"])
    np.testing.assert_array_equal(cs, ref["csc_idx"])
