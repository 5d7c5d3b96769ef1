"""Host-side checks of bench.py's workload bookkeeping (no GPU): the useful-pair
counts that turn step times into useful FLOP/s agree with the oracle's masks."""

import numpy as np
import pytest

import bench
from oracle import longformer as LF


@pytest.mark.parametrize("n,w1,G,dil,causal", [
    (512, 40, [], 0, False),
    (512, 40, [0, 1, 300], 0, False),
    (640, 17, [], 3, True),
    (640, 17, [], 2, False),
    (576, 9, [5, 6, 500], 1, False),
    (256, 300, [], 1, True),
])
def test_longformer_pair_count_matches_oracle_mask(n, w1, G, dil, causal):
    m = LF.longformer_mask(n, w1, G, dil, causal)
    assert bench.longformer_pairs(n, w1, G, dil, causal) == int(m(0, 0, n).sum())


def test_workloads_have_the_documented_shapes():
    w = bench.WORKLOADS["longformer_causal_fwd_bwd_b1_h8_n23040_w256_dil3x2"]
    assert (w["n"], w["heads"], w["w1"], w["causal"]) == (23040, 8, 256, True)
    assert sorted(w["dil"]) == [0] * 6 + [3, 3]
    assert bench.WORKLOADS[bench.PRIMARY]["n"] == 4096


@pytest.mark.parametrize("g,n,b,w", [(256, 4096, 84, 3), (430, 4096, 169, 3), (5, 100, 13, 5),
                                     (0, 64, 64, 1)])
def test_etc_pair_count_matches_oracle_mask(g, n, b, w):
    from oracle import etc as E
    m = E.etc_mask(g, n, b, w)
    N = g + n
    count = sum(int(m(0, p0, min(N, p0 + 1024)).sum()) for p0 in range(0, N, 1024))
    assert bench.etc_pairs(g, n, b, w) == count
