"""Pins for the oracle's block layout (CPU only).

Each check ties the oracle to something other than itself: published generator
outputs, a hand derivation from them, closed-form block counts of the pattern,
set invariants the pages state, and the uniform law of sampling without
replacement.
"""

import itertools
import math

import numpy as np
import pytest
from scipy import stats

from conftest import read_golden
from oracle import layout as L


# --- generator -------------------------------------------------------------

def test_splitmix64_published_vectors():
    rows = read_golden("splitmix64_vectors.txt")
    assert len(rows) == 6
    for seed, k, val in rows:
        assert L.splitmix64(int(seed), int(k)) == int(val)


def test_fisher_yates_hand_derivation():
    """Row 0 of a tiny pattern, derived by hand from the published draws."""
    for seed, nb, w, r, rand, row in read_golden("layout_row0.txt"):
        seed, nb, w, r = int(seed), int(nb), int(w), int(r)
        got = L.random_blocks(0, 0, nb, [], w, r, seed)
        assert got == [int(x) for x in rand.split(",")]
        assert L.row_blocks(0, 0, nb, [], w, r, seed) == [int(x) for x in row.split(",")]


# --- closed forms -----------------------------------------------------------

@pytest.mark.parametrize("nb", [8, 16, 64, 256])
def test_block_count_closed_form(nb):
    """G = {0, nb-1}, w = 3, r = 3: two full rows, rows 1 and nb-2 see
    {0,1,2,nb-1}+3 random = 7 blocks, every other row sees 5 + 3 = 8 blocks.
    Total 2*nb + 2*7 + (nb-4)*8 = 10*nb - 18 block pairs per head."""
    lay = L.build_layout(nb * 64, 64, 2, [0, nb - 1], 3, 3, 0x5EED)
    for h in range(2):
        lens = [len(x) for x in lay["rows"][h]]
        assert lens[0] == nb and lens[-1] == nb
        assert lens[1] == 7 and lens[nb - 2] == 7
        assert all(x == 8 for x in lens[2:nb - 2])
        assert sum(lens) == 10 * nb - 18
    assert lay["row_ptr"][-1] == 2 * (10 * nb - 18)


def test_block_counts_match_pair_counts_of_configs():
    # attended (query, key) token pairs per head = 64*64 * block pairs
    assert 64 * 64 * (10 * 8 - 18) == 253_952
    assert 64 * 64 * (10 * 64 - 18) == 2_547_712
    assert 64 * 64 * (10 * 256 - 18) == 10_412_032


# --- set invariants ---------------------------------------------------------

CASES = [
    # n, b, heads, G, w, r
    (512, 64, 1, [0, 7], 3, 3),
    (4096, 64, 3, [0, 63], 3, 3),
    (16384, 64, 2, [0, 255], 3, 3),
    (640, 64, 2, [], 1, 0),
    (640, 64, 2, [3, 4, 9], 5, 2),
    (1024, 64, 2, [0], 7, 20),       # r exceeds the candidates of some rows
    (256, 16, 2, [], 31, 3),         # window covers every block
    (64, 64, 1, [0], 1, 3),          # single block
]


@pytest.mark.parametrize("case", CASES)
def test_layout_invariants(case):
    n, b, heads, G, w, r = case
    seed = 12345
    lay = L.build_layout(n, b, heads, G, w, r, seed)
    nb = n // b
    Gs = set(G)
    for h in range(heads):
        for i in range(nb):
            row = lay["rows"][h][i]
            assert row == sorted(set(row))
            if i in Gs:
                assert row == list(range(nb))
                continue
            win = set(L.window_blocks(i, nb, w))
            assert win == {j for j in range(nb) if abs(i - j) <= (w - 1) // 2}
            assert Gs | win <= set(row)
            rnd = L.random_blocks(h, i, nb, G, w, r, seed)
            assert not (set(rnd) & (Gs | win))
            assert len(set(rnd)) == len(rnd) == min(r, nb - len(Gs | win))
            assert set(row) == Gs | win | set(rnd)
            # CSR form
            p0, p1 = lay["row_ptr"][h * nb + i], lay["row_ptr"][h * nb + i + 1]
            assert list(lay["col_idx"][p0:p1]) == row
    # CSC is the transpose of CSR, columns ascending
    for h in range(heads):
        dense = np.zeros((nb, nb), dtype=bool)
        for i in range(nb):
            dense[i, lay["rows"][h][i]] = True
        for j in range(nb):
            c0, c1 = lay["csc_ptr"][h * nb + j], lay["csc_ptr"][h * nb + j + 1]
            assert list(lay["csc_idx"][c0:c1]) == list(np.nonzero(dense[:, j])[0])
    assert lay["csc_ptr"][-1] == lay["row_ptr"][-1] == len(lay["col_idx"])
    # row lengths do not depend on the draws, so every head stores the same count
    per_head = [lay["row_ptr"][(h + 1) * nb] - lay["row_ptr"][h * nb] for h in range(heads)]
    assert len(set(per_head)) == 1


def test_heads_draw_independently():
    lay = L.build_layout(16384, 64, 4, [0, 255], 3, 3, 7)
    rows = lay["rows"]
    for a, c in itertools.combinations(range(4), 2):
        assert rows[a] != rows[c]


def test_block_and_token_mask():
    lay = L.build_layout(512, 64, 1, [0, 7], 3, 3, 99)
    bm = L.block_mask(lay["rows"][0], 8)
    tm = L.token_mask(lay["rows"][0], 8, 64)
    for p in range(0, 512, 7):
        for q in range(0, 512, 5):
            assert tm[p, q] == ((q // 64) in lay["rows"][0][p // 64])
    assert bm.sum() * 64 * 64 == tm.sum()


def test_bad_arguments_rejected():
    with pytest.raises(ValueError):
        L.build_layout(0, 64, 1, [], 3, 3, 0)         # empty sequence
    with pytest.raises(ValueError):
        L.build_layout(500, 64, 1, [8], 3, 3, 0)      # block 8 past ceil(500/64) = 8
    with pytest.raises(ValueError):
        L.build_layout(512, 64, 1, [0], 2, 3, 0)      # even window
    with pytest.raises(ValueError):
        L.build_layout(512, 64, 1, [7, 0], 3, 3, 0)   # unsorted global set
    with pytest.raises(ValueError):
        L.build_layout(512, 64, 1, [8], 3, 3, 0)      # out of range
    with pytest.raises(ValueError):
        L.build_layout(512, 64, 1, [0], 3, -1, 0)     # negative r


# --- the law of the random draws ---------------------------------------------

def test_random_subsets_uniform():
    """Sampling without replacement: every r-subset of the m candidates is equally
    likely.  nb = 12, G = {0, 11}, w = 3, query block 5 -> m = 7 candidates, r = 3
    -> 35 subsets.  Chi-square over 7000 seeds, and each candidate's marginal
    probability r/m."""
    nb, G, w, r, i = 12, [0, 11], 3, 3, 5
    cand = [j for j in range(nb) if j not in G and abs(j - i) > 1]
    assert len(cand) == 7
    subsets = {s: 0 for s in itertools.combinations(cand, r)}
    marg = {c: 0 for c in cand}
    trials = 7000
    for seed in range(trials):
        rnd = L.random_blocks(0, i, nb, G, w, r, seed * 7919 + 1)
        subsets[tuple(sorted(rnd))] += 1
        for c in rnd:
            marg[c] += 1
    counts = np.array(list(subsets.values()))
    _, p = stats.chisquare(counts)
    assert p > 1e-4, (p, counts)
    for c in cand:
        assert abs(marg[c] / trials - r / len(cand)) < 0.03


def test_draw_slots_are_disjoint_across_rows_and_heads():
    """(h*nb + i)*r + t + 1 enumerates every draw slot exactly once."""
    nb, r, heads = 16, 3, 3
    ks = [(h * nb + i) * r + t + 1 for h in range(heads) for i in range(nb) for t in range(r)]
    assert sorted(ks) == list(range(1, heads * nb * r + 1))


def test_expected_random_indegree():
    """Each non-global, non-window column is hit by a row with probability r/m, so
    the mean random in-degree over many seeds matches the closed form."""
    nb, G, w, r = 16, [0, 15], 3, 3
    trials = 300
    hits = np.zeros(nb)
    for s in range(trials):
        for i in range(nb):
            if i in G:
                continue
            for j in L.random_blocks(0, i, nb, G, w, r, s + 1000):
                hits[j] += 1
    expect = np.zeros(nb)
    for i in range(nb):
        if i in G:
            continue
        cand = [j for j in range(nb) if j not in G and abs(j - i) > 1]
        for j in cand:
            expect[j] += min(r, len(cand)) / len(cand)
    assert np.max(np.abs(hits / trials - expect)) < 0.25
    assert math.isclose(hits.sum() / trials, expect.sum(), rel_tol=1e-12)


# --- sequences that end inside a block ----------------------------------------

@pytest.mark.parametrize("n,G,w,r", [(1000, [0, 15], 3, 3), (4000, [0, 62], 3, 3),
                                     (130, [2], 1, 2), (700, [], 5, 4)])
def test_ragged_length_pairs_closed_form(n, G, w, r):
    """ceil(n/b) blocks, the last one short: each query block i contributes
    rows(i) * sum of the sizes of the blocks in N(i), sizes b except the last."""
    b = 64
    lay = L.build_layout(n, b, 2, G, w, r, 3)
    nb = lay["nb"]
    assert nb == (n + b - 1) // b
    size = [b] * (nb - 1) + [n - b * (nb - 1)]
    for h in range(2):
        want = sum(size[i] * sum(size[j] for j in lay["rows"][h][i]) for i in range(nb))
        assert int(L.token_mask(lay["rows"][h], nb, b, n).sum()) == want


def test_ragged_length_is_the_padded_pattern_cut_to_n():
    """The layout depends on ceil(n/b) only: the mask of n tokens is the mask of
    the padded length with the positions past n removed."""
    n, b = 1000, 64
    lay = L.build_layout(n, b, 1, [0, 15], 3, 3, 9)
    pad = L.build_layout(16 * b, b, 1, [0, 15], 3, 3, 9)
    assert lay["rows"] == pad["rows"]
    full = L.token_mask(pad["rows"][0], 16, b)
    assert np.array_equal(L.token_mask(lay["rows"][0], 16, b, n), full[:n, :n])
