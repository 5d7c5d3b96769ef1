"""Oracle: BigBird-ITC block layout (which key blocks each query block attends to).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix
------------------
* Big Bird: Transformers for Longer Sequences, §2 eq. (AT): query i attends to the
  set N(i) of keys; the attention is a sum over that *set*.
* Same page, §2 (global tokens): a global token attends to every token and every
  token attends to it (ITC: existing tokens are made global).
* Same page, App. D "Implementation details" and Fig. 6: sparsity is defined on
  b x b blocks; the key side of each query block is the concatenation of the
  global blocks, the window blocks and r random blocks; the result equals the
  pattern of Fig. 3(d).
* Chinese walkthrough of Big Bird (gitcode.csdn.net), §2.1-2.3: each query picks
  r random keys; each token sees w/2 neighbours per side; g tokens are global.

What the pages leave open, and the reading taken here
-----------------------------------------------------
* Window in blocks: block i sees blocks i-(w-1)/2 .. i+(w-1)/2, clipped to the
  sequence (w odd).
* Random blocks: r blocks drawn uniformly *without replacement* from the blocks
  that are neither global nor in the window; all of them if fewer remain.
  Global query blocks draw nothing (their row is already full).
* Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
  number generators", OOPSLA 2014).  Draw number k >= 1 of a stream seeded with
  s is mix(s + k * 0x9E3779B97F4A7C15 mod 2^64).  Query block i of head h uses
  draws k = (h*nb + i)*r + t + 1, t = 0..r-1 (slots of global rows stay unused).
* Selection: partial Fisher-Yates over the ascending candidate list C of size m:
  for t < min(r, m), swap C[t] with C[t + (u_t mod (m - t))]; the first
  min(r, m) entries are the random blocks.
* One layout per head, shared by every batch element.
* Sequence length not a multiple of b: App. D eq. (13) counts ceil(n/b) blocks.
  The last block then holds n - b*(ceil(n/b) - 1) tokens; the layout is the same
  block pattern over ceil(n/b) blocks, and the missing positions of the last
  block are simply not tokens (no query, no key; nothing is padded).
"""

from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15


def splitmix64(seed: int, k: int) -> int:
    """Draw number ``k`` (k >= 1) of the SplitMix64 stream seeded with ``seed``.

    Python integers are unbounded, so every product is reduced mod 2^64 by hand.
    """
    x = (seed + k * GOLDEN_GAMMA) & MASK64
    z = ((x ^ (x >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def window_blocks(i: int, nb: int, w: int) -> list[int]:
    """Window blocks of query block i: i-(w-1)/2 .. i+(w-1)/2, clipped to [0, nb)."""
    half = (w - 1) // 2
    return list(range(max(0, i - half), min(nb - 1, i + half) + 1))


def random_blocks(h: int, i: int, nb: int, global_blocks, w: int, r: int,
                  seed: int) -> list[int]:
    """Random key blocks of query block i in head h, in draw order (not sorted)."""
    excluded = set(global_blocks) | set(window_blocks(i, nb, w))
    cand = [j for j in range(nb) if j not in excluded]
    m = len(cand)
    take = min(r, m)
    for t in range(take):
        u = splitmix64(seed, (h * nb + i) * r + t + 1)
        s = t + u % (m - t)
        cand[t], cand[s] = cand[s], cand[t]
    return cand[:take]


def row_blocks(h: int, i: int, nb: int, global_blocks, w: int, r: int,
               seed: int) -> list[int]:
    """N(i) for query block i of head h, ascending, each block once (set semantics)."""
    if i in set(global_blocks):
        return list(range(nb))
    keys = set(global_blocks) | set(window_blocks(i, nb, w))
    keys |= set(random_blocks(h, i, nb, global_blocks, w, r, seed))
    return sorted(keys)


def check_args(n: int, b: int, heads: int, global_blocks, w: int, r: int) -> int:
    """Validate the pattern arguments; return nb.  Raises ValueError."""
    if b <= 0 or n <= 0:
        raise ValueError("n and b must be positive")
    if heads <= 0:
        raise ValueError("heads must be positive")
    if w < 1 or w % 2 == 0:
        raise ValueError("w must be odd and >= 1")
    if r < 0:
        raise ValueError("r must be >= 0")
    nb = -(-n // b)                  # ceil(n / b): the last block may be shorter
    g = list(global_blocks)
    if any(not (0 <= x < nb) for x in g) or g != sorted(set(g)):
        raise ValueError("global blocks must be sorted, unique and inside [0, ceil(n/b))")
    return nb


def build_layout(n: int, b: int, heads: int, global_blocks, w: int, r: int,
                 seed: int) -> dict:
    """Per-head row lists plus their CSR and CSC forms.

    Returns a dict with
      rows     : list over heads of list over query blocks of N(i)
      row_ptr  : int32 [heads*nb + 1]  (head h row i starts at row_ptr[h*nb + i])
      col_idx  : int32 [nnz]           (key block ids)
      csc_ptr  : int32 [heads*nb + 1]  (head h key block j starts at csc_ptr[h*nb + j])
      csc_idx  : int32 [nnz]           (query block ids, ascending per column)
    """
    nb = check_args(n, b, heads, global_blocks, w, r)
    rows = [[row_blocks(h, i, nb, global_blocks, w, r, seed) for i in range(nb)]
            for h in range(heads)]
    row_ptr = [0]
    col_idx: list[int] = []
    for h in range(heads):
        for i in range(nb):
            col_idx.extend(rows[h][i])
            row_ptr.append(len(col_idx))
    cols = [[[] for _ in range(nb)] for _ in range(heads)]
    for h in range(heads):
        for i in range(nb):
            for j in rows[h][i]:
                cols[h][j].append(i)
    csc_ptr = [0]
    csc_idx: list[int] = []
    for h in range(heads):
        for j in range(nb):
            csc_idx.extend(cols[h][j])
            csc_ptr.append(len(csc_idx))
    return {
        "nb": nb,
        "rows": rows,
        "row_ptr": np.asarray(row_ptr, dtype=np.int32),
        "col_idx": np.asarray(col_idx, dtype=np.int32),
        "csc_ptr": np.asarray(csc_ptr, dtype=np.int32),
        "csc_idx": np.asarray(csc_idx, dtype=np.int32),
    }


def block_mask(rows_h, nb: int) -> np.ndarray:
    """nb x nb boolean: [i, j] is True iff key block j is in N(i)."""
    m = np.zeros((nb, nb), dtype=bool)
    for i, keys in enumerate(rows_h):
        m[i, keys] = True
    return m


def token_mask(rows_h, nb: int, b: int, n: int | None = None) -> np.ndarray:
    """n x n boolean: token p may attend to token q iff block(q) is in N(block(p)).
    n defaults to nb * b; a shorter n drops the positions past the end."""
    m = np.kron(block_mask(rows_h, nb), np.ones((b, b), dtype=bool)).astype(bool)
    n = nb * b if n is None else n
    return m[:n, :n]
