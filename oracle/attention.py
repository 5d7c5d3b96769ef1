"""Oracle: masked softmax attention, forward and backward, in fp64 on the CPU.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Definition followed
-------------------
* Longformer: The Long-Document Transformer, §3.1 eq. (1): attention is
  softmax(Q K^T / sqrt(d_k)) V.  The scale is an argument here.
* Big Bird: Transformers for Longer Sequences, §2 eq. (AT): for each query the
  softmax runs over the key set N(i) only.  Keys outside the pattern get zero
  probability, which is the same as a score of -inf before the softmax.
* Same page, App. D Fig. 6: the blocked computation gives the same matrix as the
  plain pattern of Fig. 3(d), so the oracle is the plain definition on an
  explicit n x n mask, with no blocking.

The pages give no backward pass; the oracle takes the exact gradient of the
forward (chain rule through the row softmax, whose Jacobian-vector product is
dS = P * (dP - rowsum(P * dP))).

All arrays are numpy float64.  ``q, k, v, dout`` are [B, H, n, d].  A mask is
either a boolean array [n, n] (same for every head), [H, n, n], or a callable
``mask(h, p0, p1) -> bool[p1 - p0, n]`` giving rows p0..p1-1 of head h, so that
long sequences can be processed a band of rows at a time.
"""

from __future__ import annotations

import numpy as np


def _mask_rows(mask, h: int, p0: int, p1: int) -> np.ndarray:
    if callable(mask):
        return np.asarray(mask(h, p0, p1), dtype=bool)
    mask = np.asarray(mask, dtype=bool)
    if mask.ndim == 2:
        return mask[p0:p1]
    return mask[h, p0:p1]


def attention_probs(q_rows: np.ndarray, k: np.ndarray, mask_rows: np.ndarray,
                    scale: float):
    """Row-softmax probabilities and log-sum-exp for some query rows of one head.

    q_rows [m, d], k [n, d], mask_rows [m, n] -> (P [m, n], lse [m]), natural log.
    Every row must allow at least one key.
    """
    s = scale * (q_rows @ k.T)
    s = np.where(mask_rows, s, -np.inf)
    smax = s.max(axis=1, keepdims=True)
    e = np.exp(s - smax)          # exp(-inf) = 0 for masked keys
    z = e.sum(axis=1, keepdims=True)
    return e / z, smax[:, 0] + np.log(z[:, 0])


def attention_fwd(q, k, v, mask, scale: float, row_chunk: int = 2048):
    """Forward: O [B,H,n,d] and LSE [B,H,n] (natural log), fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    bsz, heads, n, d = q.shape
    out = np.zeros_like(q)
    lse = np.zeros((bsz, heads, n))
    for h in range(heads):
        for p0 in range(0, n, row_chunk):
            p1 = min(n, p0 + row_chunk)
            mrows = _mask_rows(mask, h, p0, p1)
            for bi in range(bsz):
                p, l_ = attention_probs(q[bi, h, p0:p1], k[bi, h], mrows, scale)
                out[bi, h, p0:p1] = p @ v[bi, h]
                lse[bi, h, p0:p1] = l_
    return out, lse


def attention_fwd_rows(q, k, v, mask, scale: float, bi: int, h: int, rows):
    """Forward for a few chosen query rows of one (batch, head): (O [m,d], lse [m])."""
    rows = np.asarray(rows)
    qf = np.asarray(q[bi, h], dtype=np.float64)
    kf = np.asarray(k[bi, h], dtype=np.float64)
    vf = np.asarray(v[bi, h], dtype=np.float64)
    mrows = np.concatenate([_mask_rows(mask, h, int(p), int(p) + 1) for p in rows])
    p, l_ = attention_probs(qf[rows], kf, mrows, scale)
    return p @ vf, l_


def attention_bwd(q, k, v, dout, mask, scale: float, row_chunk: int = 2048):
    """Backward: (dQ, dK, dV), each [B,H,n,d] fp64, for the loss <dout, O>."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    bsz, heads, n, d = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(heads):
        for p0 in range(0, n, row_chunk):
            p1 = min(n, p0 + row_chunk)
            mrows = _mask_rows(mask, h, p0, p1)
            for bi in range(bsz):
                p, _ = attention_probs(q[bi, h, p0:p1], k[bi, h], mrows, scale)
                do = dout[bi, h, p0:p1]
                dv[bi, h] += p.T @ do                      # O = P V
                dp = do @ v[bi, h].T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))   # softmax JVP
                dq[bi, h, p0:p1] = scale * (ds @ k[bi, h])            # S = scale Q K^T
                dk[bi, h] += scale * (ds.T @ q[bi, h, p0:p1])
    return dq, dk, dv
