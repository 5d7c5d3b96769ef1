"""Helpers shared by the GPU parity tests: seeded inputs on the device and the
matching fp64 values for the oracle."""

from __future__ import annotations

import sys

import numpy as np

from block_sparse_long_bsattn_amd import inputs as I

BF16_TOL = 2e-2    # max-abs, bf16 inputs with fp32 accumulation
F32_TOL = 1e-5     # max-abs, fp32 inputs


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device_tensor(host, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(host).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(host)).cuda()


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def qkv(shape, dtype, seeds=(I.SEED_Q, I.SEED_K, I.SEED_V), stds=None):
    """Device tensors and their exact fp64 values, one per seed (N(0, std^2) with
    stds[i], default 1)."""
    dev, ref = [], []
    for x, s in enumerate(seeds):
        h, r = I.make_tensor(s, shape, dtype, 1.0 if stds is None else stds[x])
        dev.append(device_tensor(h, dtype))
        ref.append(r)
    return dev, ref


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0


def half_ulp_bf16(ref):
    """Half the spacing of bf16 values at |ref|: the error of rounding ref to bf16
    (8 significand bits, so the spacing in [2^e, 2^(e+1)) is 2^(e-7))."""
    a = np.maximum(np.abs(np.asarray(ref, dtype=np.float64)), 2.0 ** -126)
    return 0.5 * 2.0 ** (np.floor(np.log2(a)) - 7)


def ulp_bound_excess(got, ref, tol=BF16_TOL):
    """max over elements of |got - ref| / (tol + half a bf16 ulp of |ref|): at most 1
    when every element is within tol of the exact value beyond the rounding a
    bf16 output cannot avoid."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) / (tol + half_ulp_bf16(ref))))
