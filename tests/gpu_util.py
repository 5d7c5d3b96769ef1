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


def qkv(shape, dtype, seeds=(I.SEED_Q, I.SEED_K, I.SEED_V)):
    """Device tensors and their exact fp64 values, one per seed."""
    dev, ref = [], []
    for s in seeds:
        h, r = I.make_tensor(s, shape, dtype)
        dev.append(device_tensor(h, dtype))
        ref.append(r)
    return dev, ref


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
