#!/usr/bin/env python3
"""Throughput of block-sparse (BigBird-ITC) attention on one MI355X.

One step = the whole hot path over one batch of seeded synthetic input:
redraw the block layout on the device, forward, backward (dQ, dK, dV), for
batch 4, 12 heads, n = 4096, d = 64, b = 64, global blocks {0, 63}, w = 3, r = 3,
bf16 inputs with fp32 accumulation.  Prints ONE JSON line on stdout:

  value      useful TFLOP/s = (4 + 8) * d * (attended query-key pairs) / step time,
             the pairs counted exactly from the layout (set semantics)
  roofline   the kernel with the largest share of the step, timed with HIP events
             on its own stream, against the dense bf16 MFMA peak
  cpu_baseline  the fp64 oracle (dense mask) timed on a bounded sample on the
             host cores, in the same unit
  secondary  the other workloads (forward only at n = 4096 and 16384, fp32 at
             n = 512, Longformer window 256 + 64 global tokens forward, and its
             forward + backward, the same with separate projections for the
             global tokens, BigBird-etc base (256 added global tokens,
             blocks of 84) forward + backward, and the causal character-LM shape
             with dilation on two heads, forward + backward), each timed alone

Progress goes to stderr.  Inputs are resident in device memory before timing.

Before its warm-up steps each workload runs its own step untimed for --settle-ms
milliseconds (default 100): after the host-side setup (seconds of input
generation with the GPU idle) the step takes ~280 us and only reaches its steady
~230 us after ~150 steps, a power-management ramp of the idle device that a
training loop does not see.  The settle phase is reported in the JSON line.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0
D = 64
METRIC = "useful TFLOP/s and % bf16 MFMA peak, block-sparse attn fwd+bwd, n=4096"

WORKLOADS = {
    "bigbird_fwd_bwd_b4_h12_n4096": dict(kind="bigbird", n=4096, heads=12, batch=4,
                                          G=[0, 63], w=3, r=3, dtype="bf16", bwd=True),
    "bigbird_fwd_b2_h12_n4096": dict(kind="bigbird", n=4096, heads=12, batch=2,
                                      G=[0, 63], w=3, r=3, dtype="bf16", bwd=False),
    "bigbird_fwd_b1_h16_n16384": dict(kind="bigbird", n=16384, heads=16, batch=1,
                                       G=[0, 255], w=3, r=3, dtype="bf16", bwd=False),
    "bigbird_fwd_fp32_b1_h1_n512": dict(kind="bigbird", n=512, heads=1, batch=1,
                                         G=[0, 7], w=3, r=3, dtype="f32", bwd=False),
    "longformer_fwd_b1_h12_n4096_w256_g64": dict(kind="longformer", n=4096, heads=12, batch=1,
                                                  w1=256, G=list(range(64)), dtype="bf16",
                                                  bwd=False),
    "longformer_fwd_bwd_b1_h12_n4096_w256_g64": dict(kind="longformer", n=4096, heads=12,
                                                      batch=1, w1=256, G=list(range(64)),
                                                      dtype="bf16", bwd=True),
    # the same with separate projections for the global tokens' attention (Q_g, K_g, V_g)
    "longformer_gproj_fwd_bwd_b1_h12_n4096_w256_g64": dict(kind="longformer", n=4096, heads=12,
                                                            batch=1, w1=256, G=list(range(64)),
                                                            dtype="bf16", bwd=True, gproj=True),
    # BigBird-etc base: 256 added global tokens, blocks of 84, window of 3 blocks
    "etc_fwd_bwd_b4_h12_g256_n4096_b84": dict(kind="etc", g=256, n=4096, b=84, w=3, heads=12,
                                              batch=4, dtype="bf16", bwd=True),
    # character-LM shape: 8 heads, 256 earlier tokens, dilation 3 on two heads
    "longformer_causal_fwd_bwd_b1_h8_n23040_w256_dil3x2": dict(
        kind="longformer", n=23040, heads=8, batch=1, w1=256, G=[], dtype="bf16", bwd=True,
        dil=[3, 3, 0, 0, 0, 0, 0, 0], causal=True),
}
PRIMARY = "bigbird_fwd_bwd_b4_h12_n4096"

# useful FLOPs per attended (query, key) pair credited to each kernel
FLOPS_PER_PAIR = {"bs_fwd_bf16": 4 * D, "bs_fwd_f32": 4 * D, "bs_bwd_dq": 2 * D,
                  "bs_bwd_dkdv": 6 * D, "lf_attn": 4 * D, "lf_bwd_dq": 2 * D,
                  "lf_bwd_dkdv": 6 * D}
CSRC = os.path.join(ROOT, "block_sparse_long_bsattn_amd", "csrc")
# the sources a kernel's code and launch depend on: a stored traffic figure is only
# reported while none of them has changed since the counters were taken
KERNEL_SOURCES = {
    "bs_bwd_dkdv": ["bs_bwd.hip", "bs_bwd.hpp", "attn_tile.hpp", "common.hpp", "shape.hpp",
                    "internal.hpp", "abi.cpp", "fold.hpp"],
    "bs_bwd_dq": ["bs_bwd.hip", "bs_bwd.hpp", "attn_tile.hpp", "common.hpp", "shape.hpp",
                  "internal.hpp", "abi.cpp", "fold.hpp"],
    "bs_fwd_bf16": ["bs_fwd.hip", "attn_tile.hpp", "common.hpp", "shape.hpp", "internal.hpp",
                    "abi.cpp", "fold.hpp"],
    "lf_attn": ["lf_fwd.hip", "lf_tile.hpp", "attn_tile.hpp", "common.hpp", "shape.hpp",
                "internal.hpp", "abi.cpp", "fold.hpp"],
    "lf_bwd_dkdv": ["lf_bwd.hip", "lf_tile.hpp", "attn_tile.hpp", "common.hpp", "shape.hpp",
                    "internal.hpp", "abi.cpp", "fold.hpp"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(kernel: str) -> str | None:
    """sha256 over the kernel's source files (in the listed order), None if unknown."""
    files = KERNEL_SOURCES.get(kernel)
    if not files:
        return None
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


# ---------------------------------------------------------------------------
# device setup
# ---------------------------------------------------------------------------

class Job:
    """Device tensors, handle and pre-marshalled C-ABI calls for one workload."""

    def __init__(self, name: str, cfg: dict):
        import torch
        from block_sparse_long_bsattn_amd import _lib as B
        from block_sparse_long_bsattn_amd import inputs as I
        self.name, self.cfg, self.B = name, cfg, B
        lib = B.load()
        bsz, heads = cfg["batch"], cfg["heads"]
        n = cfg["n"] + cfg.get("g", 0) if cfg["kind"] == "etc" else cfg["n"]
        shape = (bsz, heads, n, D)
        tdt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32

        def dev(seed):
            host, _ = I.make_tensor(seed, shape, cfg["dtype"])
            if cfg["dtype"] == "bf16":
                return torch.from_numpy(host.view(np.int16)).view(torch.bfloat16).cuda()
            return torch.from_numpy(host).cuda()

        self.q, self.k, self.v = dev(I.SEED_Q), dev(I.SEED_K), dev(I.SEED_V)
        self.o = torch.empty(shape, dtype=tdt, device="cuda")
        self.lse = torch.empty((bsz, heads, n), dtype=torch.float32, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        self.stream = stream
        scale = ctypes.c_float(1.0 / math.sqrt(D))
        dt = B.BSATTN_BF16 if cfg["dtype"] == "bf16" else B.BSATTN_F32
        P = lambda t: ctypes.c_void_p(None if t is None else t.data_ptr())
        # training steps keep the rounding residual of O for an exact D in the
        # backward (bf16 only); forward-only steps do not write it
        self.olo = torch.empty(shape, dtype=tdt, device="cuda") \
            if cfg["bwd"] and cfg["dtype"] == "bf16" else None
        self.calls = []
        if cfg["kind"] == "bigbird":
            self.seed = I.SEED_LAYOUT
            self.handle = B.bsattn_layout_build(n, 64, heads, cfg["G"], cfg["w"], cfg["r"],
                                                self.seed)
            nb, _, nnzb = B.bsattn_layout_info(self.handle)
            self.pairs = bsz * nnzb * 64 * 64
            wsf = B.bsattn_fwd_workspace(self.handle, bsz)
            self.wsf = torch.empty(max(16, wsf), dtype=torch.uint8, device="cuda")
            # validate shapes once through the checked binding
            B.bsattn_fwd(self.handle, self.q, self.k, self.v, self.o, self.lse, self.wsf,
                         o_lo=self.olo)
            h = ctypes.c_void_p(self.handle)
            self.calls.append((lib.bsattn_layout_rebuild, (h, ctypes.c_uint64(self.seed), stream)))
            self.calls.append((lib.bsattn_fwd, (h, bsz, D, dt, scale, P(self.q), P(self.k),
                                                P(self.v), P(self.o), P(self.lse), P(self.olo),
                                                P(self.wsf), self.wsf.numel(), stream)))
            self.flops = 4 * D * self.pairs
            if cfg["bwd"]:
                self.do = dev(I.SEED_DO)
                self.dq, self.dk, self.dv = (torch.empty_like(self.q) for _ in range(3))
                wsb = B.bsattn_bwd_workspace(self.handle, bsz)
                self.wsb = torch.empty(max(16, wsb), dtype=torch.uint8, device="cuda")
                B.bsattn_bwd(self.handle, self.q, self.k, self.v, self.o, self.lse, self.do,
                             self.dq, self.dk, self.dv, self.wsb, o_lo=self.olo)
                self.calls.append((lib.bsattn_bwd, (h, bsz, D, dt, scale, P(self.q), P(self.k),
                                                    P(self.v), P(self.o), P(self.olo),
                                                    P(self.lse), P(self.do), P(self.dq),
                                                    P(self.dk), P(self.dv), P(self.wsb),
                                                    self.wsb.numel(), stream)))
                self.flops += 8 * D * self.pairs
        else:
            dil = cfg.get("dil")
            causal = cfg.get("causal", False)
            if cfg["kind"] == "etc":
                self.handle = B.lfattn_plan_build_etc(cfg["g"], cfg["n"], cfg["b"], cfg["w"])
                self.pairs = bsz * heads * etc_pairs(cfg["g"], cfg["n"], cfg["b"], cfg["w"])
            elif dil is None and not causal:
                self.handle = B.lfattn_plan_build(n, cfg["w1"], cfg["G"])
            else:
                self.handle = B.lfattn_plan_build_dilated(n, cfg["w1"], cfg["G"], heads, dil,
                                                          causal)
            if cfg["kind"] != "etc":
                self.pairs = bsz * sum(longformer_pairs(n, cfg["w1"], cfg["G"],
                                                        dil[h] if dil else 0, causal)
                                       for h in range(heads))
            ws = B.lfattn_fwd_workspace(self.handle, bsz, heads)
            self.wsf = torch.empty(max(16, ws), dtype=torch.uint8, device="cuda")
            h = ctypes.c_void_p(self.handle)
            gproj = cfg.get("gproj", False)
            if gproj:   # the global tokens' projections, seeded after the others
                self.qg, self.kg, self.vg = (dev(I.SEED_DO + x) for x in (1, 2, 3))
                B.lfattn_fwd_gproj(self.handle, self.q, self.k, self.v, self.qg, self.kg, self.vg,
                                   self.o, self.lse, self.wsf, o_lo=self.olo)
                self.calls.append((lib.lfattn_fwd_gproj, (
                    h, bsz, heads, D, dt, scale, P(self.q), P(self.k), P(self.v), P(self.qg),
                    P(self.kg), P(self.vg), P(self.o), P(self.lse), P(self.olo), P(self.wsf),
                    self.wsf.numel(), stream)))
            else:
                B.lfattn_fwd(self.handle, self.q, self.k, self.v, self.o, self.lse, self.wsf,
                             o_lo=self.olo)
                self.calls.append((lib.lfattn_fwd, (
                    h, bsz, heads, D, dt, scale, P(self.q), P(self.k), P(self.v), P(self.o),
                    P(self.lse), P(self.olo), P(self.wsf), self.wsf.numel(), stream)))
            self.flops = 4 * D * self.pairs
            if cfg["bwd"]:
                self.do = dev(I.SEED_DO)
                self.dq, self.dk, self.dv = (torch.empty_like(self.q) for _ in range(3))
                wsb = B.lfattn_bwd_workspace(self.handle, bsz, heads)
                self.wsb = torch.empty(max(16, wsb), dtype=torch.uint8, device="cuda")
                if gproj:
                    self.dqg, self.dkg, self.dvg = (torch.empty_like(self.q) for _ in range(3))
                    B.lfattn_bwd_gproj(self.handle, self.q, self.k, self.v, self.qg, self.kg,
                                       self.vg, self.o, self.lse, self.do, self.dq, self.dk,
                                       self.dv, self.dqg, self.dkg, self.dvg, self.wsb,
                                       o_lo=self.olo)
                    self.calls.append((lib.lfattn_bwd_gproj, (
                        h, bsz, heads, D, dt, scale, P(self.q), P(self.k), P(self.v), P(self.qg),
                        P(self.kg), P(self.vg), P(self.o), P(self.olo), P(self.lse), P(self.do),
                        P(self.dq), P(self.dk), P(self.dv), P(self.dqg), P(self.dkg),
                        P(self.dvg), P(self.wsb), self.wsb.numel(), stream)))
                else:
                    B.lfattn_bwd(self.handle, self.q, self.k, self.v, self.o, self.lse, self.do,
                                 self.dq, self.dk, self.dv, self.wsb, o_lo=self.olo)
                    self.calls.append((lib.lfattn_bwd, (
                        h, bsz, heads, D, dt, scale, P(self.q), P(self.k), P(self.v), P(self.o),
                        P(self.olo), P(self.lse), P(self.do), P(self.dq), P(self.dk), P(self.dv),
                        P(self.wsb), self.wsb.numel(), stream)))
                self.flops += 8 * D * self.pairs
        torch.cuda.synchronize()

    def step(self):
        for fn, args in self.calls:
            st = fn(*args)
            if st != 0:
                raise RuntimeError(f"{fn.__name__} failed: {self.B.bsattn_last_error()}")

    def close(self):
        if self.cfg["kind"] == "bigbird":
            self.B.bsattn_layout_destroy(self.handle)
        else:
            self.B.lfattn_plan_destroy(self.handle)


def longformer_pairs(n: int, w1: int, G, dil: int = 0, causal: bool = False) -> int:
    """Attended (query, key) pairs of one head: q in p's window (q = p + k*(dil+1),
    k in [-w1, w1], or [-w1, 0] when causal), or p or q global."""
    s = dil + 1
    p = np.arange(n)
    idx = p // s                          # index of p within its residue class
    nc = (n - p % s + s - 1) // s         # length of that class
    win = np.minimum(w1, idx) + 1
    if not causal:
        win = win + np.minimum(w1, nc - 1 - idx)
    if len(G) == 0:
        return int(win.sum())
    gpos = np.asarray(sorted(G), dtype=np.int64)
    g = np.zeros(n, dtype=bool)
    g[gpos] = True
    lo = 0 if causal else -w1 * s
    total = 0
    for x in range(n):
        if g[x]:
            total += n
            continue
        delta = x - gpos
        inside = (delta % s == 0) & (delta >= lo) & (delta <= w1 * s)
        total += int(win[x]) + int(np.count_nonzero(~inside))
    return total


def etc_pairs(g: int, n: int, b: int, w: int) -> int:
    """Attended pairs of one head of the ETC pattern: g full rows of g + n keys; an
    ordinary token of block k sees the g global tokens and the blocks within
    (w-1)/2 of k (the last block holds n - b*(nb-1) tokens)."""
    nb = -(-n // b)
    size = [min(b, n - b * j) for j in range(nb)]
    half = (w - 1) // 2
    total = g * (g + n)
    for k in range(nb):
        total += size[k] * (g + sum(size[max(0, k - half):min(nb, k + half + 1)]))
    return total


def settle(job: Job, ms: float) -> int:
    """Run the workload's step untimed for `ms` milliseconds of wall time (the
    device's clocks ramp up after the idle setup phase); returns the steps run."""
    import torch
    t0 = time.perf_counter()
    k = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        job.step()
        k += 1
        if k % 20 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return k


def time_steps(job: Job, steps: int, warmup: int):
    import torch
    for _ in range(warmup):
        job.step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        job.step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def kernel_breakdown(job: Job, steps: int):
    """Per-kernel (launches, avg ms) over `steps` further steps, HIP events on the
    launch stream."""
    import torch
    B = job.B
    B.bsattn_profile_read()          # drop anything pending
    B.bsattn_profile_enable(True)
    try:
        for _ in range(steps):
            job.step()
        torch.cuda.synchronize()
        rep = B.bsattn_profile_read()
    finally:
        B.bsattn_profile_enable(False)
    return {k: {"launches": c, "avg_ms": ms / max(1, c)} for k, (c, ms) in rep.items()}


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they were
    taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256") != kernel_source_hash(kernel):
        return None
    return t.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands, on a bounded sample
# ---------------------------------------------------------------------------

def cpu_baseline(cfg: dict, budget_s: float):
    from block_sparse_long_bsattn_amd import inputs as I
    from oracle import attention as OA
    from oracle import layout as OL
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    n, heads = cfg["n"], cfg["heads"]
    lay = OL.build_layout(n, 64, heads, cfg["G"], cfg["w"], cfg["r"], I.SEED_LAYOUT)
    nb = n // 64
    shape = (cfg["batch"], heads, n, D)
    qa = I.make_tensor(I.SEED_Q, shape, "bf16")[1]
    ka = I.make_tensor(I.SEED_K, shape, "bf16")[1]
    va = I.make_tensor(I.SEED_V, shape, "bf16")[1]
    doa = I.make_tensor(I.SEED_DO, shape, "bf16")[1]
    flops = 0
    t_total = 0.0
    done = 0
    for bh in range(cfg["batch"] * heads):
        bi, h = divmod(bh, heads)
        rows = lay["rows"][h]

        def mask(hh, p0, p1, rows=rows):
            blk = np.zeros((p1 - p0, nb), dtype=bool)
            for p in range(p0, p1):
                blk[p - p0, rows[p // 64]] = True
            return np.repeat(blk, 64, axis=1)

        sl = (slice(bi, bi + 1), slice(h, h + 1))
        q, k, v, do = qa[sl], ka[sl], va[sl], doa[sl]
        t0 = time.perf_counter()
        OA.attention_fwd(q, k, v, mask, 1 / math.sqrt(D))
        if cfg["bwd"]:
            OA.attention_bwd(q, k, v, do, mask, 1 / math.sqrt(D))
        t_total += time.perf_counter() - t0
        pairs = sum(len(r) for r in rows) * 64 * 64
        flops += (12 if cfg["bwd"] else 4) * D * pairs
        done += 1
        if t_total >= budget_s:
            break
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {cfg['batch'] * heads} (batch, head) slices of the same "
                      f"workload, fp64 dense-mask forward{' + backward' if cfg['bwd'] else ''}, "
                      f"{t_total:.1f} s"}


# ---------------------------------------------------------------------------
# Results table: every configured single-pass workload on the GPU, next to the
# oracle on the same inputs (max-abs error) and the oracle's own time on one host
# thread (median of three full runs where that fits in about a minute)
# ---------------------------------------------------------------------------

# (workload, part of it given to the oracle, three timed oracle runs (else one))
TABLE_WORKLOADS = [
    ("bigbird_fwd_fp32_b1_h1_n512", "all", True),
    ("bigbird_fwd_b2_h12_n4096", "all", True),
    ("bigbird_fwd_b1_h16_n16384", "all", False),
    ("bigbird_fwd_bwd_b4_h12_n4096", "all", False),
    ("longformer_fwd_b1_h12_n4096_w256_g64", "all", True),
]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def oracle_mask(cfg: dict):
    """Mask callback (h, p0, p1) of a workload's token pattern."""
    from block_sparse_long_bsattn_amd import inputs as I
    from oracle import layout as OL
    from oracle import longformer as OLF
    if cfg["kind"] == "longformer":
        return OLF.longformer_mask(cfg["n"], cfg["w1"], cfg["G"])
    n = cfg["n"]
    nb = n // 64
    lay = OL.build_layout(n, 64, cfg["heads"], cfg["G"], cfg["w"], cfg["r"], I.SEED_LAYOUT)

    def mask(h, p0, p1):
        blk = np.zeros((p1 - p0, nb), dtype=bool)
        for p in range(p0, p1):
            blk[p - p0, lay["rows"][h][p // 64]] = True
        return np.repeat(blk, 64, axis=1)
    return mask


def results_table(steps: int, warmup: int, settle_ms: float) -> dict:
    import torch
    from threadpoolctl import threadpool_limits
    from block_sparse_long_bsattn_amd import inputs as I
    from oracle import attention as OA
    rows = []
    for name, part, time_full in TABLE_WORKLOADS:
        cfg = WORKLOADS[name]
        log(f"table: {name}")
        job = Job(name, cfg)
        settle(job, settle_ms)
        ms, _ = time_steps(job, steps, warmup)
        job.step()
        torch.cuda.synchronize()
        got = {"o": job.o, "lse": job.lse}
        if cfg["bwd"]:
            got.update(dq=job.dq, dk=job.dk, dv=job.dv)
        got = {k: v.float().cpu().numpy().astype(np.float64) for k, v in got.items()}
        flops = job.flops
        job.close()
        shape = (cfg["batch"], cfg["heads"], cfg["n"], D)
        q, k, v, do = (I.make_tensor(sd, shape, cfg["dtype"])[1]
                       for sd in (I.SEED_Q, I.SEED_K, I.SEED_V, I.SEED_DO))
        mask = oracle_mask(cfg)
        scale = 1 / math.sqrt(D)
        sl = (slice(None), slice(None)) if part == "all" else (slice(0, 1), slice(0, 1))
        mh = mask if part == "all" else (lambda _h, p0, p1: mask(0, p0, p1))
        secs = []
        with threadpool_limits(1):
            for _ in range(3 if time_full else 1):
                t0 = time.perf_counter()
                ro, rl = OA.attention_fwd(q[sl], k[sl], v[sl], mh, scale)
                ref = [ro, rl]
                if cfg["bwd"]:
                    ref += list(OA.attention_bwd(q[sl], k[sl], v[sl], do[sl], mh, scale))
                secs.append(time.perf_counter() - t0)
                log(f"  oracle run {len(secs)}: {secs[-1]:.2f} s")
        names = ["o", "lse"] + (["dq", "dk", "dv"] if cfg["bwd"] else [])
        err = max(float(np.max(np.abs(got[nm][sl] - r))) for nm, r in zip(names, ref))
        peak = PEAK_BF16_TFLOPS if cfg["dtype"] == "bf16" else PEAK_FP32_TFLOPS
        tfl = flops / (ms * 1e-3) / 1e12
        rows.append({"workload": name, "gpu_us_per_step": round(ms * 1e3, 2),
                     "useful_tflops": round(tfl, 2), "pct_peak": round(100 * tfl / peak, 2),
                     "max_abs_vs_oracle": err, "oracle_part": part,
                     "oracle_s_1thread": round(float(np.median(secs)), 3),
                     "oracle_runs": len(secs)})
        log(f"  {ms * 1e3:.1f} us, {tfl:.1f} TFLOP/s, max-abs {err:.2e}, oracle "
            f"{np.median(secs):.2f} s ({part}, 1 thread)")
    return {"cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(), "rows": rows}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed steps for this long before the warm-up steps (clock ramp)")
    ap.add_argument("--table", action="store_true",
                    help="print only the per-workload table (GPU time, error against the "
                         "oracle, oracle time on one host thread) as one JSON line")
    ap.add_argument("--workload", default=PRIMARY, choices=sorted(WORKLOADS))
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_mib > 0:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.copy_mib} MiB")
        del src, dst

    if args.table:
        print(json.dumps(results_table(args.steps, args.warmup, args.settle_ms)), flush=True)
        return 0

    cfg = WORKLOADS[args.workload]
    log(f"workload {args.workload}: setting up")
    job = Job(args.workload, cfg)
    settled = settle(job, args.settle_ms)
    ms, wall = time_steps(job, args.steps, args.warmup)
    log(f"  {ms * 1e3:.1f} us/step (wall clock {wall * 1e6 / args.steps:.1f} us/step)")
    kb = kernel_breakdown(job, args.steps)
    for k, v in sorted(kb.items(), key=lambda kv: -kv[1]["avg_ms"] * kv[1]["launches"]):
        log(f"  kernel {k:20s} {v['launches']:5d} launches  avg {v['avg_ms'] * 1e3:8.2f} us")
    value = job.flops / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if cfg["dtype"] == "bf16" else PEAK_FP32_TFLOPS

    # dominant kernel: largest summed time among the ones that carry the FLOPs
    cand = {k: v for k, v in kb.items() if k in FLOPS_PER_PAIR}
    dom = max(cand, key=lambda k: cand[k]["avg_ms"] * cand[k]["launches"])
    per_launch_flops = FLOPS_PER_PAIR[dom] * job.pairs
    achieved = per_launch_flops / (cand[dom]["avg_ms"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": load_traffic(dom, args.workload), "kernel": dom,
                "flops_per_launch": per_launch_flops}

    secondary = {}
    if not args.no_secondary:
        for name, c2 in WORKLOADS.items():
            if name == args.workload:
                continue
            log(f"workload {name}")
            j2 = Job(name, c2)
            settle(j2, args.settle_ms)
            ms2, _ = time_steps(j2, args.steps, args.warmup)
            kb2 = kernel_breakdown(j2, max(5, args.steps // 5))
            pk2 = PEAK_BF16_TFLOPS if c2["dtype"] == "bf16" else PEAK_FP32_TFLOPS
            v2 = j2.flops / (ms2 * 1e-3) / 1e12
            secondary[name] = {"useful_tflops": round(v2, 2), "pct_peak": round(100 * v2 / pk2, 2),
                               "us_per_step": round(ms2 * 1e3, 2),
                               "kernels_us": {k: round(v["avg_ms"] * 1e3, 2) for k, v in kb2.items()}}
            log(f"  {ms2 * 1e3:.1f} us/step, {v2:.1f} useful TFLOP/s")
            j2.close()

    cpu = None
    if not args.no_cpu:
        log("cpu baseline: oracle")
        cpu = cpu_baseline(cfg, args.cpu_budget)
        log(f"  {cpu['value'] * 1e3:.3f} GFLOP/s on {cpu['cores']} threads")

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"ms": args.settle_ms, "steps": settled},
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": cfg["batch"], "heads": cfg["heads"],
                   "seq_len": cfg["n"], "head_dim": D,
                   **({"block": 64, "global_blocks": cfg["G"], "window_blocks": cfg["w"],
                       "random_blocks": cfg["r"], "passes": "layout+fwd+bwd" if cfg["bwd"] else "layout+fwd"}
                      if cfg["kind"] == "bigbird" else
                      {"added_global_tokens": cfg["g"], "block": cfg["b"], "window_blocks": cfg["w"],
                       "passes": "fwd+bwd" if cfg["bwd"] else "fwd"} if cfg["kind"] == "etc" else
                      {"window_one_side": cfg["w1"], "global_tokens": len(cfg["G"]),
                       "dilation": cfg.get("dil", 0), "causal": cfg.get("causal", False),
                       "global_projections": cfg.get("gproj", False),
                       "passes": "fwd+bwd" if cfg["bwd"] else "fwd"})},
        "pct_peak": round(100 * value / peak, 3),
        "useful_pairs": job.pairs,
        "kernels_us": {k: round(v["avg_ms"] * 1e3, 2) for k, v in kb.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    job.close()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
