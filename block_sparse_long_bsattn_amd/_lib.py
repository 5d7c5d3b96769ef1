"""ctypes binding of libbsattn.so; same names as the C ABI in include/bsattn.h.

Argument marshalling only: tensors are passed by device pointer
(``tensor.data_ptr()``), streams by their HIP handle, and a non-OK status is
raised as :class:`BsattnError`.  All attention work runs in the library's HIP
kernels; if the library is missing this module raises instead of falling back.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_uint64, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbsattn.so")

BSATTN_OK = 0
BSATTN_EINVAL = -1
BSATTN_EUNSUPPORTED = -2
BSATTN_EHIP = -3
BSATTN_ENOMEM = -4
BSATTN_F32 = 0
BSATTN_BF16 = 1
BSATTN_BWD_NOALLOC_SCRATCH_BYTES = 64 << 20   # static scratch of bsattn_bwd_noalloc

# every exported symbol declared in include/bsattn.h
EXPORTS = (
    "bsattn_layout_build", "bsattn_layout_rebuild", "bsattn_layout_info",
    "bsattn_layout_to_host", "bsattn_layout_destroy", "bsattn_fwd_workspace",
    "bsattn_bwd_workspace", "bsattn_fwd", "bsattn_bwd", "bsattn_bwd_noalloc",
    "lfattn_plan_build",
    "lfattn_plan_build_dilated", "lfattn_plan_build_etc", "lfattn_plan_destroy",
    "lfattn_fwd_workspace", "lfattn_fwd", "lfattn_bwd_workspace", "lfattn_bwd",
    "lfattn_fwd_gproj", "lfattn_bwd_gproj", "bsattn_status_str",
    "bsattn_last_error", "bsattn_version", "bsattn_profile_enable", "bsattn_profile_read",
)


class BsattnError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {status_name(status)} ({status}): {message}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libbsattn.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m block_sparse_long_bsattn_amd.build` "
            "(the attention path runs only in the HIP library; there is no fallback)")
    # PyTorch ships its own HIP runtime and the tensors handed to the library live
    # in it; importing torch first makes the library bind to that runtime instead
    # of loading the system one beside it (two runtimes in one process do not share
    # devices, memory or streams)
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    sig = {
        "bsattn_layout_build": (c_int, [c_int, c_int, c_int, POINTER(c_int32), c_int, c_int, c_int,
                                        c_uint64, c_void_p, POINTER(c_void_p)]),
        "bsattn_layout_rebuild": (c_int, [c_void_p, c_uint64, c_void_p]),
        "bsattn_layout_info": (c_int, [c_void_p, POINTER(c_int), POINTER(c_int), POINTER(c_int64)]),
        "bsattn_layout_to_host": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
        "bsattn_layout_destroy": (c_int, [c_void_p]),
        "bsattn_fwd_workspace": (c_size_t, [c_void_p, c_int, c_int]),
        "bsattn_bwd_workspace": (c_size_t, [c_void_p, c_int, c_int]),
        "bsattn_fwd": (c_int, [c_void_p, c_int, c_int, c_int, c_float] + [c_void_p] * 7
                       + [c_size_t, c_void_p]),
        "bsattn_bwd": (c_int, [c_void_p, c_int, c_int, c_int, c_float] + [c_void_p] * 11
                       + [c_size_t, c_void_p]),
        "bsattn_bwd_noalloc": (c_int, [c_void_p, c_int, c_int, c_int, c_float] + [c_void_p] * 10
                               + [c_void_p]),
        "lfattn_plan_build": (c_int, [c_int, c_int, POINTER(c_int32), c_int, c_void_p,
                                      POINTER(c_void_p)]),
        "lfattn_plan_build_dilated": (c_int, [c_int, c_int, POINTER(c_int32), c_int, c_int,
                                              POINTER(c_int32), c_int, c_void_p,
                                              POINTER(c_void_p)]),
        "lfattn_plan_build_etc": (c_int, [c_int, c_int, c_int, c_int, c_void_p,
                                          POINTER(c_void_p)]),
        "lfattn_plan_destroy": (c_int, [c_void_p]),
        "lfattn_fwd_workspace": (c_size_t, [c_void_p, c_int, c_int, c_int]),
        "lfattn_fwd": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_float] + [c_void_p] * 7
                       + [c_size_t, c_void_p]),
        "lfattn_bwd_workspace": (c_size_t, [c_void_p, c_int, c_int, c_int]),
        "lfattn_bwd": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_float] + [c_void_p] * 11
                       + [c_size_t, c_void_p]),
        "lfattn_fwd_gproj": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_float]
                             + [c_void_p] * 10 + [c_size_t, c_void_p]),
        "lfattn_bwd_gproj": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_float]
                             + [c_void_p] * 17 + [c_size_t, c_void_p]),
        "bsattn_status_str": (c_char_p, [c_int]),
        "bsattn_last_error": (c_char_p, []),
        "bsattn_version": (c_char_p, []),
        "bsattn_profile_enable": (c_int, [c_int]),
        "bsattn_profile_read": (c_int, [c_int, c_void_p, c_void_p, c_void_p, POINTER(c_int)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_name(status: int) -> str:
    return {0: "BSATTN_OK", -1: "BSATTN_EINVAL", -2: "BSATTN_EUNSUPPORTED",
            -3: "BSATTN_EHIP", -4: "BSATTN_ENOMEM"}.get(status, "BSATTN_UNKNOWN")


def _check(status: int, where: str) -> None:
    if status != BSATTN_OK:
        raise BsattnError(status, where, load().bsattn_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BSATTN_BF16
    if t.dtype == torch.float32:
        return BSATTN_F32
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _check_tensors(where, shape, dtype, named, lse=None, workspace=None, ws_need=0,
                   o_lo=None):
    """Host-side guard: every tensor is a contiguous GPU tensor of the exact shape
    the kernels index, so no launch can read or write past a buffer."""
    import torch
    if o_lo is not None:
        if dtype != torch.bfloat16:
            raise ValueError(f"{where}: o_lo is for bf16 tensors only")
        named = tuple(named) + (("o_lo", o_lo),)
    for name, t in named:
        if t is None:
            raise ValueError(f"{where}: {name} is None")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{where}: {name} must be a contiguous GPU tensor")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{where}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.dtype != dtype:
            raise ValueError(f"{where}: {name} has dtype {t.dtype}, expected {dtype}")
    if lse is not None:
        if not lse.is_cuda or not lse.is_contiguous() or lse.dtype != torch.float32 \
                or tuple(lse.shape) != tuple(shape[:3]):
            raise ValueError(f"{where}: lse must be a contiguous float32 GPU tensor of shape "
                             f"{tuple(shape[:3])}")
    if ws_need > 0:
        if workspace is None or not workspace.is_cuda or not workspace.is_contiguous() or \
                workspace.numel() * workspace.element_size() < ws_need:
            raise ValueError(f"{where}: workspace must be a contiguous GPU buffer of at least "
                             f"{ws_need} bytes")


_plan_n = {}


def _int32_array(values):
    vals = [int(x) for x in values]
    return (c_int32 * max(1, len(vals)))(*vals), len(vals)


# --- layout -------------------------------------------------------------------

_layout_n = {}   # layout handle -> sequence length it was built for


def bsattn_layout_build(n, b, heads, global_blocks, w, r, seed, stream=None) -> int:
    """Returns an opaque layout handle (an int); free it with bsattn_layout_destroy."""
    arr, g = _int32_array(global_blocks)
    out = c_void_p()
    _check(load().bsattn_layout_build(n, b, heads, arr if g else None, g, w, r,
                                      c_uint64(seed & (2**64 - 1)), _stream(stream),
                                      ctypes.byref(out)), "bsattn_layout_build")
    _layout_n[out.value] = n
    return out.value


def _layout_len(layout, nb):
    """Sequence length of a layout (tensors are [B, H, n, d]); nb * 64 if unknown."""
    return _layout_n.get(layout, nb * 64)


def bsattn_layout_rebuild(layout, seed, stream=None) -> None:
    _check(load().bsattn_layout_rebuild(layout, c_uint64(seed & (2**64 - 1)), _stream(stream)),
           "bsattn_layout_rebuild")


def bsattn_layout_info(layout):
    """(nb, heads, nnzb_total)."""
    nb, heads, nnz = c_int(), c_int(), c_int64()
    _check(load().bsattn_layout_info(layout, ctypes.byref(nb), ctypes.byref(heads),
                                     ctypes.byref(nnz)), "bsattn_layout_info")
    return nb.value, heads.value, nnz.value


def bsattn_layout_to_host(layout):
    """(row_ptr, col_idx, csc_ptr, csc_idx) as numpy int32 arrays (synchronous)."""
    import numpy as np
    nb, heads, nnz = bsattn_layout_info(layout)
    rp = np.zeros(heads * nb + 1, dtype=np.int32)
    ci = np.zeros(max(1, nnz), dtype=np.int32)
    cp = np.zeros(heads * nb + 1, dtype=np.int32)
    cs = np.zeros(max(1, nnz), dtype=np.int32)
    _check(load().bsattn_layout_to_host(layout, rp.ctypes.data, ci.ctypes.data, cp.ctypes.data,
                                        cs.ctypes.data), "bsattn_layout_to_host")
    return rp, ci[:nnz], cp, cs[:nnz]


def bsattn_layout_destroy(layout) -> None:
    _check(load().bsattn_layout_destroy(layout), "bsattn_layout_destroy")
    _layout_n.pop(layout, None)


# --- BigBird forward / backward -------------------------------------------------

def bsattn_fwd_workspace(layout, batch, d=64) -> int:
    return int(load().bsattn_fwd_workspace(layout, batch, d))


def bsattn_bwd_workspace(layout, batch, d=64) -> int:
    return int(load().bsattn_bwd_workspace(layout, batch, d))


def bsattn_fwd(layout, q, k, v, o, lse=None, workspace=None, scale=None, stream=None,
               o_lo=None) -> None:
    """Tensors [B, H, n, d] on the GPU (bf16 or fp32); lse float32 [B, H, n] or None;
    o_lo (bf16 only) receives the rounding residual of O, or None."""
    bsz, _, _, d = q.shape
    nb, heads, _ = bsattn_layout_info(layout)
    shape = (bsz, heads, _layout_len(layout, nb), d)
    need = bsattn_fwd_workspace(layout, bsz, d)   # covers both dtypes
    _check_tensors("bsattn_fwd", shape, q.dtype, (("q", q), ("k", k), ("v", v), ("o", o)),
                   lse, workspace, need, o_lo)
    scale = d ** -0.5 if scale is None else scale
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().bsattn_fwd(layout, bsz, d, _dtype_code(q), c_float(scale), _ptr(q), _ptr(k),
                             _ptr(v), _ptr(o), _ptr(lse), _ptr(o_lo), _ptr(workspace), ws_bytes,
                             _stream(stream)), "bsattn_fwd")


def bsattn_bwd(layout, q, k, v, o, lse, dout, dq, dk, dv, workspace=None, scale=None,
               stream=None, o_lo=None) -> None:
    """o_lo: the forward's rounding residual of O, or None."""
    bsz, _, _, d = q.shape
    nb, heads, _ = bsattn_layout_info(layout)
    shape = (bsz, heads, _layout_len(layout, nb), d)
    if lse is None:
        raise ValueError("bsattn_bwd: lse is required")
    _check_tensors("bsattn_bwd", shape, q.dtype,
                   (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq),
                    ("dk", dk), ("dv", dv)), lse, workspace, bsattn_bwd_workspace(layout, bsz, d),
                   o_lo)
    scale = d ** -0.5 if scale is None else scale
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().bsattn_bwd(layout, bsz, d, _dtype_code(q), c_float(scale), _ptr(q), _ptr(k),
                             _ptr(v), _ptr(o), _ptr(o_lo), _ptr(lse), _ptr(dout), _ptr(dq),
                             _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, _stream(stream)),
           "bsattn_bwd")


def bsattn_bwd_noalloc(layout, q, k, v, o, lse, dout, dq, dk, dv, scale=None, stream=None,
                       o_lo=None) -> None:
    """bsattn_bwd with the library's static device scratch instead of a workspace
    (no allocation; calls that overlap on one device race)."""
    bsz, _, _, d = q.shape
    nb, heads, _ = bsattn_layout_info(layout)
    shape = (bsz, heads, _layout_len(layout, nb), d)
    if lse is None:
        raise ValueError("bsattn_bwd_noalloc: lse is required")
    _check_tensors("bsattn_bwd_noalloc", shape, q.dtype,
                   (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq),
                    ("dk", dk), ("dv", dv)), lse, None, 0, o_lo)
    scale = d ** -0.5 if scale is None else scale
    _check(load().bsattn_bwd_noalloc(layout, bsz, d, _dtype_code(q), c_float(scale), _ptr(q),
                                     _ptr(k), _ptr(v), _ptr(o), _ptr(o_lo), _ptr(lse),
                                     _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream)),
           "bsattn_bwd_noalloc")


# --- Longformer -----------------------------------------------------------------

def lfattn_plan_build(n, window_one_side, global_tokens, stream=None) -> int:
    arr, ng = _int32_array(global_tokens)
    out = c_void_p()
    _check(load().lfattn_plan_build(n, window_one_side, arr if ng else None, ng,
                                    _stream(stream), ctypes.byref(out)), "lfattn_plan_build")
    _plan_n[out.value] = n
    return out.value


def lfattn_plan_build_dilated(n, window_one_side, global_tokens, heads, dilation=None,
                              causal=False, stream=None) -> int:
    """Plan with one dilation per head (None: 0 for every head) and the optional
    causal window; calls must pass the same head count."""
    arr, ng = _int32_array(global_tokens)
    dil = None
    if dilation is not None:
        dil, nd = _int32_array(dilation)
        if nd != heads:
            raise ValueError("lfattn_plan_build_dilated: need one dilation per head")
    out = c_void_p()
    _check(load().lfattn_plan_build_dilated(n, window_one_side, arr if ng else None, ng, heads,
                                            dil, 1 if causal else 0, _stream(stream),
                                            ctypes.byref(out)), "lfattn_plan_build_dilated")
    _plan_n[out.value] = n
    return out.value


def lfattn_plan_build_etc(g, n, b, w, stream=None) -> int:
    """BigBird-ETC plan: g added global tokens, then n ordinary tokens in blocks of b
    with a window of w blocks; tensors hold g + n tokens."""
    out = c_void_p()
    _check(load().lfattn_plan_build_etc(g, n, b, w, _stream(stream), ctypes.byref(out)),
           "lfattn_plan_build_etc")
    _plan_n[out.value] = g + n
    return out.value


def lfattn_plan_destroy(plan) -> None:
    _check(load().lfattn_plan_destroy(plan), "lfattn_plan_destroy")
    _plan_n.pop(plan, None)


def lfattn_fwd_workspace(plan, batch, heads, d=64) -> int:
    return int(load().lfattn_fwd_workspace(plan, batch, heads, d))


def lfattn_fwd(plan, q, k, v, o, lse=None, workspace=None, scale=None, stream=None,
               o_lo=None) -> None:
    bsz, heads, _, d = q.shape
    if plan not in _plan_n:
        raise ValueError("lfattn_fwd: unknown plan handle")
    shape = (bsz, heads, _plan_n[plan], d)
    _check_tensors("lfattn_fwd", shape, q.dtype, (("q", q), ("k", k), ("v", v), ("o", o)),
                   lse, workspace, lfattn_fwd_workspace(plan, bsz, heads, d), o_lo)
    scale = d ** -0.5 if scale is None else scale
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().lfattn_fwd(plan, bsz, heads, d, _dtype_code(q), c_float(scale), _ptr(q),
                             _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(o_lo), _ptr(workspace),
                             ws_bytes, _stream(stream)), "lfattn_fwd")


def lfattn_bwd_workspace(plan, batch, heads, d=64) -> int:
    return int(load().lfattn_bwd_workspace(plan, batch, heads, d))


def lfattn_bwd(plan, q, k, v, o, lse, dout, dq, dk, dv, workspace=None, scale=None,
               stream=None, o_lo=None) -> None:
    bsz, heads, _, d = q.shape
    if plan not in _plan_n:
        raise ValueError("lfattn_bwd: unknown plan handle")
    if lse is None:
        raise ValueError("lfattn_bwd: lse is required")
    shape = (bsz, heads, _plan_n[plan], d)
    _check_tensors("lfattn_bwd", shape, q.dtype,
                   (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq),
                    ("dk", dk), ("dv", dv)), lse, workspace,
                   lfattn_bwd_workspace(plan, bsz, heads, d), o_lo)
    scale = d ** -0.5 if scale is None else scale
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().lfattn_bwd(plan, bsz, heads, d, _dtype_code(q), c_float(scale), _ptr(q),
                             _ptr(k), _ptr(v), _ptr(o), _ptr(o_lo), _ptr(lse), _ptr(dout),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes,
                             _stream(stream)), "lfattn_bwd")


def lfattn_fwd_gproj(plan, q, k, v, qg, kg, vg, o, lse=None, workspace=None, scale=None,
                     stream=None, o_lo=None) -> None:
    """Forward with separate projections (qg, kg, vg) for the rows of global tokens."""
    bsz, heads, _, d = q.shape
    if plan not in _plan_n:
        raise ValueError("lfattn_fwd_gproj: unknown plan handle")
    shape = (bsz, heads, _plan_n[plan], d)
    _check_tensors("lfattn_fwd_gproj", shape, q.dtype,
                   (("q", q), ("k", k), ("v", v), ("qg", qg), ("kg", kg), ("vg", vg), ("o", o)),
                   lse, workspace, lfattn_fwd_workspace(plan, bsz, heads, d), o_lo)
    scale = d ** -0.5 if scale is None else scale
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().lfattn_fwd_gproj(plan, bsz, heads, d, _dtype_code(q), c_float(scale), _ptr(q),
                                   _ptr(k), _ptr(v), _ptr(qg), _ptr(kg), _ptr(vg), _ptr(o),
                                   _ptr(lse), _ptr(o_lo), _ptr(workspace), ws_bytes,
                                   _stream(stream)), "lfattn_fwd_gproj")


def lfattn_bwd_gproj(plan, q, k, v, qg, kg, vg, o, lse, dout, dq, dk, dv, dqg, dkg, dvg,
                     workspace=None, scale=None, stream=None, o_lo=None) -> None:
    """Backward of lfattn_fwd_gproj: gradients for both projection sets."""
    bsz, heads, _, d = q.shape
    if plan not in _plan_n:
        raise ValueError("lfattn_bwd_gproj: unknown plan handle")
    if lse is None:
        raise ValueError("lfattn_bwd_gproj: lse is required")
    shape = (bsz, heads, _plan_n[plan], d)
    _check_tensors("lfattn_bwd_gproj", shape, q.dtype,
                   (("q", q), ("k", k), ("v", v), ("qg", qg), ("kg", kg), ("vg", vg), ("o", o),
                    ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv), ("dqg", dqg),
                    ("dkg", dkg), ("dvg", dvg)),
                   lse, workspace, lfattn_bwd_workspace(plan, bsz, heads, d), o_lo)
    scale = d ** -0.5 if scale is None else scale
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().lfattn_bwd_gproj(plan, bsz, heads, d, _dtype_code(q), c_float(scale), _ptr(q),
                                   _ptr(k), _ptr(v), _ptr(qg), _ptr(kg), _ptr(vg), _ptr(o),
                                   _ptr(o_lo), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                   _ptr(dqg), _ptr(dkg), _ptr(dvg), _ptr(workspace), ws_bytes,
                                   _stream(stream)), "lfattn_bwd_gproj")


# --- diagnostics ----------------------------------------------------------------

def bsattn_status_str(status) -> str:
    return load().bsattn_status_str(status).decode()


def bsattn_last_error() -> str:
    return load().bsattn_last_error().decode()


def bsattn_version() -> str:
    return load().bsattn_version().decode()


def bsattn_profile_enable(on: bool) -> None:
    _check(load().bsattn_profile_enable(1 if on else 0), "bsattn_profile_enable")


def bsattn_profile_read(max_kernels: int = 64) -> dict:
    """{kernel name: (launches, total milliseconds)} since the last read (synchronous)."""
    import numpy as np
    names = ctypes.create_string_buffer(48 * max_kernels)
    counts = np.zeros(max_kernels, dtype=np.int64)
    ms = np.zeros(max_kernels, dtype=np.float64)
    n = c_int()
    _check(load().bsattn_profile_read(max_kernels, names, counts.ctypes.data, ms.ctypes.data,
                                      ctypes.byref(n)), "bsattn_profile_read")
    out = {}
    for i in range(n.value):
        nm = names.raw[48 * i:48 * i + 48].split(b"\0", 1)[0].decode()
        out[nm] = (int(counts[i]), float(ms[i]))
    return out
