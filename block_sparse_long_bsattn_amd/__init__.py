"""Block-sparse (BigBird-ITC) and banded (Longformer) attention for AMD MI355X.

The compute path is libbsattn.so (hand-written gfx950 HIP kernels behind the C
ABI in include/bsattn.h).  ``_lib`` is its ctypes binding with the same function
names; ``inputs`` draws the seeded synthetic tensors used by tests and benchmarks.
"""

from . import inputs  # noqa: F401
from ._lib import (  # noqa: F401
    BSATTN_BF16,
    BSATTN_F32,
    BsattnError,
    bsattn_bwd,
    bsattn_bwd_workspace,
    bsattn_fwd,
    bsattn_fwd_workspace,
    bsattn_last_error,
    bsattn_layout_build,
    bsattn_layout_destroy,
    bsattn_layout_info,
    bsattn_layout_rebuild,
    bsattn_layout_to_host,
    bsattn_status_str,
    bsattn_version,
    lfattn_bwd,
    lfattn_bwd_gproj,
    lfattn_bwd_workspace,
    lfattn_fwd,
    lfattn_fwd_gproj,
    lfattn_fwd_workspace,
    lfattn_plan_build,
    lfattn_plan_build_dilated,
    lfattn_plan_build_etc,
    lfattn_plan_destroy,
)
