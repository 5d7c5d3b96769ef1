"""Plain fp64 CPU oracle for block-sparse (BigBird-ITC) and banded (Longformer) attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this package; only the
tests, the smoke check and the CPU-baseline leg of the benchmark call it.  It shares
no code with the HIP path: it has its own layout builder, its own masks and its own
softmax, written from the pages' definitions, not from the kernels.

Modules
-------
layout      block layout: window / global / seeded random key blocks per query block
attention   masked softmax attention forward and backward on a materialised mask
longformer  token-level sliding window (dilated, causal) + symmetric global mask
etc         BigBird-ETC: added global tokens + blocked window, any sequence length

Parity status: every public function is pinned by tests under ``tests/``
(``test_oracle_*.py``) against closed forms, library routines, published
generator vectors or brute force.  No function here is "parity unpinned".
"""

from .layout import (  # noqa: F401
    splitmix64,
    window_blocks,
    random_blocks,
    row_blocks,
    build_layout,
    block_mask,
    token_mask,
)
from .attention import (  # noqa: F401
    attention_probs,
    attention_fwd,
    attention_bwd,
    attention_fwd_rows,
)
from .longformer import (  # noqa: F401
    longformer_mask, longformer_allowed, in_window, longformer_gproj_fwd, longformer_gproj_bwd)
from .etc import etc_mask, etc_allowed  # noqa: F401
