"""fp64 CPU oracle for the video sparse attention forward (test infrastructure only)."""
from .vsa_oracle import (  # noqa: F401
    BLOCK,
    block_sizes,
    coarse,
    combine,
    pool,
    select_topk,
    sparse_block,
    tie_free,
    varlen_metadata,
    vsa_forward,
    vsa_forward_varlen,
    forward_packed_blocks,
)
from . import tiles  # noqa: F401
from . import vsa_backward  # noqa: F401
