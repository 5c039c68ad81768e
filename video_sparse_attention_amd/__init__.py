"""Video sparse attention (VSA) forward and backward for AMD Instinct MI355X (gfx950).

The computation lives in ``lib/libvsa.so`` (hand-written HIP kernels behind
the C ABI of ``include/vsa.h``); this package is its thin PyTorch binding.
Every entry point loads the library on first use and raises ``ImportError``
if it has not been built (there is no fallback path).
"""
from ._abi import VsaError, load as load_library  # noqa: F401

from .binding import (  # noqa: E402,F401
    BLOCK,
    VarlenMeta,
    alloc_workspace,
    block_shapes,
    dense_problem,
    token_shapes,
    DEFAULT_TILE,
    tile_block,
    tile_gather,
    tile_partition,
    tile_scatter,
    vsa_build_metadata,
    vsa_build_tile_metadata,
    vsa_forward_video,
    vsa_coarse_topk,
    vsa_combine,
    vsa_forward,
    vsa_forward_noalloc,
    vsa_noalloc_scratch_bytes,
    vsa_forward_varlen,
    vsa_sparse_attn_combine,
    vsa_sparse_attn_from_indices,
    vsa_workspace_size,
    alloc_backward_workspace,
    lse_shape,
    video_sparse_attn,
    video_sparse_attn_varlen,
    vsa_backward,
    vsa_backward_workspace_size,
    vsa_sparse_attn_combine_train,
)

__all__ = [
    "BLOCK", "VarlenMeta", "VsaError", "alloc_workspace", "block_shapes", "dense_problem",
    "token_shapes", "DEFAULT_TILE", "tile_block", "tile_gather", "tile_partition", "tile_scatter",
    "vsa_build_tile_metadata", "vsa_forward_video", "vsa_build_metadata", "vsa_coarse_topk", "vsa_combine", "vsa_forward",
    "vsa_forward_noalloc", "vsa_noalloc_scratch_bytes", "vsa_forward_varlen", "vsa_sparse_attn_combine", "vsa_sparse_attn_from_indices", "vsa_workspace_size",
    "alloc_backward_workspace", "lse_shape", "video_sparse_attn", "video_sparse_attn_varlen", "vsa_backward",
    "vsa_backward_workspace_size", "vsa_sparse_attn_combine_train",
]
