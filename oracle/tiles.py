"""Plain CPU oracle of the 3-D tile partition that feeds video latents to VSA.

TEST INFRASTRUCTURE ONLY, like ``vsa_oracle``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` may use it.

Source: "[kernel] Extract VSA utility functions into fastvideo_kernel"
(Summary, Changes, Design decisions and the review thread): the tile
partition of a video's token grid, its inverse, the per-tile valid-token
counts (``variable_block_sizes``, the tile size a parameter) and the
positions of the valid tokens in the padded layout (``non_pad_index``).  The
pages name these functions and their outputs but print no definition, so the
plainest reading is taken (listed with the other readings in the design
notes):

* the latent is a ``T x H x W`` grid of tokens flattened in raster order
  (``w`` fastest, then ``h``, then ``t``);
* it is cut into tiles of ``tt x th x tw`` tokens (``tt * th * tw <= 256``;
  64 = 4 x 4 x 4 is the default), the last tile along an axis being shorter
  when the extent is not a multiple of the tile;
* tiles are ordered in raster order of their tile coordinates, and the
  tokens inside a tile in raster order of their coordinates in the tile;
* ``tile_partition_indices[p]`` is the raster index of the token at position
  ``p`` of that tiled order, ``reverse_tile_partition_indices`` is its inverse
  permutation, ``variable_block_sizes[b]`` the number of tokens of tile ``b``
  and ``non_pad_index[p]`` the slot of position ``p`` when every tile is
  padded to its VSA block of ``bs`` slots (slot ``bs b + u`` for the ``u``-th
  token of tile ``b``).  ``bs`` is 64 for tiles of at most 64 tokens and 128
  or 256 for the larger tiles of the 128/256-token variants ("[chore] release
  fastvideo-kernel 0.3.0", Block-sparse / VSA attention improvements): the
  smallest of 64, 128, 256 that holds the tile (reading: the tile is the VSA
  block, e.g. 4 x 8 x 8 = 256 tokens in a 256-slot block).

Each function below spells that out with explicit loops.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence, Tuple

import numpy as np

from .vsa_oracle import BLOCK, forward_packed_blocks

DEFAULT_TILE = (4, 4, 4)


def tile_block(tile: Tuple[int, int, int]) -> int:
    """Slots of the VSA block that holds one tile: the smallest of 64, 128
    and 256 that is at least the tile's token count."""
    n = tile[0] * tile[1] * tile[2]
    for bs in (BLOCK, 2 * BLOCK, 4 * BLOCK):
        if n <= bs:
            return bs
    raise ValueError("a tile holds at most 256 tokens")


def tile_partition(T: int, H: int, W: int, tile: Tuple[int, int, int] = DEFAULT_TILE) -> Dict[str, np.ndarray]:
    """Tile order, its inverse, tile sizes and padded positions (loops over
    tiles, then over the tokens of each tile)."""
    tt, th, tw = tile
    if min(T, H, W) < 1 or min(tt, th, tw) < 1 or tt * th * tw > 4 * BLOCK:
        raise ValueError("grid and tile extents must be >= 1 and a tile at most 256 tokens")
    bs = tile_block(tile)
    n_t, n_h, n_w = -(-T // tt), -(-H // th), -(-W // tw)
    fwd, nonpad, sizes = [], [], []
    for bt in range(n_t):
        for bh in range(n_h):
            for bw in range(n_w):
                et = min(tt, T - bt * tt)
                eh = min(th, H - bh * th)
                ew = min(tw, W - bw * tw)
                b = len(sizes)
                u = 0
                for lt in range(et):
                    for lh in range(eh):
                        for lw in range(ew):
                            fwd.append(((bt * tt + lt) * H + (bh * th + lh)) * W + (bw * tw + lw))
                            nonpad.append(bs * b + u)
                            u += 1
                sizes.append(u)
    rev = [0] * len(fwd)
    for p, r in enumerate(fwd):
        rev[r] = p
    return dict(tile_partition_indices=np.asarray(fwd, dtype=np.int64),
                reverse_tile_partition_indices=np.asarray(rev, dtype=np.int64),
                variable_block_sizes=np.asarray(sizes, dtype=np.int64),
                non_pad_index=np.asarray(nonpad, dtype=np.int64))


def tile_gather(x: np.ndarray, grid: Tuple[int, int, int], tile=DEFAULT_TILE) -> np.ndarray:
    """``x`` ``[..., T*H*W, D]`` in raster order -> ``[..., bs * n_tiles, D]``
    in tile order, each tile padded to its ``bs = tile_block(tile)`` slots with
    zeros."""
    meta = tile_partition(*grid, tile)
    fwd, nonpad = meta["tile_partition_indices"], meta["non_pad_index"]
    n_tiles = len(meta["variable_block_sizes"])
    y = np.zeros(x.shape[:-2] + (tile_block(tile) * n_tiles, x.shape[-1]), dtype=x.dtype)
    for p in range(len(fwd)):
        y[..., nonpad[p], :] = x[..., fwd[p], :]
    return y


def tile_scatter(y: np.ndarray, grid: Tuple[int, int, int], tile=DEFAULT_TILE) -> np.ndarray:
    """Inverse of ``tile_gather`` (padding slots are dropped)."""
    meta = tile_partition(*grid, tile)
    fwd, nonpad = meta["tile_partition_indices"], meta["non_pad_index"]
    x = np.zeros(y.shape[:-2] + (len(fwd), y.shape[-1]), dtype=y.dtype)
    for p in range(len(fwd)):
        x[..., fwd[p], :] = y[..., nonpad[p], :]
    return x


def vsa_forward_video(q, k, v, grid: Tuple[int, int, int], topk: int, gate=None, tile=DEFAULT_TILE,
                      blocks: Optional[Sequence[Tuple[int, int]]] = None) -> Dict[str, np.ndarray]:
    """VSA forward of ``B`` videos of one ``T x H x W`` grid, inputs and
    outputs in raster order ``[B, H_heads, T*H*W, D]``: every video is
    gathered into its padded tile order, the blocks of the forward are the
    tiles (with their valid-token counts), the videos are packed one after
    another, and the output is scattered back.  ``gate`` is ``None``,
    ``[B, H_heads, S]`` or ``[B, H_heads, S, D]``.  ``blocks`` as in
    ``forward_packed_blocks`` (global tile numbers, video ``b`` owning tiles
    ``[b n_tiles, (b + 1) n_tiles)``).  Returns the packed results plus
    ``out_raster``."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    B, Hh, S, D = q.shape
    meta = tile_partition(*grid, tile)
    sizes = [int(x) for x in meta["variable_block_sizes"]]
    n_tiles = len(sizes)

    bs = tile_block(tile)

    def pack(x):  # [B, Hh, S, ...] raster -> [Hh, B * bs * n_tiles, ...]
        if x.ndim == 3:
            g = tile_gather(x[..., None], grid, tile)[..., 0]
        else:
            g = tile_gather(x, grid, tile)
        return np.concatenate([g[b] for b in range(B)], axis=1)

    gq, gk, gv = pack(q), pack(k), pack(v)
    gg = None if gate is None else pack(np.asarray(gate, dtype=np.float64))
    res = forward_packed_blocks(gq, gk, gv, [sizes] * B, [sizes] * B, [topk] * B, gg, blocks, bs)
    slots = bs * n_tiles
    out = res["out"]
    out_raster = np.stack([tile_scatter(out[:, b * slots:(b + 1) * slots], grid, tile) for b in range(B)])
    res["out_raster"] = out_raster
    res["variable_block_sizes"] = np.asarray(sizes)
    return res
