"""GPU parity of the 3-D tile path: gather / scatter bit-exact against the
oracle's index arithmetic, and the tiled video forward against the oracle's
tiled forward ("[kernel] Extract VSA utility functions into fastvideo_kernel",
Summary)."""
import numpy as np
import pytest
import torch

import oracle.tiles as TL
import synth
import video_sparse_attention_amd as vsa
from tests import gpu_common as G
from tests import numerics as N

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.cpu().view(torch.int16).numpy()


@pytest.mark.parametrize("grid,tile,E", [
    ((5, 6, 7), (4, 4, 4), 128), ((3, 9, 2), (4, 4, 4), 64), ((6, 10, 5), (2, 4, 8), 16),
    ((5, 6, 7), (4, 4, 4), 1), ((4, 5, 3), (4, 4, 4), 3), ((1, 1, 130), (1, 1, 64), 8),
    # tiles of 128 / 256 tokens in blocks of 128 / 256 slots
    ((9, 10, 11), (4, 4, 8), 128), ((5, 9, 17), (4, 8, 8), 64), ((3, 7, 7), (3, 5, 7), 1),
    ((1, 1, 300), (1, 1, 256), 8),
])
def test_tile_gather_scatter_bit_exact(grid, tile, E):
    G.note(f"case tile copy grid={grid} tile={tile} E={E}")
    B, Hh = 2, 3
    S = grid[0] * grid[1] * grid[2]
    gen = torch.Generator().manual_seed(sum(grid) + E)
    shape = (B, Hh, S) if E == 1 else (B, Hh, S, E)
    x = torch.randn(shape, generator=gen).to(torch.bfloat16)
    y = vsa.tile_gather(x.to(G.DEV), grid, tile)
    xb = _bits(x)
    want = TL.tile_gather(xb[..., None] if E == 1 else xb, grid, tile)  # [B, Hh, slots(, E)]
    want = np.concatenate([want[b] for b in range(B)], axis=1)        # [Hh, B*slots(, E)]
    if E == 1:
        want = want[..., 0]
    assert np.array_equal(_bits(y), want)
    back = vsa.tile_scatter(y, grid, B, tile)
    assert np.array_equal(_bits(back), xb)


def _video_inputs(B, Hh, grid, D, seed, gated=True):
    S = grid[0] * grid[1] * grid[2]
    inp = synth.dense_inputs(B, Hh, S, D, 1, seed=seed, gated=gated)
    return inp.q, inp.k, inp.v, inp.gate


@pytest.mark.parametrize("grid,tile,D,topk", [
    ((5, 6, 7), (4, 4, 4), 64, 3),        # partial tiles along every axis
    ((8, 8, 12), (4, 4, 4), 128, 4),      # full tiles only
    ((6, 10, 5), (2, 4, 8), 128, 5),      # a non-cubic tile
    ((9, 10, 11), (4, 4, 8), 128, 3),     # 128-token tiles, partial along every axis
    ((8, 16, 20), (4, 8, 8), 64, 4),      # 256-token tiles, partial along w
    ((5, 9, 17), (4, 8, 8), 128, 2),      # 256-token tiles, partial along every axis
])
def test_video_forward_matches_oracle(grid, tile, D, topk):
    B, Hh = 2, 3
    G.note(f"case video forward grid={grid} tile={tile} D={D} topk={topk}")
    q, k, v, gate = _video_inputs(B, Hh, grid, D, seed=5000 + sum(grid) + D)
    ref = TL.vsa_forward_video(N.f64(q), N.f64(k), N.f64(v), grid, topk, N.f64(gate), tile=tile)
    G.assert_tie_free(ref)
    out, oc, idx, num = vsa.vsa_forward_video(q.to(G.DEV), k.to(G.DEV), v.to(G.DEV), grid, topk,
                                              gate.to(G.DEV), tile, return_aux=True)
    torch.cuda.synchronize()
    G.assert_indices_equal(idx.cpu(), num.cpu(), ref)
    N.check_out_c(N.f64(oc), ref["out_c"])
    mx, mean = N.check_out(N.f64(out), ref["out_raster"])
    G.note(f"  out max-abs {mx:.2e} mean-abs {mean:.2e}")


@pytest.mark.parametrize("bs", [64, 128, 256])
def test_video_1d_equals_dense(bs):
    """A 1 x 1 x S grid in 1 x 1 x bs tiles is the dense forward with VSA
    blocks of bs tokens, bit for bit."""
    S, D = bs * 6 + 19, 128
    q, k, v, gate = _video_inputs(2, 3, (1, 1, S), D, seed=77 + bs)
    dev = [t.to(G.DEV) for t in (q, k, v, gate)]
    a = vsa.vsa_forward_video(*dev[:3], (1, 1, S), 4, dev[3], (1, 1, bs))
    b = vsa.vsa_forward(*dev[:3], 4, dev[3], block_size=bs)
    torch.cuda.synchronize()
    assert torch.equal(a.cpu(), b.cpu())


def test_video_forward_latent_sized():
    """A small video latent (16 x 30 x 52 tokens: 4 x 8 x 13 tiles, partial
    along h), 4 heads, D=128, top-20%: every index and coarse row, sampled
    output tiles."""
    grid, tile, B, Hh, D = (16, 30, 52), (4, 4, 4), 1, 4, 128
    nt = 4 * 8 * 13
    topk = -(-nt // 5)
    q, k, v, gate = _video_inputs(B, Hh, grid, D, seed=6000)
    rng = np.random.default_rng(8)
    blocks = [(int(h), int(g)) for h, g in zip(rng.integers(0, Hh, 24), rng.integers(0, nt, 24))]
    blocks += [(0, nt - 1), (Hh - 1, 7)]
    G.note(f"case latent grid={grid} tiles={nt} topk={topk}, {len(blocks)} sampled tiles")
    ref = TL.vsa_forward_video(N.f64(q), N.f64(k), N.f64(v), grid, topk, N.f64(gate), tile=tile, blocks=blocks)
    G.assert_tie_free(ref)
    out, oc, idx, num = vsa.vsa_forward_video(q.to(G.DEV), k.to(G.DEV), v.to(G.DEV), grid, topk,
                                              gate.to(G.DEV), tile, return_aux=True)
    torch.cuda.synchronize()
    G.assert_indices_equal(idx.cpu(), num.cpu(), ref)
    N.check_out_c(N.f64(oc), ref["out_c"])
    N.check_out(N.f64(out), ref["out_raster"])
