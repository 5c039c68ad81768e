"""GPU parity of the 128- and 256-token VSA blocks and of the [B, S, H, D]
(BSHD) entry against the fp64 oracle (which takes the block size as a
parameter and works on [B, H, S, D]; BSHD inputs are the same tensors
transposed), on seeded inputs with ragged tails, plus the full-size large
shape at both block sizes on sampled query blocks, and packed sequences with
VSA blocks of 128 / 256 slots."""
import numpy as np
import pytest
import torch

import synth
import video_sparse_attention_amd as vsa
from tests import gpu_common as G
from tests import numerics as N

pytestmark = pytest.mark.gpu


def _inputs(B, H, Sq, Skv, D, topk, gate, seed):
    inp = synth.dense_inputs(B, H, Sq, D, topk, seed=seed, gated=gate == "token", S_kv=Skv)
    if gate == "full":
        inp.gate = synth.full_gate((B, H, Sq, D), seed + 1)
    return inp


def _check_all(inp, gpu, ref):
    G.assert_tie_free(ref)
    G.assert_indices_equal(gpu["q2k_idx"], gpu["q2k_num"], ref)
    N.check_out_c(N.f64(gpu["out_c"]), ref["out_c"])
    rel = N.check_sparse(N.f64(gpu["out_s"]), ref["out_s"])
    mx, mean = N.check_out(N.f64(gpu["out"]), ref["out"])
    N.check_out(N.f64(gpu["out_fused"]), ref["out"], "out (fused combine)")
    N.check_fused(N.f64(gpu["out_fused"]), N.f64(gpu["out"]), N.f64(gpu["out_s"]))
    G.note(f"  out max-abs {mx:.2e} mean-abs {mean:.2e}; sparse rel-rms {rel:.2e}")


@pytest.mark.parametrize("block,B,H,Sq,Skv,D,topk,gate", [
    (128, 1, 2, 128 * 5 + 37, 128 * 5 + 37, 128, 2, "token"),  # ragged 37-token tail (one 64-sub-block)
    (128, 2, 2, 700, 900, 64, 3, None),                        # Sq != Skv, tails of 60 and 4 tokens
    (128, 1, 1, 128 * 6 + 64, 128 * 6 + 64, 128, 3, "full"),   # last VSA block = one full 64-sub-block
    (256, 1, 3, 256 * 4 + 100, 256 * 4 + 100, 128, 2, "full"), # 100-token tail: sub-blocks 64 + 36
    (256, 1, 1, 256 * 3, 256 * 6 - 7, 64, 100, "token"),       # top-k above the VSA block count
    (256, 2, 1, 256 * 5 + 200, 256 * 5 + 200, 64, 1, None),    # top-1, 200-token tail (4 sub-blocks, last 8)
    (128, 1, 2, 1, 1, 128, 1, None),                           # single token
    (256, 1, 1, 256 + 30, 256 * 4095 + 100, 64, 40, "token"),  # the maximum: 4096 VSA blocks of 256
])
def test_large_vsa_blocks(block, B, H, Sq, Skv, D, topk, gate):
    inp = _inputs(B, H, Sq, Skv, D, topk, gate, seed=3000 + block + Sq + Skv + D)
    G.note(f"case block={block} B={B} H={H} Sq={Sq} Skv={Skv} D={D} topk={topk} gate={gate}")
    ref = G.oracle_dense(inp, block=block)
    gpu = G.run_dense_stages(inp, block_size=block)
    _check_all(inp, gpu, ref)
    # the one-call forward launches the same kernels: identical bits
    q, k, v = (t.to(G.DEV) for t in (inp.q, inp.k, inp.v))
    g = None if inp.gate is None else inp.gate.to(G.DEV)
    out, oc, idx, num = vsa.vsa_forward(q, k, v, topk, g, block_size=block, return_aux=True)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), gpu["out_fused"])
    assert torch.equal(oc.cpu(), gpu["out_c"])
    assert torch.equal(idx.cpu(), gpu["q2k_idx"])
    assert torch.equal(num.cpu(), gpu["q2k_num"])


@pytest.mark.parametrize("block", [64, 128, 256])
@pytest.mark.parametrize("gate", ["token", "full", None])
def test_bshd_matches_dense_bits(block, gate):
    """BSHD tensors are the dense ones with strided rows: the same kernels in
    the same order give the same bits, and both match the oracle."""
    B, H, Sq, Skv, D = 2, 3, 64 * 9 + 17, 64 * 11 + 50, 128
    inp = _inputs(B, H, Sq, Skv, D, 3, gate, seed=4000 + block)
    G.note(f"case bshd block={block} gate={gate} B={B} H={H} Sq={Sq} Skv={Skv}")
    ref = G.oracle_dense(inp, block=block)
    dense = G.run_dense_stages(inp, block_size=block)
    bshd = G.run_dense_stages(inp, block_size=block, bshd=True)
    _check_all(inp, bshd, ref)
    for key in ("out", "out_s", "out_c", "q2k_idx", "q2k_num", "out_fused"):
        assert torch.equal(bshd[key], dense[key]), key


@pytest.mark.parametrize("D", [64, 128])
def test_bshd_forward_entry(D):
    """vsa_forward_bshd (one call) on [B, S, H, D], with the gate given as a
    [B, S, H] tensor and as a transposed view of a [B, H, S] one."""
    B, H, Sq, Skv = 1, 4, 64 * 7 + 9, 64 * 7 + 9
    inp = _inputs(B, H, Sq, Skv, D, 2, "token", seed=4100 + D)
    G.note(f"case bshd forward D={D}")
    ref = G.oracle_dense(inp)
    G.assert_tie_free(ref)
    q, k, v = (G.to_bshd(t).to(G.DEV) for t in (inp.q, inp.k, inp.v))
    g_bsh = G.to_bshd(inp.gate).to(G.DEV)
    g_view = inp.gate.to(G.DEV).transpose(1, 2)  # [B, S, H] view of [B, H, S] storage
    assert not g_view.is_contiguous()
    outs = []
    for g in (g_bsh, g_view):
        out, oc, idx, num = vsa.vsa_forward(q, k, v, 2, g, bshd=True, return_aux=True)
        torch.cuda.synchronize()
        G.assert_indices_equal(idx.cpu(), num.cpu(), ref)
        N.check_out_c(N.f64(oc), ref["out_c"])
        N.check_out(N.f64(G.from_bshd(out.cpu())), ref["out"])
        outs.append(out.cpu())
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("block,topk", [(128, 25), (256, 13)])
def test_large_shape_large_blocks(block, topk):
    """The large video-DiT shape (B=1, H=56, S=15488, D=128, gated) with VSA
    blocks of 128 (121 blocks) and 256 tokens (61 blocks, the last 128 tokens),
    top-k about 20 % of the blocks: every index and coarse row, sampled token
    outputs."""
    inp = synth.dense_inputs(1, 56, 15488, 128, topk, seed=5000 + block, gated=True)
    B, H, Sq, Skv, D = inp.shape
    nq = -(-Sq // block)
    rng = np.random.default_rng(block)
    picks = rng.choice(H * nq, 24, replace=False)
    blocks = [(0, int(p) // nq, int(p) % nq) for p in picks] + [(0, H - 1, nq - 1), (0, 0, 0)]
    G.note(f"case large block={block} topk={topk}, {len(blocks)} sampled VSA blocks")
    gpu = G.run_dense_stages(inp, block_size=block)
    ref = G.oracle_dense(inp, blocks=blocks, block=block)
    _check_all(inp, gpu, ref)


# ---------------------------------------------------------------------------
# packed sequences with VSA blocks of 128 / 256 slots
# ---------------------------------------------------------------------------

# lengths giving VSA blocks whose trailing 64-token blocks are empty (at 256:
# 37 tokens = 37 + 0 + 0 + 0, 300 = 256 + (44 + 0 + 0 + 0), 129 = 64 + 64 + 1 + 0)
_LENS_Q = [3 * 256 + 37, 300, 1, 129, 2 * 256]
_LENS_KV = [2 * 256 + 9, 300, 70, 256 * 3 - 5, 129]
_TOPK = [2, 1, 3, 2, 5]


@pytest.mark.parametrize("block", [128, 256])
@pytest.mark.parametrize("gate", ["token", "full", None])
def test_varlen_large_blocks(block, gate):
    inp = synth.varlen_inputs(_LENS_Q, _LENS_KV, 3, 128, _TOPK, seed=6000 + block, gated=gate == "token",
                              block=block)
    if gate == "full":
        inp.gate = synth.full_gate(tuple(inp.q.shape), 6001 + block)
    G.note(f"case varlen block={block} gate={gate} lens_q={_LENS_Q} lens_kv={_LENS_KV}")
    ref = G.oracle_varlen(inp)
    gpu = G.run_varlen_stages(inp)
    _check_all(inp, gpu, ref)
    # padding slots (including whole empty 64-token blocks) hold 0
    o = 0
    for sq in inp.seqlens_q:
        nb = -(-sq // block)
        for key in ("out", "out_s", "out_fused"):
            assert (gpu[key][:, o + sq:o + block * nb] == 0).all(), key
        o += block * nb
    # the one-call packed forward launches the same kernels: identical bits
    dev = G.DEV
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    g = None if inp.gate is None else inp.gate.to(dev)
    out, oc, idx, num = vsa.vsa_forward_varlen(q, k, v, gpu["meta"], g, return_aux=True)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), gpu["out_fused"])
    assert torch.equal(oc.cpu(), gpu["out_c"])
    assert torch.equal(idx.cpu(), gpu["q2k_idx"])
    assert torch.equal(num.cpu(), gpu["q2k_num"])


@pytest.mark.parametrize("block", [128, 256])
def test_varlen_large_blocks_equals_per_sequence(block):
    """One packed launch with 128- / 256-slot blocks gives the bits of one
    dense launch per sequence with the same VSA block size (indices rebased)."""
    D = 64
    inp = synth.varlen_inputs(_LENS_Q, _LENS_KV, 2, D, _TOPK, seed=6100 + block, gated=True, block=block)
    G.note(f"case varlen = per sequence, block={block}")
    packed = G.run_varlen_stages(inp)
    oq = bq = bkv = 0
    for s, seq in enumerate(inp.per_seq):
        d = synth.DenseInputs(seq["q"][None], seq["k"][None], seq["v"][None], seq["gate"][None], _TOPK[s])
        one = G.run_dense_stages(d, block_size=block)
        nq, nkv = -(-_LENS_Q[s] // block), -(-_LENS_KV[s] // block)
        kk = min(_TOPK[s], nkv)
        sl = slice(oq, oq + _LENS_Q[s])
        for key in ("out", "out_s", "out_fused"):
            assert torch.equal(packed[key][:, sl], one[key][0]), (s, key)
        assert torch.equal(packed["out_c"][:, bq:bq + nq], one["out_c"][0]), s
        pi = packed["q2k_idx"][:, bq:bq + nq]
        assert torch.equal(pi[..., :kk], one["q2k_idx"][0] + bkv), s
        assert (pi[..., kk:] == -1).all()
        oq += block * nq
        bq += nq
        bkv += nkv


def test_varlen_large_blocks_caller_lists():
    """The packed sparse stage (VSA blocks of 256 slots) on caller-made lists in
    any order: entries of another sequence, negative and out-of-range entries
    are skipped; the rest is attention over the listed blocks' valid tokens
    (their trailing empty 64-token blocks included in the skip)."""
    import oracle
    bs, H, D = 256, 2, 128
    lq, lkv = [300, 200], [600, 130]  # Q VSA blocks 2 + 1, KV VSA blocks 3 + 1 (global 0..2, 3)
    inp = synth.varlen_inputs(lq, lkv, H, D, [3, 3], seed=6200, gated=False, block=bs)
    rows = [[2, 3, 0], [-5, 1, 99], [3, 0, 50]]    # per global query block
    valid = [[2, 0], [1], [0]]                       # local KV blocks that count
    idx = np.array([rows] * H, dtype=np.int32)      # [H, Nq, max_topk = 3]
    num = np.full((H, 3), 3, dtype=np.int32)
    G.note("case packed caller lists, 256-slot blocks")
    gpu = G.run_varlen_stages(inp, idx_override=(idx, num))
    out_s = N.f64(gpu["out_s"])
    owner = [(0, 0), (0, 1), (1, 0)]  # (sequence, local query block) of each global query block
    q_off = [0, bs * 2]
    for h in range(H):
        for g, (s, i) in enumerate(owner):
            per = inp.per_seq[s]
            q, k, v = (N.f64(per[x])[h] for x in ("q", "k", "v"))
            n = oracle.block_sizes(lq[s], bs)[i]
            want = oracle.sparse_block(q[bs * i:bs * i + n], k, v, oracle.block_sizes(lkv[s], bs), valid[g], bs)
            lo = q_off[s] + bs * i
            N.check_sparse(out_s[h, lo:lo + n], want, f"caller list h{h} block {g}")
            assert (out_s[h, lo + n:lo + bs] == 0).all()
