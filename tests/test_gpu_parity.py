"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle on
seeded inputs small enough for the oracle to finish in seconds, spanning
several blocks and ragged tails, plus the degenerate and edge cases."""
import numpy as np
import pytest
import torch

import oracle
import synth
import video_sparse_attention_amd as vsa
from tests import gpu_common as G
from tests import numerics as N

pytestmark = pytest.mark.gpu


def _full_check_dense(inp, gpu=None, tag=""):
    G.note(f"case {tag or inp.name}: shape={inp.shape} topk={inp.topk} gated={inp.gate is not None}")
    ref = G.oracle_dense(inp)
    G.assert_tie_free(ref)
    gpu = gpu or G.run_dense_stages(inp)
    G.assert_indices_equal(gpu["q2k_idx"], gpu["q2k_num"], ref)
    N.check_out_c(N.f64(gpu["out_c"]), ref["out_c"])
    rel = N.check_sparse(N.f64(gpu["out_s"]), ref["out_s"])
    mx, mean = N.check_out(N.f64(gpu["out"]), ref["out"])
    fmx, fmean = N.check_out(N.f64(gpu["out_fused"]), ref["out"], "out (fused combine)")
    N.check_fused(N.f64(gpu["out_fused"]), N.f64(gpu["out"]), N.f64(gpu["out_s"]))
    G.note(f"  out max-abs {mx:.2e} mean-abs {mean:.2e} (fused {fmx:.2e} / {fmean:.2e}); "
           f"sparse rel-rms {rel:.2e}")
    return gpu, ref


def test_tiny():
    _full_check_dense(synth.workload("tiny"))


def test_dense_equivalence():
    """top-k equal to every block: the sparse stage is dense attention."""
    inp = synth.workload("dense_equiv")
    gpu, ref = _full_check_dense(inp)
    nkv = inp.shape[3] // 64
    assert (gpu["q2k_idx"].numpy() == np.arange(nkv)).all()


@pytest.mark.parametrize("name", ["dense_equiv", "tiny", "gated"])
def test_forward_equals_stage_sequence(name):
    """vsa_forward launches exactly the stage kernels (coarse/top-k, then the
    sparse attention with the fused combine): identical bits."""
    if name == "gated":
        inp = synth.dense_inputs(2, 3, 64 * 5 + 17, 128, 2, seed=43, gated=True)
    else:
        inp = synth.workload(name)
    gpu = G.run_dense_stages(inp)
    q, k, v = (t.to(G.DEV) for t in (inp.q, inp.k, inp.v))
    g = None if inp.gate is None else inp.gate.to(G.DEV)
    out, oc, idx, num = vsa.vsa_forward(q, k, v, inp.topk, g, return_aux=True)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), gpu["out_fused"])
    assert torch.equal(oc.cpu(), gpu["out_c"])
    assert torch.equal(idx.cpu(), gpu["q2k_idx"])
    assert torch.equal(num.cpu(), gpu["q2k_num"])


def test_deterministic():
    inp = synth.workload("tiny")
    a = G.run_dense_stages(inp)
    b = G.run_dense_stages(inp)
    for key in ("out", "out_c", "q2k_idx"):
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("B,H,Sq,Skv,D,topk,gate", [
    (2, 3, 1000, 777, 64, 5, "token"),      # ragged tails, Sq != Skv, D=64
    (1, 2, 1, 1, 128, 1, "token"),          # single token
    (1, 2, 64, 64, 128, 3, None),           # single full block, topk clamped
    (1, 4, 130, 130, 128, 100, "full"),     # topk > nKV, full [B,H,S,D] gate
    (1, 2, 448, 640, 128, 4, "transposed"), # gate given as a transposed [B,S,H] view
    (3, 1, 200, 70, 64, 1, None),           # top-1, partial KV tail block
    (1, 1, 64 * 40 + 3, 64 * 40 + 3, 128, 8, "token"),  # many blocks + 3-token tail
    (1, 1, 128, 64 * 300, 128, 20, None),    # 300 KV blocks: 16 keys per lane in the top-k
    (1, 1, 200, 64 * 1100 - 5, 64, 7, None), # 1100 KV blocks: 64 keys per lane, 4 rows per group
    (1, 1, 64 * 3 + 17, 64 * 4095 + 5, 64, 300, "token"),  # the maximum, 4096 KV blocks, 5-token tail
    (1, 2, 64 * 70 + 9, 64 * 600 + 3, 128, 9, "token"),  # D = 128, 601 KV blocks: the 4-way output split,
                                                          # a 7-row last row tile and a 3-token KV tail
])
def test_dense_edge_cases(B, H, Sq, Skv, D, topk, gate):
    inp = synth.dense_inputs(B, H, Sq, D, topk, seed=2000 + Sq + Skv + D + topk,
                             gated=gate is not None, S_kv=Skv)
    if gate == "full":
        gen = torch.Generator().manual_seed(77)
        inp.gate = torch.sigmoid(torch.randn(B, H, Sq, D, generator=gen)).to(torch.bfloat16)
    G.note(f"case dense B={B} H={H} Sq={Sq} Skv={Skv} D={D} topk={topk} gate={gate}")
    ref = G.oracle_dense(inp)
    G.assert_tie_free(ref)
    q, k, v = (t.to(G.DEV) for t in (inp.q, inp.k, inp.v))
    g = None
    if inp.gate is not None:
        g = inp.gate.to(G.DEV)
        if gate == "transposed":
            g = g.permute(0, 2, 1).contiguous().permute(0, 2, 1)  # [B,S,H] storage
            assert not g.is_contiguous()
    out, oc, idx, num = vsa.vsa_forward(q, k, v, topk, g, return_aux=True)
    torch.cuda.synchronize()
    G.assert_indices_equal(idx.cpu(), num.cpu(), ref)
    N.check_out_c(N.f64(oc), ref["out_c"])
    N.check_out(N.f64(out), ref["out"])


@pytest.mark.parametrize("scale", [4.0, 16.0])
def test_sharp_softmax(scale):
    """Q and K scaled up so that every softmax is nearly one-hot and the
    running maximum jumps by far more than the lazy-rescale threshold from
    block to block (and the coarse scores spread over a wide range)."""
    inp = synth.dense_inputs(1, 2, 64 * 20 + 5, 128, 5, seed=2100 + int(scale), gated=True)
    inp.q = (inp.q.float() * scale).to(torch.bfloat16)
    inp.k = (inp.k.float() * scale).to(torch.bfloat16)
    G.note(f"case sharp softmax scale={scale}")
    ref = G.oracle_dense(inp)
    G.assert_tie_free(ref)
    q, k, v, g = (t.to(G.DEV) for t in (inp.q, inp.k, inp.v, inp.gate))
    out, oc, idx, num = vsa.vsa_forward(q, k, v, inp.topk, g, return_aux=True)
    torch.cuda.synchronize()
    G.assert_indices_equal(idx.cpu(), num.cpu(), ref)
    N.check_out_c(N.f64(oc), ref["out_c"])
    N.check_out(N.f64(out), ref["out"])
    assert torch.isfinite(out.float()).all()


def test_zero_inputs():
    """All-zero Q, K, V: every coarse score ties, so the routing is the first
    k blocks of every row (the lower-index rule); every softmax is uniform
    over zeros and the output is exactly zero."""
    B, H, S, D, topk = 1, 2, 64 * 9 + 20, 64, 4
    q = torch.zeros(B, H, S, D, dtype=torch.bfloat16)
    gen = torch.Generator().manual_seed(5)
    gate = torch.sigmoid(torch.randn(B, H, S, generator=gen)).to(torch.bfloat16)
    ref = oracle.vsa_forward(N.f64(q), N.f64(q), N.f64(q), topk, N.f64(gate))
    nq = -(-S // 64)
    assert np.array_equal(ref["q2k_idx"], np.broadcast_to(np.arange(topk), (B, H, nq, topk)))
    qd, gd = q.to(G.DEV), gate.to(G.DEV)
    out, oc, idx, num = vsa.vsa_forward(qd, qd, qd, topk, gd, return_aux=True)
    torch.cuda.synchronize()
    G.assert_indices_equal(idx.cpu(), num.cpu(), ref)
    assert torch.count_nonzero(oc).item() == 0
    assert torch.count_nonzero(out).item() == 0


def test_sparse_on_oracle_indices():
    """The sparse stage fed the oracle's routing reproduces the oracle's out_s."""
    for name in ("tiny", "dense_equiv"):
        inp = synth.workload(name)
        ref = G.oracle_dense(inp)
        gpu = G.run_dense_stages(inp, idx_override=(ref["q2k_idx"], ref["q2k_num"]))
        N.check_sparse(N.f64(gpu["out_s"]), ref["out_s"], f"{name} out_s")
    # a caller-made list: every other block, descending order, one invalid entry
    inp = synth.dense_inputs(1, 2, 64 * 9 - 20, 128, 4, seed=31)
    ref_full = G.oracle_dense(inp)
    nq = 9
    idx = np.full((1, 2, nq, 4), 0, dtype=np.int32)
    num = np.full((1, 2, nq), 4, dtype=np.int32)
    for i in range(nq):
        idx[0, :, i] = [8 - (i % 2), 6, 4, 99]  # 99 is out of range: skipped
    gpu = G.run_dense_stages(inp, idx_override=(idx, num))
    q, k, v = (N.f64(t)[0] for t in (inp.q, inp.k, inp.v))
    ks = oracle.block_sizes(inp.shape[3])
    for h in range(2):
        for i in range(nq):
            lo, n = 64 * i, oracle.block_sizes(inp.shape[2])[i]
            want = oracle.sparse_block(q[h, lo:lo + n], k[h], v[h], ks, idx[0, h, i, :3])
            N.check_sparse(N.f64(gpu["out_s"])[0, h, lo:lo + n], want, f"custom list h{h} i{i}")
    del ref_full


@pytest.mark.parametrize("gated", ["token", "full", None])
def test_combine_bit_exact(gated):
    """The combine is fp32 FMA (or add) with one RNE rounding to bf16, applied to
    the GPU's own sparse output and coarse output: bit-exact."""
    inp = synth.dense_inputs(2, 3, 64 * 5 + 17, 128, 2, seed=41, gated=gated is not None)
    if gated == "full":
        gen = torch.Generator().manual_seed(5)
        inp.gate = torch.sigmoid(torch.randn(2, 3, 64 * 5 + 17, 128, generator=gen)).to(torch.bfloat16)
    gpu = G.run_dense_stages(inp)
    os_bits = N.bf16_bits(gpu["out_s"])
    oc = gpu["out_c"].numpy()  # [B,H,nQ,D]
    S = inp.shape[2]
    blk = np.arange(S) // 64
    oc_tok = oc[:, :, blk, :]  # broadcast over tokens (test-side expansion)
    os32 = N.bits_to_f32(os_bits)
    if gated is None:
        want = N.add_bf16_bits(oc_tok, os32)
    else:
        g = N.bits_to_f32(N.bf16_bits(inp.gate))
        if g.ndim == 3:
            g = np.broadcast_to(g[..., None], os32.shape)
        want = N.fma_bf16_bits(oc_tok, g, os32)
    got = N.bf16_bits(gpu["out"])
    assert np.array_equal(got, want), f"{int((got != want).sum())} elements differ"


def test_varlen_small():
    inp = synth.workload("varlen_small")
    G.note(f"case varlen_small: lens={inp.seqlens_q} topk={inp.topk}")
    ref = G.oracle_varlen(inp)
    G.assert_tie_free(ref)
    gpu = G.run_varlen_stages(inp)
    G.assert_indices_equal(gpu["q2k_idx"], gpu["q2k_num"], ref)
    N.check_out_c(N.f64(gpu["out_c"]), ref["out_c"])
    N.check_sparse(N.f64(gpu["out_s"]), ref["out_s"])
    N.check_out(N.f64(gpu["out"]), ref["out"])
    N.check_out(N.f64(gpu["out_fused"]), ref["out"], "out (fused combine)")
    N.check_fused(N.f64(gpu["out_fused"]), N.f64(gpu["out"]), N.f64(gpu["out_s"]))
    # padding slots hold 0
    for key in ("out", "out_fused"):
        out = gpu[key].float().numpy()
        o = 0
        for sq in inp.seqlens_q:
            nb = -(-sq // 64)
            assert (out[:, o + sq:o + 64 * nb] == 0).all(), key
            o += 64 * nb


@pytest.mark.parametrize("gated", [False, True])
def test_varlen_packed_equals_per_sequence(gated):
    """One packed launch gives bit-identical results to one dense launch per
    sequence (and indices equal to the per-sequence ones rebased)."""
    lens_q = [5 * 64, 9 * 64, 13 * 64 + 40, 64, 1, 130]
    lens_kv = [6 * 64, 9 * 64, 14 * 64 - 7, 64, 130, 1]
    topk = [2, 3, 4, 1, 5, 2]
    inp = synth.varlen_inputs(lens_q, lens_kv, 4, 128, topk, seed=77, gated=gated)
    packed = G.run_varlen_stages(inp)
    oq = bq = bkv = 0
    for s, seq in enumerate(inp.per_seq):
        d = synth.DenseInputs(seq["q"][None], seq["k"][None], seq["v"][None],
                              None if seq["gate"] is None else seq["gate"][None], topk[s])
        one = G.run_dense_stages(d)
        nq, nkv = -(-lens_q[s] // 64), -(-lens_kv[s] // 64)
        kk = min(topk[s], nkv)
        assert torch.equal(packed["out"][:, oq:oq + lens_q[s]], one["out"][0]), s
        assert torch.equal(packed["out_fused"][:, oq:oq + lens_q[s]], one["out_fused"][0]), s
        assert torch.equal(packed["out_c"][:, bq:bq + nq], one["out_c"][0]), s
        pi = packed["q2k_idx"][:, bq:bq + nq]
        assert torch.equal(pi[..., :kk], one["q2k_idx"][0] + bkv), s
        assert (pi[..., kk:] == -1).all()
        oq += 64 * nq
        bq += nq
        bkv += nkv


def test_single_sequence_varlen_equals_dense():
    inp = synth.dense_inputs(1, 3, 64 * 7 - 9, 128, 3, seed=88, gated=True)
    dense = G.run_dense_stages(inp)
    S = inp.shape[2]
    nb = -(-S // 64)
    pad = lambda t, D: torch.cat([t, torch.zeros(*t.shape[:1], 64 * nb - S, *D, dtype=t.dtype)], 1)
    vin = synth.VarlenInputs(pad(inp.q[0], (128,)), pad(inp.k[0], (128,)), pad(inp.v[0], (128,)),
                             pad(inp.gate[0], ()), [S], [S], [3])
    var = G.run_varlen_stages(vin)
    assert torch.equal(var["out"][:, :S], dense["out"][0])
    assert torch.equal(var["out_fused"][:, :S], dense["out_fused"][0])
    assert torch.equal(var["q2k_idx"], dense["q2k_idx"][0])


def test_binding_rejects_bad_tensors():
    q = torch.zeros(1, 2, 128, 64, dtype=torch.bfloat16, device=G.DEV)
    with pytest.raises(TypeError):
        vsa.vsa_forward(q.float(), q, q, 1)
    with pytest.raises(ValueError):
        vsa.vsa_forward(q, q[:, :1], q, 1)
    with pytest.raises(ValueError):
        vsa.vsa_forward(q, q, q, 1, gate=torch.zeros(1, 2, 127, dtype=torch.bfloat16, device=G.DEV))
    with pytest.raises(RuntimeError):
        vsa.vsa_forward(q.clone().requires_grad_(True), q, q, 1)
    with pytest.raises(vsa.VsaError):
        vsa.vsa_forward(q, q.clone(), q.clone(), 0)
