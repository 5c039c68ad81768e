"""GPU parity of the backward pass (vsa_sparse_attn_combine_train + vsa_backward,
through the C ABI) against the fp64 oracle of ``oracle/vsa_backward.py`` on
seeded inputs that span several blocks with ragged tails, every gate mode,
Sq != Skv, single-block and single-token sequences, and packed sequences.

Tolerances (gradients are compared relative to the reference's own scale,
since their magnitude follows dout and the softmax sharpness): the sparse
part rounds P and dS to bf16 as MFMA operands (relative 2^-9 each) and every
output once to bf16 (2^-9); the errors of the sums over 64 * top-k tokens
are unbiased, so the worst element stays within a few times 2^-9 of the
largest gradient and the mean within a fraction of that of the mean one."""
import numpy as np
import pytest
import torch

import oracle
import synth
import video_sparse_attention_amd as vsa
from oracle import vsa_backward as BW
from tests import gpu_common as G
from tests import numerics as N

pytestmark = pytest.mark.gpu

GRAD_MAX_REL = 1e-2   # max |gpu - ref| / max |ref| (measured 2-5e-3)
GRAD_MEAN_REL = 5e-3  # mean |gpu - ref| / mean |ref| (measured 1-2.4e-3)
LSE_ABS = 4e-3        # log2 units: the bf16 rounding of the summed probabilities
GRAD_FLOOR_MAX = 1e-2
GRAD_FLOOR_MEAN = 1e-3


def check_grad(gpu: np.ndarray, ref: np.ndarray, what: str, max_rel=None, mean_rel=None):
    assert np.isfinite(gpu).all(), f"{what}: non-finite values"
    d = np.abs(gpu - ref)
    # a gradient that vanishes in exact arithmetic (one key per row: P = 1,
    # dS = 0) keeps rounding residue; with unit-variance inputs and dout the
    # scales are floored at GRAD_FLOOR_MAX / GRAD_FLOOR_MEAN
    scale_max = max(float(np.abs(ref).max()), GRAD_FLOOR_MAX)
    scale_mean = max(float(np.abs(ref).mean()), GRAD_FLOOR_MEAN)
    mx, mean = float(d.max()) / scale_max, float(d.mean()) / scale_mean
    G.note(f"  {what}: max-err/max {mx:.2e}, mean-err/mean {mean:.2e} (|ref| max {scale_max:.2e})")
    max_rel = GRAD_MAX_REL if max_rel is None else max_rel
    mean_rel = GRAD_MEAN_REL if mean_rel is None else mean_rel
    assert mx <= max_rel, f"{what}: max error {mx:.3e} of the largest gradient > {max_rel}"
    assert mean <= mean_rel, f"{what}: mean error {mean:.3e} of the mean gradient > {mean_rel}"


def run_dense_train(q, k, v, gate, dout, topk, dev=G.DEV, block_size=64, bshd=False):
    """Coarse/top-k, the training forward, the plain fused forward and the
    backward on dense [B, H, S, D] CPU bf16 tensors; returns CPU results in
    [B, H, S(, D)].  With ``bshd`` the tensors go to the library as
    [B, S, H, D] (gate [B, S, H(, D)]) and come back transposed."""
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    conv = G.to_bshd if bshd else (lambda t: t)
    q, k, v, dout = (conv(t).to(dev) for t in (q, k, v, dout))
    gate = None if gate is None else conv(gate).to(dev)
    prob = vsa.dense_problem(B, H, Sq, Skv, D, topk, block_size, bshd)
    cs, isz, ns = vsa.block_shapes(prob)
    out_c = torch.empty(cs, dtype=torch.float32, device=dev)
    idx = torch.empty(isz, dtype=torch.int32, device=dev)
    num = torch.empty(ns, dtype=torch.int32, device=dev)
    vsa.vsa_coarse_topk(prob, q, k, v, out_c, idx, num, vsa.alloc_workspace(prob, dev))
    out = torch.empty_like(q)
    out_s = torch.empty_like(q)
    lse = torch.empty(vsa.lse_shape(prob), dtype=torch.float32, device=dev)
    vsa.vsa_sparse_attn_combine_train(prob, q, k, v, idx, num, out_c, gate, out, out_s, lse)
    out_plain = torch.empty_like(q)
    vsa.vsa_sparse_attn_combine(prob, q, k, v, idx, num, out_c, gate, out_plain)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = None if gate is None else torch.empty(gate.shape, dtype=torch.bfloat16, device=dev)
    vsa.vsa_backward(prob, q, k, v, idx, num, out_c, gate, out_s, lse, dout, dq, dk, dv, dg)
    torch.cuda.synchronize()
    back = G.from_bshd if bshd else (lambda t: t)
    cpu = lambda t: None if t is None else back(t.cpu())
    return dict(out=cpu(out), out_plain=cpu(out_plain), out_s=cpu(out_s), lse=lse.cpu(), q2k_idx=idx.cpu(),
                q2k_num=num.cpu(), dq=cpu(dq), dk=cpu(dk), dv=cpu(dv), dgate=cpu(dg), out_c=out_c.cpu())


def check_dense_case(q, k, v, gate, topk, seed, tag, block_size=64, bshd=False, max_rel=None, mean_rel=None,
                     lse_abs=LSE_ABS):
    G.note(f"case {tag}: q {tuple(q.shape)} kv {tuple(k.shape)} topk={topk} block={block_size} bshd={bshd} "
           f"gate={'none' if gate is None else tuple(gate.shape)}")
    dout = synth.output_grad(q.shape, seed)
    gpu = run_dense_train(q, k, v, gate, dout, topk, block_size=block_size, bshd=bshd)
    ref = BW.vsa_backward(N.f64(q), N.f64(k), N.f64(v), topk, None if gate is None else N.f64(gate), N.f64(dout),
                          block=block_size)
    G.assert_tie_free(ref)
    G.assert_indices_equal(gpu["q2k_idx"], gpu["q2k_num"], ref)
    assert torch.equal(gpu["out"], gpu["out_plain"]), "training forward changed the output bits"
    N.check_out(N.f64(gpu["out"]), ref["out"])
    N.check_sparse(N.f64(gpu["out_s"]), ref["out_s"])
    dl = float(np.abs(N.f64(gpu["lse"]) - ref["lse"]).max())
    G.note(f"  lse max-abs {dl:.2e}")
    assert dl <= lse_abs, f"lse: max-abs {dl:.3e} > {lse_abs}"
    for name in ("dq", "dk", "dv"):
        check_grad(N.f64(gpu[name]), ref[name], name, max_rel, mean_rel)
    if gate is not None:
        check_grad(N.f64(gpu["dgate"]), ref["dgate"], "dgate", max_rel, mean_rel)
    return gpu, ref


def test_backward_tiny():
    inp = synth.workload("tiny")
    check_dense_case(inp.q, inp.k, inp.v, None, inp.topk, 2001, "tiny")


@pytest.mark.parametrize("D", [64, 128])
def test_backward_token_gate_ragged(D):
    inp = synth.dense_inputs(1, 2, 64 * 5 + 17, D, 2, seed=2002 + D, gated=True)
    check_dense_case(inp.q, inp.k, inp.v, inp.gate, 2, 2003 + D, f"token gate D={D}")


@pytest.mark.parametrize("D", [64, 128])
def test_backward_full_gate_sq_ne_skv(D):
    inp = synth.dense_inputs(2, 2, 64 * 3 + 10, D, 3, seed=2010 + D, S_kv=64 * 5 + 33)
    gate = synth.full_gate((2, 2, 64 * 3 + 10, D), 2011 + D)
    check_dense_case(inp.q, inp.k, inp.v, gate, 3, 2012 + D, f"full gate Sq!=Skv D={D}")


def test_backward_every_block_selected():
    """top-k = every KV block: the sparse part is dense attention."""
    inp = synth.dense_inputs(1, 3, 64 * 4, 128, 4, seed=2020)
    gpu, _ = check_dense_case(inp.q, inp.k, inp.v, None, 4, 2021, "every block")
    assert (gpu["q2k_num"].numpy() == 4).all()


@pytest.mark.parametrize("Sq,Skv", [(1, 200), (70, 40), (64, 64), (130, 1)])
def test_backward_degenerate_lengths(Sq, Skv):
    """One-token queries, a single (partial) KV block, exact block multiples."""
    inp = synth.dense_inputs(1, 2, Sq, 64, 2, seed=2030 + Sq, S_kv=Skv, gated=True)
    check_dense_case(inp.q, inp.k, inp.v, inp.gate, 2, 2031 + Sq + Skv, f"Sq={Sq} Skv={Skv}")


@pytest.mark.parametrize("scale", [1.5, 3.0, 8.0])
def test_backward_sharp_softmax(scale):
    """Q and K scaled up: nearly one-hot probabilities, large log-sum-exp
    values and a running maximum that moves far past the lazy-rescale
    threshold; the recomputed probabilities and dS must still match.  The
    error relative to the largest gradient keeps the usual bound; the mean
    bound is wider here (measured 2.5e-3, 5.9e-3 and 1.4e-2 for dq at the
    three scales): as the softmax sharpens, dq and dk concentrate on a few
    large entries, so their mean shrinks against the largest one, while the
    bf16 rounding of dS and of the output that delta = sum(dout * out_s) is
    formed from scales with the largest entries.  (The pages' backward test
    uses a 5 % relative tolerance.)"""
    inp = synth.dense_inputs(1, 2, 64 * 6 + 9, 128, 3, seed=2040 + int(scale), gated=True)
    q = (inp.q.float() * scale).to(torch.bfloat16)
    k = (inp.k.float() * scale).to(torch.bfloat16)
    check_dense_case(q, k, inp.v, inp.gate, 3, 2041 + int(scale), f"sharp softmax x{scale}",
                     mean_rel=3e-2)


def test_backward_is_deterministic():
    inp = synth.dense_inputs(1, 2, 64 * 6 + 3, 128, 3, seed=2040, gated=True)
    dout = synth.output_grad(inp.q.shape, 2041)
    a = run_dense_train(inp.q, inp.k, inp.v, inp.gate, dout, 3)
    b = run_dense_train(inp.q, inp.k, inp.v, inp.gate, dout, 3)
    for name in ("dq", "dk", "dv", "dgate", "out", "lse"):
        assert torch.equal(a[name], b[name]), name


def test_autograd_wrapper_matches_entry_points():
    """video_sparse_attn under autograd calls the same kernels: bitwise the
    gradients of the direct calls."""
    inp = synth.dense_inputs(1, 2, 64 * 3 + 5, 64, 2, seed=2050, gated=True)
    dout = synth.output_grad(inp.q.shape, 2051)
    direct = run_dense_train(inp.q, inp.k, inp.v, inp.gate, dout, 2)
    q, k, v, g = (t.to(G.DEV).requires_grad_(True) for t in (inp.q, inp.k, inp.v, inp.gate))
    out = vsa.video_sparse_attn(q, k, v, 2, g)
    out.backward(dout.to(G.DEV))
    torch.cuda.synchronize()
    assert torch.equal(out.detach().cpu(), direct["out"])
    for t, name in ((q, "dq"), (k, "dk"), (v, "dv"), (g, "dgate")):
        assert torch.equal(t.grad.cpu(), direct[name]), name


# ---------------------------------------------------------------------------
# packed sequences: every sequence against its own dense oracle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("block", [64, 128, 256])
def test_backward_varlen_matches_per_sequence(block):
    """With VSA blocks of 128 / 256 slots the packed blocks hold empty 64-token
    blocks (135 tokens at 256: 64 + 64 + 7 + 0; 129 KV tokens: 64 + 64 + 1 + 0;
    320 KV tokens: a second VSA block of 64 + 0 + 0 + 0)."""
    seqlens_q = [64 * 2 + 7, 64 * 4, 30]
    seqlens_kv = [64 * 3 + 50, 64 * 2 + 1, 64 * 5]
    topk = [2, 1, 3]
    H, D = 2, 128
    inp = synth.varlen_inputs(seqlens_q, seqlens_kv, H, D, topk, seed=2060 + block, gated=True, block=block)
    G.note(f"case varlen block={block}: seqlens_q={seqlens_q} seqlens_kv={seqlens_kv} topk={topk}")
    dev = G.DEV
    meta = vsa.vsa_build_metadata(seqlens_q, seqlens_kv, topk, device=dev, block_size=block)
    prob = meta.problem(H, D)
    q, k, v, gate = (t.to(dev) for t in (inp.q, inp.k, inp.v, inp.gate))
    dout_cpu = synth.output_grad(inp.q.shape, 2061)
    dout = dout_cpu.to(dev)
    cs, isz, ns = vsa.block_shapes(prob)
    out_c = torch.empty(cs, dtype=torch.float32, device=dev)
    idx = torch.empty(isz, dtype=torch.int32, device=dev)
    num = torch.empty(ns, dtype=torch.int32, device=dev)
    vsa.vsa_coarse_topk(prob, q, k, v, out_c, idx, num, vsa.alloc_workspace(prob, dev))
    out = torch.full_like(q, float("nan"))
    out_s = torch.full_like(q, float("nan"))
    lse = torch.empty(vsa.lse_shape(prob), dtype=torch.float32, device=dev)
    vsa.vsa_sparse_attn_combine_train(prob, q, k, v, idx, num, out_c, gate, out, out_s, lse)
    nan = float("nan")
    dq, dk, dv = (torch.full_like(t, nan) for t in (q, k, v))
    dg = torch.full_like(gate, nan)
    vsa.vsa_backward(prob, q, k, v, idx, num, out_c, gate, out_s, lse, dout, dq, dk, dv, dg)
    torch.cuda.synchronize()
    dq, dk, dv, dg, lse = (t.cpu() for t in (dq, dk, dv, dg, lse))
    # the autograd wrapper over the same packed problem: the same bits
    qa, ka, va, ga = (t.clone().requires_grad_(True) for t in (q, k, v, gate))
    outa = vsa.video_sparse_attn_varlen(qa, ka, va, meta, ga)
    outa.backward(dout)
    torch.cuda.synchronize()
    assert torch.equal(outa.detach().cpu(), out.cpu())
    for t, want, name in ((qa, dq, "dq"), (ka, dk, "dk"), (va, dv, "dv"), (ga, dg, "dgate")):
        assert torch.equal(t.grad.cpu(), want), f"autograd {name}"
    oq = okv = 0
    for s, (sq, skv) in enumerate(zip(seqlens_q, seqlens_kv)):
        per = inp.per_seq[s]
        g64 = lambda t: N.f64(t)[None]
        ref = BW.vsa_backward(g64(per["q"]), g64(per["k"]), g64(per["v"]), topk[s], g64(per["gate"]),
                              N.f64(dout_cpu[:, oq:oq + sq])[None], block=block)
        G.assert_tie_free(ref)
        G.note(f"  sequence {s}")
        check_grad(N.f64(dq[:, oq:oq + sq]), ref["dq"][0], "dq")
        check_grad(N.f64(dk[:, okv:okv + skv]), ref["dk"][0], "dk")
        check_grad(N.f64(dv[:, okv:okv + skv]), ref["dv"][0], "dv")
        check_grad(N.f64(dg[:, oq:oq + sq]), ref["dgate"][0], "dgate")
        dl = float(np.abs(N.f64(lse[:, oq:oq + sq]) - ref["lse"][0]).max())
        assert dl <= LSE_ABS, f"lse of sequence {s}: {dl:.3e}"
        nq, nkv = -(-sq // block), -(-skv // block)
        # padding slots of every gradient are written with 0
        assert (dq[:, oq + sq:oq + block * nq] == 0).all() and (dg[:, oq + sq:oq + block * nq] == 0).all()
        assert (dk[:, okv + skv:okv + block * nkv] == 0).all() and (dv[:, okv + skv:okv + block * nkv] == 0).all()
        oq += block * nq
        okv += block * nkv


# ---------------------------------------------------------------------------
# VSA blocks of 128 / 256 tokens and [B, S, H, D] tensors
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("block,B,H,Sq,Skv,D,topk,gate", [
    (128, 1, 2, 128 * 3 + 37, 128 * 3 + 37, 128, 2, "token"),  # ragged 37-token last VSA block
    (128, 2, 1, 128 * 2 + 70, 128 * 4 + 9, 64, 2, "full"),     # Sq != Skv, full gate, D = 64
    (256, 1, 2, 256 * 2 + 100, 256 * 2 + 100, 128, 1, "token"),  # top-1, 100-token tail (2 sub-blocks)
    (256, 1, 1, 256 * 3, 256 * 3 - 30, 64, 3, None),           # every VSA block selected
])
def test_backward_large_vsa_blocks(block, B, H, Sq, Skv, D, topk, gate):
    inp = synth.dense_inputs(B, H, Sq, D, topk, seed=2500 + block + Sq, gated=gate == "token", S_kv=Skv)
    g = inp.gate if gate == "token" else (synth.full_gate((B, H, Sq, D), 2501 + Sq) if gate == "full" else None)
    check_dense_case(inp.q, inp.k, inp.v, g, topk, 2502 + Sq, f"block {block}", block_size=block)


@pytest.mark.parametrize("block,gate", [(64, "token"), (128, "full"), (256, None)])
def test_backward_bshd_matches_dense_bits(block, gate):
    """[B, S, H, D] tensors through the training forward and the backward give
    the bits of the [B, H, S, D] path (the same kernels, strided rows), and
    both match the oracle."""
    B, H, Sq, Skv, D = 2, 3, 64 * 5 + 17, 64 * 6 + 40, 128
    inp = synth.dense_inputs(B, H, Sq, D, 2, seed=2600 + block, gated=gate == "token", S_kv=Skv)
    g = inp.gate if gate == "token" else (synth.full_gate((B, H, Sq, D), 2601) if gate == "full" else None)
    gpu_b, _ = check_dense_case(inp.q, inp.k, inp.v, g, 2, 2602, f"bshd block {block}", block_size=block, bshd=True)
    dout = synth.output_grad(inp.q.shape, 2602)
    gpu_d = run_dense_train(inp.q, inp.k, inp.v, g, dout, 2, block_size=block)
    for key in ("out", "out_s", "lse", "q2k_idx", "q2k_num", "dq", "dk", "dv", "out_c") + (("dgate",) if g is not None else ()):
        assert torch.equal(gpu_b[key], gpu_d[key]), key


def test_autograd_large_blocks_bshd():
    """video_sparse_attn with 128-token VSA blocks on [B, S, H, D] tensors:
    the autograd gradients are the entry points' bits."""
    B, H, S, D = 1, 2, 128 * 3 + 20, 64
    inp = synth.dense_inputs(B, H, S, D, 2, seed=2700, gated=True)
    dout = synth.output_grad(inp.q.shape, 2701)
    ref = run_dense_train(inp.q, inp.k, inp.v, inp.gate, dout, 2, block_size=128, bshd=True)
    q, k, v, g = (G.to_bshd(t).to(G.DEV).requires_grad_(True) for t in (inp.q, inp.k, inp.v, inp.gate))
    out = vsa.video_sparse_attn(q, k, v, 2, g, block_size=128, bshd=True)
    out.backward(G.to_bshd(dout).to(G.DEV))
    torch.cuda.synchronize()
    assert torch.equal(G.from_bshd(out.detach().cpu()), ref["out"])
    for t, name in ((q, "dq"), (k, "dk"), (v, "dv"), (g, "dgate")):
        assert torch.equal(G.from_bshd(t.grad.cpu()), ref[name]), name


# ---------------------------------------------------------------------------
# full size: the large shape in the benchmark's launch configuration, whole
# heads sampled (heads are independent, so a head's gradients need only it)
# ---------------------------------------------------------------------------

def test_backward_large_shape_sampled_heads():
    """B=1, H=56, D=128, S=15488 (242 blocks), top-49, token gate: the backward
    of all heads in one launch sequence, heads 0 and 55 against the oracle
    (about 30 s of oracle time per head)."""
    inp = synth.workload("large")
    B, H, Sq, Skv, D = inp.shape
    G.note(f"case large backward: H={H} S={Sq} topk={inp.topk}")
    dout = synth.output_grad(inp.q.shape, 1100)
    gpu = run_dense_train(inp.q, inp.k, inp.v, inp.gate, dout, inp.topk)
    for h in (0, H - 1):
        sl = slice(h, h + 1)
        ref = BW.vsa_backward(N.f64(inp.q[:, sl]), N.f64(inp.k[:, sl]), N.f64(inp.v[:, sl]), inp.topk,
                              N.f64(inp.gate[:, sl]), N.f64(dout[:, sl]))
        G.note(f"  head {h}")
        G.assert_tie_free(ref)
        G.assert_indices_equal(gpu["q2k_idx"][:, sl], gpu["q2k_num"][:, sl], ref)
        dl = float(np.abs(N.f64(gpu["lse"][:, sl]) - ref["lse"]).max())
        assert dl <= LSE_ABS, f"lse: {dl:.3e}"
        for name in ("dq", "dk", "dv", "dgate"):
            check_grad(N.f64(gpu[name][:, sl]), ref[name], name)


# ---------------------------------------------------------------------------
# HIP graph capture of the backward
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("block,pooled", [(64, False), (256, False), (64, True), (256, True)])
def test_backward_graph_replay(block, pooled):
    """vsa_backward (or, pooled, vsa_backward_pooled reading the forward
    workspace's block means) captured once in a graph on preallocated
    buffers; between replays a new output gradient is copied in and the
    backward runs eagerly on its own outputs; every replay equals the eager
    result bit for bit."""
    B, H, S, D, topk = 1, 2, 64 * 7 + 29, 128, 2
    inp = synth.dense_inputs(B, H, S, D, topk, seed=2900 + block, gated=True)
    dev = G.DEV
    q, k, v, g = (t.to(dev) for t in (inp.q, inp.k, inp.v, inp.gate))
    prob = vsa.dense_problem(B, H, S, S, D, topk, block)
    cs, isz, ns = vsa.block_shapes(prob)
    out_c = torch.empty(cs, dtype=torch.float32, device=dev)
    idx = torch.empty(isz, dtype=torch.int32, device=dev)
    num = torch.empty(ns, dtype=torch.int32, device=dev)
    fws = vsa.alloc_workspace(prob, dev)
    vsa.vsa_coarse_topk(prob, q, k, v, out_c, idx, num, fws)
    out, out_s = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty(vsa.lse_shape(prob), dtype=torch.float32, device=dev)
    vsa.vsa_sparse_attn_combine_train(prob, q, k, v, idx, num, out_c, g, out, out_s, lse)
    dout = synth.output_grad(q.shape, 2950).to(dev)
    grads_g = [torch.empty_like(t) for t in (q, k, v, g)]
    grads_e = [torch.empty_like(t) for t in (q, k, v, g)]
    ws_g, ws_e = vsa.alloc_backward_workspace(prob, dev), vsa.alloc_backward_workspace(prob, dev)
    run = lambda gr, ws: vsa.vsa_backward(prob, q, k, v, idx, num, out_c, g, out_s, lse, dout, *gr, ws,
                                          forward_workspace=fws if pooled else None)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a warm-up call outside the capture
        run(grads_g, ws_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(grads_g, ws_g)
    torch.cuda.synchronize()
    for rep in range(4):
        dout.copy_(synth.output_grad(q.shape, 2951 + rep).to(dev))
        run(grads_e, ws_e)
        torch.cuda.synchronize()
        for t in grads_g:
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for a, b, name in zip(grads_g, grads_e, ("dq", "dk", "dv", "dgate")):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager backward"
    G.note(f"  4 backward replays equal to the eager backward (block {block}, pooled {pooled})")


# ---------------------------------------------------------------------------
# vsa_backward_pooled: the block means come from the forward's workspace
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("case", ["dense64", "bshd128", "packed256", "chunked"])
def test_backward_pooled_matches_vsa_backward(case):
    """vsa_backward_pooled reads the float64 block means of q, k and v from
    the workspace of the vsa_coarse_topk call that made the routing instead of
    pooling the three tensors; its gradients must be bitwise those of
    vsa_backward (the same pooling arithmetic ran in the forward).  The
    chunked case runs the coarse stage in two chunks of query blocks (3000
    blocks on two heads), so the forward's block means must be complete
    although its score matrix only ever holds one chunk."""
    dev = G.DEV
    if case == "packed256":
        seqlens = [300, 130, 520]
        topk = [1, 1, 2]
        inp = synth.varlen_inputs(seqlens, None, 2, 128, topk, seed=2300, gated=True, block=256)
        # the problem points into meta's device arrays: meta must outlive every call
        meta = vsa.vsa_build_metadata(seqlens, None, topk, device=dev, block_size=256)
        prob = meta.problem(2, 128)
        q, k, v, gate = (t.to(dev) for t in (inp.q, inp.k, inp.v, inp.gate))
    else:
        if case == "dense64":
            B, H, Sq, Skv, D, topk, bs, bshd, mode = 2, 2, 64 * 3 + 20, 64 * 4 + 5, 128, 2, 64, False, "token"
        elif case == "bshd128":
            B, H, Sq, Skv, D, topk, bs, bshd, mode = 1, 3, 128 * 2 + 70, 128 * 3 + 9, 64, 2, 128, True, "full"
        else:
            B, H, Sq, Skv, D, topk, bs, bshd, mode = 1, 2, 64 * 3000, 64 * 3000, 64, 7, 64, False, "token"
        inp = synth.dense_inputs(B, H, Sq, D, topk, seed=2301, gated=True, S_kv=Skv)
        conv = G.to_bshd if bshd else (lambda t: t)
        q, k, v = (conv(t).to(dev) for t in (inp.q, inp.k, inp.v))
        gate = conv(inp.gate if mode == "token" else inp.gate[..., None].expand(*inp.q.shape).contiguous()).to(dev)
        prob = vsa.dense_problem(B, H, Sq, Skv, D, topk, bs, bshd)
    G.note(f"case pooled backward: {case}")
    cs, isz, ns = vsa.block_shapes(prob)
    out_c = torch.empty(cs, dtype=torch.float32, device=dev)
    idx = torch.empty(isz, dtype=torch.int32, device=dev)
    num = torch.empty(ns, dtype=torch.int32, device=dev)
    ws = vsa.alloc_workspace(prob, dev)
    vsa.vsa_coarse_topk(prob, q, k, v, out_c, idx, num, ws)
    out, out_s = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty(vsa.lse_shape(prob), dtype=torch.float32, device=dev)
    vsa.vsa_sparse_attn_combine_train(prob, q, k, v, idx, num, out_c, gate, out, out_s, lse)
    dout = synth.output_grad(tuple(q.shape), 2302).to(dev)
    grads = {}
    for name, fw in (("plain", None), ("pooled", ws)):
        nan = float("nan")
        dq, dk, dv, dg = (torch.full_like(t, nan) for t in (q, k, v, gate))
        vsa.vsa_backward(prob, q, k, v, idx, num, out_c, gate, out_s, lse, dout, dq, dk, dv, dg,
                         forward_workspace=fw)
        torch.cuda.synchronize()
        grads[name] = [t.cpu() for t in (dq, dk, dv, dg)]
    for what, a, b in zip(("dq", "dk", "dv", "dgate"), grads["plain"], grads["pooled"]):
        assert torch.isfinite(a.float()).all(), f"{case}: {what} has non-finite values"
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{case}: {what} differs"
