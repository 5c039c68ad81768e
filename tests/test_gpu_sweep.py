"""Seeded random sweep of the forward against the fp64 oracle (shapes,
head dims, VSA block sizes, both dense layouts, every gate mode, top-k up to
past the block count), packed batches (VSA blocks of 64, 128 and 256 slots;
forward and backward), and capture of the forward in a HIP graph replayed
against eager runs."""
import numpy as np
import pytest
import torch

import synth
import video_sparse_attention_amd as vsa
from tests import gpu_common as G
from tests import numerics as N

pytestmark = pytest.mark.gpu


def sweep_configs(n=24, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        block = int(rng.choice([64, 128, 256]))
        Sq = int(rng.integers(1, 9 * 64))
        Skv = Sq if rng.random() < 0.5 else int(rng.integers(1, 9 * 64))
        nkvb = -(-Skv // block)
        out.append(dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)), Sq=Sq, Skv=Skv,
                        D=int(rng.choice([64, 128])), block=block, bshd=bool(rng.random() < 0.5),
                        gate=str(rng.choice(["none", "token", "full"])),
                        topk=int(rng.integers(1, nkvb + 2)), seed=9000 + c))
    return out


def sweep_inputs(cfg):
    inp = synth.dense_inputs(cfg["B"], cfg["H"], cfg["Sq"], cfg["D"], cfg["topk"], seed=cfg["seed"],
                             gated=cfg["gate"] == "token", S_kv=cfg["Skv"])
    if cfg["gate"] == "full":
        inp.gate = synth.full_gate((cfg["B"], cfg["H"], cfg["Sq"], cfg["D"]), cfg["seed"] + 1)
    return inp


@pytest.mark.parametrize("cfg", sweep_configs(), ids=lambda c: f"s{c['seed']}")
def test_random_forward(cfg):
    G.note(f"case {cfg}")
    inp = sweep_inputs(cfg)
    ref = G.oracle_dense(inp, block=cfg["block"])
    G.assert_tie_free(ref)
    conv = G.to_bshd if cfg["bshd"] else (lambda t: t)
    q, k, v = (conv(t).to(G.DEV) for t in (inp.q, inp.k, inp.v))
    g = None if inp.gate is None else conv(inp.gate).to(G.DEV)
    out, oc, idx, num = vsa.vsa_forward(q, k, v, cfg["topk"], g, block_size=cfg["block"], bshd=cfg["bshd"],
                                        return_aux=True)
    torch.cuda.synchronize()
    out = G.from_bshd(out.cpu()) if cfg["bshd"] else out.cpu()
    G.assert_indices_equal(idx.cpu(), num.cpu(), ref)
    N.check_out_c(N.f64(oc), ref["out_c"])
    mx, mean = N.check_out(N.f64(out), ref["out"])
    G.note(f"  out max-abs {mx:.2e} mean-abs {mean:.2e}")


@pytest.mark.parametrize("block,bshd", [(64, False), (128, True)])
def test_forward_graph_replay(block, bshd):
    """vsa_forward captured once in a graph on preallocated buffers; between
    replays new inputs are copied in and the forward runs eagerly on its own
    buffers; every replay equals the eager result bit for bit."""
    B, H, S, D, topk = 1, 4, 64 * 9 + 13, 128, 3
    conv = G.to_bshd if bshd else (lambda t: t)
    first = synth.dense_inputs(B, H, S, D, topk, seed=9500, gated=True)
    q, k, v, g = (conv(t).to(G.DEV) for t in (first.q, first.k, first.v, first.gate))
    prob = vsa.dense_problem(B, H, S, S, D, topk, block, bshd)
    ws_g, ws_e = vsa.alloc_workspace(prob, G.DEV), vsa.alloc_workspace(prob, G.DEV)
    out_g, out_e = torch.empty_like(q), torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a warm-up call outside the capture
        vsa.vsa_forward(q, k, v, topk, g, block_size=block, bshd=bshd, out=out_g, workspace=ws_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        vsa.vsa_forward(q, k, v, topk, g, block_size=block, bshd=bshd, out=out_g, workspace=ws_g)
    torch.cuda.synchronize()
    for rep in range(4):
        nxt = synth.dense_inputs(B, H, S, D, topk, seed=9501 + rep, gated=True)
        for dst, src in ((q, nxt.q), (k, nxt.k), (v, nxt.v), (g, nxt.gate)):
            dst.copy_(conv(src).to(G.DEV))
        vsa.vsa_forward(q, k, v, topk, g, block_size=block, bshd=bshd, out=out_e, workspace=ws_e)
        torch.cuda.synchronize()
        out_g.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep} differs from the eager forward"
    G.note(f"  {4} replays equal to the eager forward (block {block}, bshd {bshd})")


@pytest.mark.parametrize("block", [64, 256])
def test_varlen_graph_replay(block):
    """vsa_forward_varlen (packed, VSA blocks of 64 or 256 slots) captured once
    in a graph on preallocated buffers; between replays new inputs are copied
    in and the forward runs eagerly on its own buffers; every replay equals the
    eager result bit for bit, padding slots included."""
    lq, lkv, H, D, topk = [300, 77, 530], [260, 400, 530], 2, 128, [2, 3, 2]

    def make(seed):
        return synth.varlen_inputs(lq, lkv, H, D, topk, seed=seed, gated=True, block=block)

    first = make(9550)
    q, k, v, g = (t.to(G.DEV) for t in (first.q, first.k, first.v, first.gate))
    meta = vsa.vsa_build_metadata(lq, lkv, topk, device=G.DEV, block_size=block)
    prob = meta.problem(H, D)
    ws_g, ws_e = vsa.alloc_workspace(prob, G.DEV), vsa.alloc_workspace(prob, G.DEV)
    out_g, out_e = torch.empty_like(q), torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a warm-up call outside the capture
        vsa.vsa_forward_varlen(q, k, v, meta, g, out=out_g, workspace=ws_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        vsa.vsa_forward_varlen(q, k, v, meta, g, out=out_g, workspace=ws_g)
    torch.cuda.synchronize()
    for rep in range(4):
        nxt = make(9551 + rep)
        for dst, src in ((q, nxt.q), (k, nxt.k), (v, nxt.v), (g, nxt.gate)):
            dst.copy_(src.to(G.DEV))
        vsa.vsa_forward_varlen(q, k, v, meta, g, out=out_e, workspace=ws_e)
        torch.cuda.synchronize()
        out_g.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep} differs from the eager forward"
    G.note(f"  4 replays equal to the eager packed forward (block {block})")


def varlen_configs(n=8, seed=78):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        ns = int(rng.integers(1, 6))
        lq = [int(x) for x in rng.integers(1, 6 * 64, ns)]
        lkv = lq if rng.random() < 0.5 else [int(x) for x in rng.integers(1, 6 * 64, ns)]
        topk = [int(rng.integers(1, -(-s // 64) + 2)) for s in lkv]
        out.append(dict(lq=lq, lkv=lkv, topk=topk, H=int(rng.integers(1, 4)), D=int(rng.choice([64, 128])),
                        gated=bool(rng.random() < 0.5), seed=9600 + c))
    return out


@pytest.mark.parametrize("cfg", varlen_configs(), ids=lambda c: f"v{c['seed']}")
def test_random_varlen(cfg):
    """Packed sequences of random lengths (Q and KV lengths equal or not,
    per-sequence top-k up to past the sequence's block count): every stage
    against the oracle's separate varlen path."""
    G.note(f"case {cfg}")
    inp = synth.varlen_inputs(cfg["lq"], cfg["lkv"], cfg["H"], cfg["D"], cfg["topk"], cfg["seed"], cfg["gated"])
    ref = G.oracle_varlen(inp)
    G.assert_tie_free(ref)
    gpu = G.run_varlen_stages(inp)
    G.assert_indices_equal(gpu["q2k_idx"], gpu["q2k_num"], ref)
    N.check_out_c(N.f64(gpu["out_c"]), ref["out_c"])
    N.check_sparse(N.f64(gpu["out_s"]), ref["out_s"])
    mx, mean = N.check_out(N.f64(gpu["out_fused"]), ref["out"], "out (fused combine)")
    G.note(f"  out max-abs {mx:.2e} mean-abs {mean:.2e}")


def backward_configs(n=10, seed=79):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        block = int(rng.choice([64, 128, 256]))
        Sq = int(rng.integers(1, 6 * 64))
        Skv = Sq if rng.random() < 0.5 else int(rng.integers(1, 6 * 64))
        out.append(dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 3)), Sq=Sq, Skv=Skv,
                        D=int(rng.choice([64, 128])), block=block, bshd=bool(rng.random() < 0.5),
                        gate=str(rng.choice(["none", "token", "full"])),
                        topk=int(rng.integers(1, -(-Skv // block) + 2)), seed=9700 + c))
    return out


@pytest.mark.parametrize("cfg", backward_configs(), ids=lambda c: f"b{c['seed']}")
def test_random_backward(cfg):
    """The training forward and the backward on random configurations
    against the backward oracle (tolerances of tests/test_gpu_backward.py)."""
    from tests.test_gpu_backward import check_dense_case
    inp = sweep_inputs(cfg)
    check_dense_case(inp.q, inp.k, inp.v, inp.gate, cfg["topk"], cfg["seed"] + 5, f"sweep {cfg}",
                     block_size=cfg["block"], bshd=cfg["bshd"])


def varlen_block_configs(n=8, seed=80, base=9800):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        block = int(rng.choice([128, 256]))
        ns = int(rng.integers(1, 5))
        lq = [int(x) for x in rng.integers(1, 4 * block, ns)]
        lkv = lq if rng.random() < 0.5 else [int(x) for x in rng.integers(1, 4 * block, ns)]
        topk = [int(rng.integers(1, -(-s // block) + 2)) for s in lkv]
        out.append(dict(lq=lq, lkv=lkv, topk=topk, H=int(rng.integers(1, 3)), D=int(rng.choice([64, 128])),
                        gated=bool(rng.random() < 0.5), block=block, seed=base + c))
    return out


@pytest.mark.parametrize("cfg", varlen_block_configs(), ids=lambda c: f"vb{c['seed']}")
def test_random_varlen_large_blocks(cfg):
    """Packed sequences of random lengths in VSA blocks of 128 / 256 slots
    (trailing 64-token blocks of a VSA block often empty): every stage against
    the oracle's separate varlen path."""
    G.note(f"case {cfg}")
    inp = synth.varlen_inputs(cfg["lq"], cfg["lkv"], cfg["H"], cfg["D"], cfg["topk"], cfg["seed"], cfg["gated"],
                              block=cfg["block"])
    ref = G.oracle_varlen(inp)
    G.assert_tie_free(ref)
    gpu = G.run_varlen_stages(inp)
    G.assert_indices_equal(gpu["q2k_idx"], gpu["q2k_num"], ref)
    N.check_out_c(N.f64(gpu["out_c"]), ref["out_c"])
    N.check_sparse(N.f64(gpu["out_s"]), ref["out_s"])
    mx, mean = N.check_out(N.f64(gpu["out_fused"]), ref["out"], "out (fused combine)")
    G.note(f"  out max-abs {mx:.2e} mean-abs {mean:.2e}")


@pytest.mark.parametrize("cfg", varlen_block_configs(n=6, seed=81, base=9900), ids=lambda c: f"vbb{c['seed']}")
def test_random_varlen_backward(cfg):
    """The packed training forward and backward (autograd wrapper) with VSA
    blocks of 128 / 256 slots: each sequence's gradients against the backward
    oracle run on that sequence alone; padding slots of every gradient 0."""
    from oracle import vsa_backward as BW
    from tests.test_gpu_backward import check_grad
    G.note(f"case {cfg}")
    inp = synth.varlen_inputs(cfg["lq"], cfg["lkv"], cfg["H"], cfg["D"], cfg["topk"], cfg["seed"], True,
                              block=cfg["block"])
    bs = cfg["block"]
    dev = G.DEV
    meta = vsa.vsa_build_metadata(cfg["lq"], cfg["lkv"], cfg["topk"], device=dev, block_size=bs)
    dout = synth.output_grad(inp.q.shape, cfg["seed"] + 7)
    q, k, v, g = (t.to(dev).requires_grad_(True) for t in (inp.q, inp.k, inp.v, inp.gate))
    vsa.video_sparse_attn_varlen(q, k, v, meta, g).backward(dout.to(dev))
    torch.cuda.synchronize()
    dq, dk, dv, dg = (t.grad.cpu() for t in (q, k, v, g))
    oq = okv = 0
    for s, (sq, skv) in enumerate(zip(cfg["lq"], cfg["lkv"])):
        per = inp.per_seq[s]
        one = lambda t: N.f64(t)[None]
        ref = BW.vsa_backward(one(per["q"]), one(per["k"]), one(per["v"]), cfg["topk"][s], one(per["gate"]),
                              N.f64(dout[:, oq:oq + sq])[None], block=bs)
        G.assert_tie_free(ref)
        check_grad(N.f64(dq[:, oq:oq + sq]), ref["dq"][0], f"dq[{s}]")
        check_grad(N.f64(dk[:, okv:okv + skv]), ref["dk"][0], f"dk[{s}]")
        check_grad(N.f64(dv[:, okv:okv + skv]), ref["dv"][0], f"dv[{s}]")
        check_grad(N.f64(dg[:, oq:oq + sq]), ref["dgate"][0], f"dgate[{s}]")
        nq, nkv = -(-sq // bs), -(-skv // bs)
        assert (dq[:, oq + sq:oq + bs * nq] == 0).all() and (dg[:, oq + sq:oq + bs * nq] == 0).all()
        assert (dk[:, okv + skv:okv + bs * nkv] == 0).all() and (dv[:, okv + skv:okv + bs * nkv] == 0).all()
        oq += bs * nq
        okv += bs * nkv
