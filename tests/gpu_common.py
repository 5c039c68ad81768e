"""Shared pieces of the GPU parity tests: running the HIP path through the C ABI
on seeded workloads and running the oracle on the same inputs."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth
import video_sparse_attention_amd as vsa
from tests.numerics import f64

DEV = "cuda:0"


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_bshd(t):
    """[B, H, S(, D)] -> contiguous [B, S, H(, D)] (None stays None)."""
    if t is None:
        return None
    return t.transpose(1, 2).contiguous()


def from_bshd(t):
    return t.transpose(1, 2).contiguous()


def run_dense_stages(inp, dev=DEV, idx_override=None, block_size=64, bshd=False):
    """Stage calls on a dense workload: returns dict with out, out_s, out_c,
    q2k_idx, q2k_num (CPU tensors).  With ``idx_override`` (numpy idx, num) the
    sparse stage runs on those indices instead of the GPU's own.  With
    ``bshd`` the inputs are handed over as [B, S, H, D] tensors (vsa problem
    of layout BSHD) and the token outputs are returned as [B, H, S, D]."""
    B, H, Sq, Skv, D = inp.shape
    conv = to_bshd if bshd else (lambda t: t)
    q, k, v = (conv(t).to(dev) for t in (inp.q, inp.k, inp.v))
    gate = None if inp.gate is None else conv(inp.gate).to(dev)
    prob = vsa.dense_problem(B, H, Sq, Skv, D, inp.topk, block_size, bshd)
    cs, isz, ns = vsa.block_shapes(prob)
    out_c = torch.empty(cs, dtype=torch.float32, device=dev)
    idx = torch.empty(isz, dtype=torch.int32, device=dev)
    num = torch.empty(ns, dtype=torch.int32, device=dev)
    ws = vsa.alloc_workspace(prob, dev)
    vsa.vsa_coarse_topk(prob, q, k, v, out_c, idx, num, ws)
    if idx_override is not None:
        sidx = torch.from_numpy(np.ascontiguousarray(idx_override[0])).to(dev)
        snum = torch.from_numpy(np.ascontiguousarray(idx_override[1])).to(dev)
    else:
        sidx, snum = idx, num
    out = torch.empty_like(q)
    vsa.vsa_sparse_attn_from_indices(prob, q, k, v, sidx, snum, out)
    out_s = out.clone()
    vsa.vsa_combine(prob, out_c, gate, out)
    out_f = torch.empty_like(q)
    vsa.vsa_sparse_attn_combine(prob, q, k, v, sidx, snum, out_c, gate, out_f)
    torch.cuda.synchronize()
    back = from_bshd if bshd else (lambda t: t)
    return dict(out=back(out.cpu()), out_s=back(out_s.cpu()), out_c=out_c.cpu(), q2k_idx=idx.cpu(),
                q2k_num=num.cpu(), out_fused=back(out_f.cpu()))


def run_varlen_stages(inp, dev=DEV, idx_override=None):
    meta = vsa.vsa_build_metadata(inp.seqlens_q, inp.seqlens_kv, inp.topk, device=dev, block_size=inp.block)
    H, D = inp.heads, inp.head_dim
    prob = meta.problem(H, D)
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    gate = None if inp.gate is None else inp.gate.to(dev)
    cs, isz, ns = vsa.block_shapes(prob)
    out_c = torch.empty(cs, dtype=torch.float32, device=dev)
    idx = torch.empty(isz, dtype=torch.int32, device=dev)
    num = torch.empty(ns, dtype=torch.int32, device=dev)
    ws = vsa.alloc_workspace(prob, dev)
    vsa.vsa_coarse_topk(prob, q, k, v, out_c, idx, num, ws)
    if idx_override is not None:
        sidx = torch.from_numpy(np.ascontiguousarray(idx_override[0])).to(dev)
        snum = torch.from_numpy(np.ascontiguousarray(idx_override[1])).to(dev)
    else:
        sidx, snum = idx, num
    out = torch.full_like(q, float("nan"))  # padding slots must come back as 0
    vsa.vsa_sparse_attn_from_indices(prob, q, k, v, sidx, snum, out)
    out_s = out.clone()
    vsa.vsa_combine(prob, out_c, gate, out)
    out_f = torch.full_like(q, float("nan"))
    vsa.vsa_sparse_attn_combine(prob, q, k, v, sidx, snum, out_c, gate, out_f)
    torch.cuda.synchronize()
    return dict(out=out.cpu(), out_s=out_s.cpu(), out_c=out_c.cpu(), q2k_idx=idx.cpu(),
                q2k_num=num.cpu(), meta=meta, out_fused=out_f.cpu())


def oracle_dense(inp, blocks=None, block=64):
    g = None if inp.gate is None else f64(inp.gate)
    return oracle.vsa_forward(f64(inp.q), f64(inp.k), f64(inp.v), inp.topk, g, blocks=blocks, block=block)


def oracle_varlen(inp, blocks=None):
    g = None if inp.gate is None else f64(inp.gate)
    return oracle.vsa_forward_varlen(f64(inp.q), f64(inp.k), f64(inp.v), inp.seqlens_q,
                                     inp.seqlens_kv, inp.topk, g, blocks=blocks, block=inp.block)


def assert_tie_free(ref):
    ok, min_gap, nbad = oracle.tie_free(ref["gap"], float(np.max(ref["max_abs_dot"])))
    note(f"  routing margin: min gap {min_gap:.3e}, rows at/below threshold {nbad}")
    assert ok, f"inputs are not tie-free ({nbad} rows), index parity is not meaningful"


def assert_indices_equal(gpu_idx, gpu_num, ref):
    gi = gpu_idx.numpy()
    gn = gpu_num.numpy()
    assert np.array_equal(gn, ref["q2k_num"]), "q2k_num differs"
    assert np.array_equal(gi, ref["q2k_idx"]), \
        f"q2k_idx differs in {int((gi != ref['q2k_idx']).any(axis=-1).sum())} rows"
