"""Thin PyTorch binding over libvsa: argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI
(``include/vsa.h``); this module checks tensor shapes, dtypes and devices,
takes device memory from PyTorch (outputs, workspace), passes raw pointers
and the current HIP stream, and turns error codes into ``VsaError``.  The
function names are those of the C entry points.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

from . import _abi
from ._abi import (VSA_GATE_FULL, VSA_GATE_NONE, VSA_GATE_TOKEN, VSA_LAYOUT_BSHD, VSA_LAYOUT_DENSE,
                   VSA_LAYOUT_PACKED, VsaError, VsaMetaSizes, VsaProblem)

BLOCK = 64


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape=None, contiguous=True, grad_ok=False):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.requires_grad and not grad_ok and torch.is_grad_enabled():
        raise RuntimeError(f"{name} requires grad: this entry point records no gradient, "
                           "use video_sparse_attn for training")


def _gate_args(gate: Optional[torch.Tensor], token_shape, full_shape, bshd: bool = False):
    """(mode, strides array or None) for a gate tensor, strict on shape; the
    C ABI takes element strides in (batch, head, token) order, so a BSHD gate's
    (batch, token, head) strides are reordered."""
    if gate is None:
        return VSA_GATE_NONE, None
    _need(gate, "gate", torch.bfloat16, contiguous=False)
    shp = tuple(gate.shape)
    if shp == tuple(token_shape):
        mode = VSA_GATE_TOKEN
        st = list(gate.stride())
    elif shp == tuple(full_shape):
        if gate.stride(-1) != 1:
            raise ValueError("a full gate needs unit stride over head_dim")
        mode = VSA_GATE_FULL
        st = list(gate.stride()[:-1])
    else:
        raise ValueError(f"gate has shape {shp}, expected {tuple(token_shape)} or {tuple(full_shape)}")
    if len(st) == 2:  # packed: [H, slots(, D)] -> (unused, head, slot)
        st = [0] + st
    elif bshd:  # [B, S, H(, D)] -> (batch, head, token)
        st = [st[0], st[2], st[1]]
    return mode, (ctypes.c_int64 * 3)(*st)


# ---------------------------------------------------------------------------
# metadata and problems
# ---------------------------------------------------------------------------

@dataclass
class VarlenMeta:
    sizes: VsaMetaSizes
    seqlens_q: List[int]
    seqlens_kv: List[int]
    cu_blocks_q: torch.Tensor      # host int32 [num_seqs + 1]
    cu_blocks_kv: torch.Tensor
    block_sizes_q: torch.Tensor    # host int32 [Nq]
    block_sizes_kv: torch.Tensor
    topk: torch.Tensor             # host int32 [num_seqs], clamped
    device_arrays: Optional[dict] = None
    block_size: int = BLOCK        # VSA block: slots per block

    def to(self, device) -> "VarlenMeta":
        names = ("cu_blocks_q", "cu_blocks_kv", "block_sizes_q", "block_sizes_kv", "topk")
        self.device_arrays = {n: getattr(self, n).to(device) for n in names}
        return self

    def problem(self, heads: int, head_dim: int) -> VsaProblem:
        if self.device_arrays is None:
            raise RuntimeError("call .to(device) before building a packed problem")
        d = self.device_arrays
        s = self.sizes
        p = VsaProblem(
            layout=VSA_LAYOUT_PACKED, heads=heads, head_dim=head_dim, block_size=self.block_size,
            num_seqs=s.num_seqs, total_q_blocks=s.total_q_blocks,
            total_kv_blocks=s.total_kv_blocks, max_q_blocks=s.max_q_blocks,
            max_kv_blocks=s.max_kv_blocks, max_topk=s.max_topk,
            cu_blocks_q=d["cu_blocks_q"].data_ptr(), cu_blocks_kv=d["cu_blocks_kv"].data_ptr(),
            block_sizes_q=d["block_sizes_q"].data_ptr(),
            block_sizes_kv=d["block_sizes_kv"].data_ptr(), topk_per_seq=d["topk"].data_ptr())
        # the problem carries raw device addresses of these arrays: it keeps
        # them alive itself, so a problem outliving its VarlenMeta stays valid
        p._device_arrays = d
        return p


def vsa_build_metadata(seqlens_q: Sequence[int], seqlens_kv: Optional[Sequence[int]] = None,
                       topk: Sequence[int] = (), device=None, block_size: int = BLOCK) -> VarlenMeta:
    """Host block metadata for packed sequences (vsa_build_metadata), VSA
    blocks of ``block_size`` (64, 128 or 256) tokens and slots."""
    lib = _abi.load()
    n = len(seqlens_q)
    sq = (ctypes.c_int32 * max(n, 1))(*seqlens_q)
    skv = None if seqlens_kv is None else (ctypes.c_int32 * max(n, 1))(*seqlens_kv)
    if len(topk) != n:
        raise ValueError("topk needs one entry per sequence")
    tk = (ctypes.c_int32 * max(n, 1))(*topk)
    sizes = VsaMetaSizes()
    _abi.check(lib.vsa_build_metadata(n, sq, skv, tk, block_size, ctypes.byref(sizes),
                                      None, None, None, None, None), "vsa_build_metadata")
    cu_q = torch.zeros(n + 1, dtype=torch.int32)
    cu_kv = torch.zeros(n + 1, dtype=torch.int32)
    bs_q = torch.zeros(sizes.total_q_blocks, dtype=torch.int32)
    bs_kv = torch.zeros(sizes.total_kv_blocks, dtype=torch.int32)
    tkc = torch.zeros(n, dtype=torch.int32)
    _abi.check(lib.vsa_build_metadata(n, sq, skv, tk, block_size, ctypes.byref(sizes), _ptr(cu_q),
                                      _ptr(cu_kv), _ptr(bs_q), _ptr(bs_kv), _ptr(tkc)), "vsa_build_metadata")
    meta = VarlenMeta(sizes, list(seqlens_q), list(seqlens_q if seqlens_kv is None else seqlens_kv),
                      cu_q, cu_kv, bs_q, bs_kv, tkc, block_size=block_size)
    return meta.to(device) if device is not None else meta


def dense_problem(batch: int, heads: int, seqlen_q: int, seqlen_kv: int, head_dim: int,
                  topk: int, block_size: int = BLOCK, bshd: bool = False) -> VsaProblem:
    """A DENSE ([B,H,S,D]) or, with ``bshd``, BSHD ([B,S,H,D]) problem;
    ``block_size`` 64, 128 or 256."""
    return VsaProblem(layout=VSA_LAYOUT_BSHD if bshd else VSA_LAYOUT_DENSE, heads=heads, head_dim=head_dim,
                      block_size=block_size, batch=batch, seqlen_q=seqlen_q, seqlen_kv=seqlen_kv, topk=topk)


def vsa_workspace_size(problem: VsaProblem) -> int:
    return int(_abi.load().vsa_workspace_size(ctypes.byref(problem)))


def alloc_workspace(problem: VsaProblem, device) -> torch.Tensor:
    n = vsa_workspace_size(problem)
    if n == 0:
        raise VsaError(_abi.VSA_ERR_SHAPE, (_abi.load().vsa_last_error() or b"").decode(),
                       "vsa_workspace_size")
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n]


def block_shapes(problem: VsaProblem):
    """(out_c shape, q2k_idx shape, q2k_num shape) of a problem."""
    if problem.layout in (VSA_LAYOUT_DENSE, VSA_LAYOUT_BSHD):
        nq = -(-problem.seqlen_q // problem.block_size)
        nkv = -(-problem.seqlen_kv // problem.block_size)
        kk = min(problem.topk, nkv)
        b, h, d = problem.batch, problem.heads, problem.head_dim
        return (b, h, nq, d), (b, h, nq, kk), (b, h, nq)
    h, nq, d = problem.heads, problem.total_q_blocks, problem.head_dim
    return (h, nq, d), (h, nq, problem.max_topk), (h, nq)


def token_shapes(problem: VsaProblem):
    """(q/out shape, k/v shape) of a problem."""
    h, d = problem.heads, problem.head_dim
    if problem.layout == VSA_LAYOUT_DENSE:
        b = problem.batch
        return (b, h, problem.seqlen_q, d), (b, h, problem.seqlen_kv, d)
    if problem.layout == VSA_LAYOUT_BSHD:
        b = problem.batch
        return (b, problem.seqlen_q, h, d), (b, problem.seqlen_kv, h, d)
    bs = problem.block_size
    return (h, bs * problem.total_q_blocks, d), (h, bs * problem.total_kv_blocks, d)


# ---------------------------------------------------------------------------
# stage entry points
# ---------------------------------------------------------------------------

def _check_qkv(problem, q, k, v):
    qs, ks = token_shapes(problem)
    _need(q, "q", torch.bfloat16, qs)
    _need(k, "k", torch.bfloat16, ks)
    _need(v, "v", torch.bfloat16, ks)


def vsa_coarse_topk(problem: VsaProblem, q, k, v, out_c, q2k_idx, q2k_num, workspace) -> None:
    _check_qkv(problem, q, k, v)
    cs, isz, ns = block_shapes(problem)
    _need(out_c, "out_c", torch.float32, cs)
    _need(q2k_idx, "q2k_idx", torch.int32, isz)
    _need(q2k_num, "q2k_num", torch.int32, ns)
    _need(workspace, "workspace", torch.uint8)
    _abi.check(_abi.load().vsa_coarse_topk(
        ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(out_c), _ptr(q2k_idx),
        _ptr(q2k_num), _ptr(workspace), workspace.numel(), _stream(q.device)), "vsa_coarse_topk")


def vsa_sparse_attn_from_indices(problem: VsaProblem, q, k, v, q2k_idx, q2k_num, out) -> None:
    _check_qkv(problem, q, k, v)
    _, isz, ns = block_shapes(problem)
    if tuple(q2k_idx.shape[:-1]) != tuple(isz[:-1]):
        raise ValueError(f"q2k_idx has shape {tuple(q2k_idx.shape)}, expected {isz[:-1]} + (k,)")
    if problem.layout != VSA_LAYOUT_PACKED and q2k_idx.shape[-1] != isz[-1]:
        raise ValueError(f"q2k_idx rows must hold min(topk, nKV) = {isz[-1]} entries")
    _need(q2k_idx, "q2k_idx", torch.int32)
    _need(q2k_num, "q2k_num", torch.int32, ns)
    _need(out, "out", torch.bfloat16, token_shapes(problem)[0])
    _abi.check(_abi.load().vsa_sparse_attn_from_indices(
        ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(q2k_idx), _ptr(q2k_num), _ptr(out),
        _stream(q.device)), "vsa_sparse_attn_from_indices")


def vsa_sparse_attn_combine(problem: VsaProblem, q, k, v, q2k_idx, q2k_num, out_c, gate, out) -> None:
    """Block-sparse attention with the combine fused into its epilogue:
    ``out = out_c[block] * gate + attention`` (``+`` without a gate), one
    rounding to bf16."""
    _check_qkv(problem, q, k, v)
    cs, isz, ns = block_shapes(problem)
    if tuple(q2k_idx.shape[:-1]) != tuple(isz[:-1]):
        raise ValueError(f"q2k_idx has shape {tuple(q2k_idx.shape)}, expected {isz[:-1]} + (k,)")
    if problem.layout != VSA_LAYOUT_PACKED and q2k_idx.shape[-1] != isz[-1]:
        raise ValueError(f"q2k_idx rows must hold min(topk, nKV) = {isz[-1]} entries")
    _need(q2k_idx, "q2k_idx", torch.int32)
    _need(q2k_num, "q2k_num", torch.int32, ns)
    _need(out_c, "out_c", torch.float32, cs)
    _need(out, "out", torch.bfloat16, token_shapes(problem)[0])
    mode, st = _gate_args(gate, *_gate_shapes(problem))
    _abi.check(_abi.load().vsa_sparse_attn_combine(
        ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(q2k_idx), _ptr(q2k_num), _ptr(out_c),
        _ptr(gate), mode, st, _ptr(out), _stream(q.device)), "vsa_sparse_attn_combine")


def _gate_shapes(problem):
    qs = token_shapes(problem)[0]
    return qs[:-1], qs, problem.layout == VSA_LAYOUT_BSHD


def vsa_combine(problem: VsaProblem, out_c, gate, out) -> None:
    cs, _, _ = block_shapes(problem)
    _need(out_c, "out_c", torch.float32, cs)
    _need(out, "out", torch.bfloat16, token_shapes(problem)[0])
    mode, st = _gate_args(gate, *_gate_shapes(problem))
    _abi.check(_abi.load().vsa_combine(
        ctypes.byref(problem), _ptr(out_c), _ptr(gate), mode, st, _ptr(out),
        _stream(out.device)), "vsa_combine")


# ---------------------------------------------------------------------------
# training: forward that keeps out_s and lse, backward
# ---------------------------------------------------------------------------

def lse_shape(problem: VsaProblem):
    """[B, H, Sq] for both dense layouts (also for [B, S, H, D] tensors),
    [H, slots] packed."""
    if problem.layout in (VSA_LAYOUT_DENSE, VSA_LAYOUT_BSHD):
        return (problem.batch, problem.heads, problem.seqlen_q)
    return token_shapes(problem)[0][:-1]


def vsa_sparse_attn_combine_train(problem: VsaProblem, q, k, v, q2k_idx, q2k_num, out_c, gate, out,
                                  out_s, lse) -> None:
    """vsa_sparse_attn_combine that also writes ``out_s`` (the bf16 sparse
    attention output on its own) and ``lse`` (float32 per query row, log2 of
    the softmax denominator in exp2 units of the scaled scores)."""
    _check_qkv(problem, q, k, v)
    cs, isz, ns = block_shapes(problem)
    if tuple(q2k_idx.shape[:-1]) != tuple(isz[:-1]):
        raise ValueError(f"q2k_idx has shape {tuple(q2k_idx.shape)}, expected {isz[:-1]} + (k,)")
    _need(q2k_idx, "q2k_idx", torch.int32)
    _need(q2k_num, "q2k_num", torch.int32, ns)
    _need(out_c, "out_c", torch.float32, cs)
    qs = token_shapes(problem)[0]
    _need(out, "out", torch.bfloat16, qs)
    _need(out_s, "out_s", torch.bfloat16, qs)
    _need(lse, "lse", torch.float32, lse_shape(problem))
    mode, st = _gate_args(gate, *_gate_shapes(problem))
    _abi.check(_abi.load().vsa_sparse_attn_combine_train(
        ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(q2k_idx), _ptr(q2k_num), _ptr(out_c),
        _ptr(gate), mode, st, _ptr(out), _ptr(out_s), _ptr(lse), _stream(q.device)),
        "vsa_sparse_attn_combine_train")


def vsa_backward_workspace_size(problem: VsaProblem) -> int:
    return int(_abi.load().vsa_backward_workspace_size(ctypes.byref(problem)))


def alloc_backward_workspace(problem: VsaProblem, device) -> torch.Tensor:
    n = vsa_backward_workspace_size(problem)
    if n == 0:
        raise VsaError(_abi.VSA_ERR_SHAPE, (_abi.load().vsa_last_error() or b"").decode(),
                       "vsa_backward_workspace_size")
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n]


def vsa_backward(problem: VsaProblem, q, k, v, q2k_idx, q2k_num, out_c, gate, out_s, lse, dout,
                 dq, dk, dv, dgate=None, workspace=None, forward_workspace=None) -> None:
    """Gradients of ``sum(out * dout)`` of the forward with these inputs and
    routing (vsa_backward): writes ``dq``, ``dk``, ``dv`` and, with a gate,
    ``dgate`` (contiguous, the gate's shape: [B, H, Sq(, D)], or [B, Sq, H(, D)]
    for a BSHD problem).  ``forward_workspace``: the workspace of the
    ``vsa_coarse_topk`` call that produced the routing, unchanged since; its
    block means of q, k and v are then reused (vsa_backward_pooled) instead of
    pooling the three tensors again."""
    _check_qkv(problem, q, k, v)
    cs, isz, ns = block_shapes(problem)
    if tuple(q2k_idx.shape[:-1]) != tuple(isz[:-1]):
        raise ValueError(f"q2k_idx has shape {tuple(q2k_idx.shape)}, expected {isz[:-1]} + (k,)")
    _need(q2k_idx, "q2k_idx", torch.int32)
    _need(q2k_num, "q2k_num", torch.int32, ns)
    _need(out_c, "out_c", torch.float32, cs)
    qs, ks = token_shapes(problem)
    _need(out_s, "out_s", torch.bfloat16, qs)
    _need(lse, "lse", torch.float32, lse_shape(problem))
    _need(dout, "dout", torch.bfloat16, qs)
    _need(dq, "dq", torch.bfloat16, qs)
    _need(dk, "dk", torch.bfloat16, ks)
    _need(dv, "dv", torch.bfloat16, ks)
    mode, st = _gate_args(gate, *_gate_shapes(problem))
    if mode != VSA_GATE_NONE:
        _need(dgate, "dgate", torch.bfloat16, gate.shape)
    if workspace is None:
        workspace = alloc_backward_workspace(problem, q.device)
    _need(workspace, "workspace", torch.uint8)
    dg = _ptr(dgate if mode != VSA_GATE_NONE else None)
    if forward_workspace is None:
        _abi.check(_abi.load().vsa_backward(
            ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(q2k_idx), _ptr(q2k_num), _ptr(out_c),
            _ptr(gate), mode, st, _ptr(out_s), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), dg,
            _ptr(workspace), workspace.numel(), _stream(q.device)), "vsa_backward")
        return
    _need(forward_workspace, "forward_workspace", torch.uint8)
    _abi.check(_abi.load().vsa_backward_pooled(
        ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(q2k_idx), _ptr(q2k_num), _ptr(out_c),
        _ptr(gate), mode, st, _ptr(out_s), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), dg,
        _ptr(forward_workspace), forward_workspace.numel(), _ptr(workspace), workspace.numel(),
        _stream(q.device)), "vsa_backward_pooled")


class _VideoSparseAttn(torch.autograd.Function):
    """Autograd wrapper: forward = vsa_coarse_topk + vsa_sparse_attn_combine_train,
    backward = vsa_backward_pooled (the routing is held fixed; the forward's
    workspace is kept for the backward, which reuses its block means of q, k
    and v)."""

    @staticmethod
    def forward(ctx, q, k, v, gate, problem, keep):
        # keep: the packed metadata whose device arrays the problem points to
        q, k, v = q.detach(), k.detach(), v.detach()
        g = None if gate is None else gate.detach()
        cs, isz, ns = block_shapes(problem)
        dev = q.device
        out_c = torch.empty(cs, dtype=torch.float32, device=dev)
        idx = torch.empty(isz, dtype=torch.int32, device=dev)
        num = torch.empty(ns, dtype=torch.int32, device=dev)
        ws = alloc_workspace(problem, dev)
        vsa_coarse_topk(problem, q, k, v, out_c, idx, num, ws)
        out = torch.empty_like(q)
        out_s = torch.empty_like(q)
        lse = torch.empty(lse_shape(problem), dtype=torch.float32, device=dev)
        vsa_sparse_attn_combine_train(problem, q, k, v, idx, num, out_c, g, out, out_s, lse)
        ctx.problem = problem
        ctx.keep = keep
        ctx.has_gate = g is not None
        ctx.save_for_backward(q, k, v, *( [g] if g is not None else []), idx, num, out_c, out_s, lse, ws)
        ctx.mark_non_differentiable(idx, num)
        return out, idx, num

    @staticmethod
    def backward(ctx, dout, _didx, _dnum):
        saved = list(ctx.saved_tensors)
        q, k, v = saved[:3]
        g = saved[3] if ctx.has_gate else None
        idx, num, out_c, out_s, lse, ws = saved[4 if ctx.has_gate else 3:]
        dout = dout.contiguous()
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dg = None if g is None else torch.empty(g.shape, dtype=torch.bfloat16, device=q.device)
        vsa_backward(ctx.problem, q, k, v, idx, num, out_c, g, out_s, lse, dout, dq, dk, dv, dg,
                     forward_workspace=ws)
        return dq, dk, dv, dg, None, None


def video_sparse_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, topk: int,
                      gate: Optional[torch.Tensor] = None, return_routing: bool = False, *,
                      block_size: int = BLOCK, bshd: bool = False):
    """Differentiable VSA on dense ``[B, H, S, D]`` bf16 tensors (``[B, S, H, D]``
    with ``bshd``): the forward of ``vsa_forward`` and, through autograd, the
    gradients of q, k, v and the gate (``[B, H, Sq]`` or ``[B, H, Sq, D]``;
    ``[B, Sq, H(, D)]`` with ``bshd``) from vsa_backward.  ``block_size``: the
    VSA block, 64, 128 or 256 tokens."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, H, S, D] ([B, S, H, D] with bshd)")
    if bshd:
        B, Sq, H, D = q.shape
        Skv = k.shape[1]
    else:
        B, H, Sq, D = q.shape
        Skv = k.shape[2]
    problem = dense_problem(B, H, Sq, Skv, D, topk, block_size, bshd)
    out, idx, num = _VideoSparseAttn.apply(q, k, v, gate, problem, None)
    return (out, idx, num) if return_routing else out


def video_sparse_attn_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, meta: VarlenMeta,
                             gate: Optional[torch.Tensor] = None, return_routing: bool = False):
    """Differentiable VSA over block-padded packed sequences (``q``
    ``[H, bs*Nq, D]``, ``k``/``v`` ``[H, bs*Nkv, D]``, ``meta`` from
    ``vsa_build_metadata`` with the same block size): the forward of
    ``vsa_forward_varlen`` and, through autograd, the gradients of q, k, v and
    the gate (``[H, bs*Nq]`` or ``[H, bs*Nq, D]``) from vsa_backward, padding
    slots 0.  With ``return_routing`` also returns ``q2k_idx`` (global KV
    block numbers) and ``q2k_num``."""
    if q.dim() != 3:
        raise ValueError("packed q must be [H, slots, D]")
    H, _, D = q.shape
    if meta.device_arrays is None:
        meta.to(q.device)
    problem = meta.problem(H, D)
    out, idx, num = _VideoSparseAttn.apply(q, k, v, gate, problem, meta)
    return (out, idx, num) if return_routing else out


# ---------------------------------------------------------------------------
# whole forward
# ---------------------------------------------------------------------------

def vsa_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, topk: int,
                gate: Optional[torch.Tensor] = None, *, block_size: int = BLOCK, bshd: bool = False,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                return_aux: bool = False):
    """VSA forward on dense ``[B, H, S, D]`` bf16 tensors (vsa_forward), or on
    ``[B, S, H, D]`` tensors with ``bshd`` (vsa_forward_bshd).

    ``gate``: None, ``[B, H, Sq]`` or ``[B, H, Sq, D]`` bf16 (``[B, Sq, H]`` or
    ``[B, Sq, H, D]`` with ``bshd``; any strides, e.g. a transposed view).
    ``block_size``: 64, 128 or 256.  With ``return_aux`` also returns
    ``(out_c, q2k_idx, q2k_num)``.
    """
    if q.dim() != 4:
        raise ValueError("q must be [B, H, S, D] ([B, S, H, D] with bshd)")
    if bshd:
        B, Sq, H, D = q.shape
        Skv = k.shape[1] if k.dim() == 4 else -1
    else:
        B, H, Sq, D = q.shape
        Skv = k.shape[2] if k.dim() == 4 else -1
    problem = dense_problem(B, H, Sq, Skv, D, topk, block_size, bshd)
    _check_qkv(problem, q, k, v)
    mode, st = _gate_args(gate, *_gate_shapes(problem))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, q.shape)
    if workspace is None:
        workspace = alloc_workspace(problem, q.device)
    aux = None
    if return_aux:
        cs, isz, ns = block_shapes(problem)
        aux = (torch.empty(cs, dtype=torch.float32, device=q.device),
               torch.empty(isz, dtype=torch.int32, device=q.device),
               torch.empty(ns, dtype=torch.int32, device=q.device))
    oc, idx, num = aux if aux else (None, None, None)
    fn = _abi.load().vsa_forward_bshd if bshd else _abi.load().vsa_forward
    _abi.check(fn(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), mode, st, _ptr(out), _ptr(idx), _ptr(num),
        _ptr(oc), B, H, Sq, Skv, D, block_size, topk, _ptr(workspace), workspace.numel(),
        _stream(q.device)), "vsa_forward_bshd" if bshd else "vsa_forward")
    return (out, *aux) if return_aux else out


def vsa_forward_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, topk: int,
                        gate: Optional[torch.Tensor] = None, *, block_size: int = BLOCK,
                        out: Optional[torch.Tensor] = None, return_aux: bool = False):
    """vsa_forward on dense ``[B, H, S, D]`` tensors through the entry point
    that allocates nothing (vsa_forward_noalloc): its workspace is the
    library's per-device scratch array (vsa_noalloc_scratch_bytes), shared by
    every call on that GPU.  Outputs as for ``vsa_forward`` (``out`` and the
    aux outputs are the caller's tensors)."""
    if q.dim() != 4:
        raise ValueError("q must be [B, H, S, D]")
    B, H, Sq, D = q.shape
    Skv = k.shape[2] if k.dim() == 4 else -1
    problem = dense_problem(B, H, Sq, Skv, D, topk, block_size)
    _check_qkv(problem, q, k, v)
    mode, st = _gate_args(gate, *_gate_shapes(problem))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, q.shape)
    aux = None
    if return_aux:
        cs, isz, ns = block_shapes(problem)
        aux = (torch.empty(cs, dtype=torch.float32, device=q.device),
               torch.empty(isz, dtype=torch.int32, device=q.device),
               torch.empty(ns, dtype=torch.int32, device=q.device))
    oc, idx, num = aux if aux else (None, None, None)
    _abi.check(_abi.load().vsa_forward_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), mode, st, _ptr(out), _ptr(idx), _ptr(num),
        _ptr(oc), B, H, Sq, Skv, D, block_size, topk, _stream(q.device)), "vsa_forward_noalloc")
    return (out, *aux) if return_aux else out


def vsa_noalloc_scratch_bytes() -> int:
    """Bytes of the per-device scratch array of vsa_forward_noalloc."""
    return int(_abi.load().vsa_noalloc_scratch_bytes())


def vsa_forward_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, meta: VarlenMeta,
                       gate: Optional[torch.Tensor] = None, *, out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, return_aux: bool = False):
    """VSA forward over block-padded packed sequences (vsa_forward_varlen).

    ``q`` is ``[H, bs*Nq, D]``, ``k``/``v`` ``[H, bs*Nkv, D]`` with bs the
    metadata's block size; ``meta`` from ``vsa_build_metadata(...,
    device=q.device)``.  ``gate``: None, ``[H, bs*Nq]`` or ``[H, bs*Nq, D]``.
    """
    if q.dim() != 3:
        raise ValueError("packed q must be [H, slots, D]")
    H, _, D = q.shape
    if meta.device_arrays is None:
        meta.to(q.device)
    problem = meta.problem(H, D)
    _check_qkv(problem, q, k, v)
    mode, st = _gate_args(gate, *_gate_shapes(problem))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, q.shape)
    if workspace is None:
        workspace = alloc_workspace(problem, q.device)
    aux = None
    if return_aux:
        cs, isz, ns = block_shapes(problem)
        aux = (torch.empty(cs, dtype=torch.float32, device=q.device),
               torch.empty(isz, dtype=torch.int32, device=q.device),
               torch.empty(ns, dtype=torch.int32, device=q.device))
    oc, idx, num = aux if aux else (None, None, None)
    d = meta.device_arrays
    s = meta.sizes
    _abi.check(_abi.load().vsa_forward_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), mode, st, _ptr(out), _ptr(idx), _ptr(num), _ptr(oc),
        _ptr(d["cu_blocks_q"]), _ptr(d["cu_blocks_kv"]), _ptr(d["block_sizes_q"]),
        _ptr(d["block_sizes_kv"]), _ptr(d["topk"]), s.num_seqs, s.total_q_blocks,
        s.total_kv_blocks, s.max_q_blocks, s.max_kv_blocks, s.max_topk, H, D, meta.block_size,
        _ptr(workspace), workspace.numel(), _stream(q.device)), "vsa_forward_varlen")
    return (out, *aux) if return_aux else out


# ---------------------------------------------------------------------------
# video latents: 3-D tile partition, gather / scatter, tiled forward
# ---------------------------------------------------------------------------

DEFAULT_TILE = (4, 4, 4)


def tile_partition(T: int, H: int, W: int, tile=DEFAULT_TILE) -> dict:
    """Host index arrays of the 3-D tile partition (vsa_tile_partition):
    ``tile_partition_indices``, ``reverse_tile_partition_indices``,
    ``variable_block_sizes`` and ``non_pad_index`` (CPU int64 tensors)."""
    lib = _abi.load()
    nt = ctypes.c_int32(0)
    _abi.check(lib.vsa_tile_partition(T, H, W, *tile, ctypes.byref(nt), None, None, None, None),
               "vsa_tile_partition")
    S = T * H * W
    sizes = torch.zeros(nt.value, dtype=torch.int32)
    fwd = torch.zeros(S, dtype=torch.int64)
    rev = torch.zeros(S, dtype=torch.int64)
    nonpad = torch.zeros(S, dtype=torch.int64)
    _abi.check(lib.vsa_tile_partition(T, H, W, *tile, ctypes.byref(nt), _ptr(sizes), _ptr(fwd), _ptr(rev),
                                      _ptr(nonpad)), "vsa_tile_partition")
    return dict(tile_partition_indices=fwd, reverse_tile_partition_indices=rev,
                variable_block_sizes=sizes.to(torch.int64), non_pad_index=nonpad)


def vsa_build_tile_metadata(num_videos: int, grid, topk: int, tile=DEFAULT_TILE, device=None) -> VarlenMeta:
    """Packed-layout metadata of ``num_videos`` videos of one ``grid = (T, H,
    W)``, one block per tile (vsa_build_tile_metadata)."""
    lib = _abi.load()
    T, H, W = grid
    sizes = VsaMetaSizes()
    _abi.check(lib.vsa_build_tile_metadata(num_videos, T, H, W, *tile, topk, ctypes.byref(sizes),
                                           None, None, None, None, None), "vsa_build_tile_metadata")
    n = num_videos
    cu_q = torch.zeros(n + 1, dtype=torch.int32)
    cu_kv = torch.zeros(n + 1, dtype=torch.int32)
    bs_q = torch.zeros(sizes.total_q_blocks, dtype=torch.int32)
    bs_kv = torch.zeros(sizes.total_kv_blocks, dtype=torch.int32)
    tkc = torch.zeros(n, dtype=torch.int32)
    _abi.check(lib.vsa_build_tile_metadata(num_videos, T, H, W, *tile, topk, ctypes.byref(sizes), _ptr(cu_q),
                                           _ptr(cu_kv), _ptr(bs_q), _ptr(bs_kv), _ptr(tkc)),
               "vsa_build_tile_metadata")
    S = T * H * W
    meta = VarlenMeta(sizes, [S] * n, [S] * n, cu_q, cu_kv, bs_q, bs_kv, tkc, block_size=tile_block(tile))
    return meta.to(device) if device is not None else meta


def _tile_count(grid, tile) -> int:
    return -(-grid[0] // tile[0]) * -(-grid[1] // tile[1]) * -(-grid[2] // tile[2])


def tile_block(tile) -> int:
    """Slots per tile (the VSA block size of the tiled forward): 64 for
    tiles of at most 64 tokens, else 128 or 256."""
    n = tile[0] * tile[1] * tile[2]
    return BLOCK if n <= BLOCK else (2 * BLOCK if n <= 2 * BLOCK else 4 * BLOCK)


def tile_gather(x: torch.Tensor, grid, tile=DEFAULT_TILE, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``x`` ``[B, heads, T*H*W(, E)]`` raster -> ``[heads, B * bs * n_tiles(, E)]``
    tile order with zero padding, bs = tile_block(tile) (vsa_tile_gather)."""
    T, H, W = grid
    squeeze = x.dim() == 3
    if x.dim() not in (3, 4) or x.shape[2] != T * H * W:
        raise ValueError(f"x must be [B, heads, {T * H * W}(, E)], got {tuple(x.shape)}")
    _need(x, "x", torch.bfloat16)
    B, Hh = x.shape[0], x.shape[1]
    E = 1 if squeeze else x.shape[3]
    slots = tile_block(tile) * _tile_count(grid, tile)
    shape = (Hh, B * slots) if squeeze else (Hh, B * slots, E)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, shape)
    _abi.check(_abi.load().vsa_tile_gather(_ptr(x), _ptr(out), B, Hh, T, H, W, *tile, E, _stream(x.device)),
               "vsa_tile_gather")
    return out


def tile_scatter(y: torch.Tensor, grid, batch: int, tile=DEFAULT_TILE,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Inverse of ``tile_gather``: ``[heads, B * bs * n_tiles(, E)]`` ->
    ``[B, heads, T*H*W(, E)]`` (vsa_tile_scatter)."""
    T, H, W = grid
    slots = tile_block(tile) * _tile_count(grid, tile)
    squeeze = y.dim() == 2
    if y.dim() not in (2, 3) or y.shape[1] != batch * slots:
        raise ValueError(f"y must be [heads, {batch * slots}(, E)], got {tuple(y.shape)}")
    _need(y, "y", torch.bfloat16)
    Hh = y.shape[0]
    E = 1 if squeeze else y.shape[2]
    shape = (batch, Hh, T * H * W) if squeeze else (batch, Hh, T * H * W, E)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=y.device)
    _need(out, "out", torch.bfloat16, shape)
    _abi.check(_abi.load().vsa_tile_scatter(_ptr(y), _ptr(out), batch, Hh, T, H, W, *tile, E, _stream(y.device)),
               "vsa_tile_scatter")
    return out


# Device copies of the tile metadata, one per (videos, grid, top-k, tile,
# device): built and copied to the device on the first forward of a shape,
# so later forwards of that shape issue no host -> device copy.
_TILE_META_CACHE: dict = {}


def _cached_tile_metadata(num_videos: int, grid, topk: int, tile, device) -> VarlenMeta:
    key = (int(num_videos), tuple(int(x) for x in grid), int(topk), tuple(int(x) for x in tile),
           torch.device(device))
    meta = _TILE_META_CACHE.get(key)
    if meta is None:
        meta = vsa_build_tile_metadata(num_videos, grid, topk, tile, device=device)
        _TILE_META_CACHE[key] = meta
    return meta


def vsa_forward_video(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, grid, topk: int,
                      gate: Optional[torch.Tensor] = None, tile=DEFAULT_TILE, *, return_aux: bool = False):
    """VSA forward of ``B`` videos of one ``grid = (T, H, W)`` given in raster
    order, ``q``/``k``/``v`` ``[B, heads, T*H*W, D]``: the tokens are gathered
    into tile order, the forward runs with one block per tile
    (vsa_forward_varlen with vsa_build_tile_metadata) and the output is
    scattered back to raster order.  ``gate``: None, ``[B, heads, T*H*W]`` or
    ``[B, heads, T*H*W, D]`` (contiguous).  With ``return_aux`` also returns
    ``(out_c, q2k_idx, q2k_num)`` in the packed tile layout."""
    if q.dim() != 4:
        raise ValueError("q must be [B, heads, T*H*W, D]")
    B, Hh, S, D = q.shape
    for name, t in (("k", k), ("v", v)):
        if tuple(t.shape) != tuple(q.shape):
            raise ValueError(f"{name} must have the shape of q {tuple(q.shape)}, got {tuple(t.shape)}")
    meta = _cached_tile_metadata(B, grid, topk, tile, q.device)
    gq, gk, gv = (tile_gather(t, grid, tile) for t in (q, k, v))
    gg = None if gate is None else tile_gather(gate, grid, tile)
    res = vsa_forward_varlen(gq, gk, gv, meta, gg, return_aux=return_aux)
    out_t = res[0] if return_aux else res
    out = tile_scatter(out_t, grid, B, tile)
    return (out, *res[1:]) if return_aux else out
