"""Plain CPU oracle of the VSA backward pass (gradients of the forward).

TEST INFRASTRUCTURE ONLY, like ``vsa_oracle``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` may use it.

Sources: "[kernel] Add varlen support for block-sparse attention" (Test plan:
backward correctness of the block-sparse attention against per-sequence
references) and "[chore] release fastvideo-kernel 0.3.0" (Block-sparse / VSA
attention improvements: block-sparse attention forward and backward).  The
pages give no formulas; the backward is the gradient of the forward that
``vsa_oracle`` defines, with the routing (``q2k_idx``) held fixed: the top-k
choice is piecewise constant in the inputs, so it carries no gradient.

How: the forward is written a second time with float64 PyTorch CPU ops, block
by block in the same order as ``vsa_oracle.vsa_forward`` (pool, coarse
attention, sparse attention over the selected blocks, combine), and
``torch.autograd`` differentiates it.  The routing comes from
``vsa_oracle``.  Pins (``tests/oracle_pins.py``): this forward reproduces
``vsa_oracle.vsa_forward`` and its gradients pass
``torch.autograd.gradcheck`` against finite differences; with every block
selected they are those of dense attention.  ``sparse_row_lse2`` (the
per-row log-sum-exp a training forward keeps) is pinned to scipy's
``logsumexp`` with every block selected and to the oracle's sparse output
through the probabilities it defines.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np
import torch

from . import vsa_oracle as O


def forward_torch(q, k, v, gate, idx, block: int = O.BLOCK):
    """Differentiable float64 forward over ``[B, H, S, D]`` tensors for fixed
    routing ``idx`` (``[B, H, nQ, kk]``).  ``gate``: None, ``[B, H, S]`` or
    ``[B, H, S, D]``.  Returns ``(out, out_c, out_s)``."""
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    qs, ks = O.block_sizes(Sq, block), O.block_sizes(Skv, block)
    scale = 1.0 / math.sqrt(D)
    out_rows, outc_rows, outs_rows = [], [], []
    for b in range(B):
        ob, cb, sb = [], [], []
        for h in range(H):
            qc = torch.stack([q[b, h, block * i: block * i + n].mean(0) for i, n in enumerate(qs)])
            kc = torch.stack([k[b, h, block * j: block * j + n].mean(0) for j, n in enumerate(ks)])
            vc = torch.stack([v[b, h, block * j: block * j + n].mean(0) for j, n in enumerate(ks)])
            pc = torch.softmax(qc @ kc.T * scale, dim=1)
            oc = pc @ vc
            rows, srows = [], []
            for i, n in enumerate(qs):
                sel = [int(j) for j in idx[b, h, i]]
                keys = torch.cat([k[b, h, block * j: block * j + ks[j]] for j in sel])
                vals = torch.cat([v[b, h, block * j: block * j + ks[j]] for j in sel])
                qi = q[b, h, block * i: block * i + n]
                o_s = torch.softmax(qi @ keys.T * scale, dim=1) @ vals
                if gate is None:
                    o = oc[i][None, :] + o_s
                elif gate.dim() == 3:
                    o = oc[i][None, :] * gate[b, h, block * i: block * i + n][:, None] + o_s
                else:
                    o = oc[i][None, :] * gate[b, h, block * i: block * i + n] + o_s
                rows.append(o)
                srows.append(o_s)
            ob.append(torch.cat(rows))
            sb.append(torch.cat(srows))
            cb.append(oc)
        out_rows.append(torch.stack(ob))
        outs_rows.append(torch.stack(sb))
        outc_rows.append(torch.stack(cb))
    return torch.stack(out_rows), torch.stack(outc_rows), torch.stack(outs_rows)


def sparse_row_lse2(q, k, idx, block: int = O.BLOCK) -> np.ndarray:
    """Base-2 log of the softmax denominator of every query row of the sparse
    branch: ``log2(sum_t exp(q . k_t / sqrt(D)))`` over the valid tokens of
    the row's selected KV blocks, ``[B, H, Sq]`` from ``[B, H, S, D]`` inputs
    and routing ``idx`` (``[B, H, nQ, kk]``).  A training forward keeps it so
    that the backward can recompute the probabilities as ``exp2(q . k_t
    log2(e) / sqrt(D) - lse)``."""
    q, k = np.asarray(q, dtype=np.float64), np.asarray(k, dtype=np.float64)
    B, H, Sq, D = q.shape
    qs, ks = O.block_sizes(Sq, block), O.block_sizes(k.shape[2], block)
    out = np.empty((B, H, Sq))
    for b in range(B):
        for h in range(H):
            for i, n in enumerate(qs):
                keys = np.concatenate([k[b, h, block * j: block * j + ks[j]] for j in idx[b, h, i]])
                s = q[b, h, block * i: block * i + n] @ keys.T / math.sqrt(D)
                m = s.max(axis=1, keepdims=True)
                out[b, h, block * i: block * i + n] = (m[:, 0] + np.log(np.exp(s - m).sum(axis=1))) / math.log(2.0)
    return out


def vsa_backward(q, k, v, topk: int, gate, dout, block: int = O.BLOCK) -> Dict[str, np.ndarray]:
    """Gradients of ``sum(out * dout)`` with respect to q, k, v and the gate
    (float64 numpy in, float64 numpy out), plus the forward's routing and
    outputs for reference.  ``block`` is the VSA block size (64, 128 or 256),
    as in ``vsa_oracle.vsa_forward``."""
    fwd = O.vsa_forward(q, k, v, topk, gate, block=block)
    t = lambda x: torch.tensor(np.asarray(x, dtype=np.float64), dtype=torch.float64, requires_grad=True)
    tq, tk, tv = t(q), t(k), t(v)
    tg = None if gate is None else t(gate)
    out, out_c, out_s = forward_torch(tq, tk, tv, tg, fwd["q2k_idx"], block)
    out.backward(torch.tensor(np.asarray(dout, dtype=np.float64)))
    res = dict(dq=tq.grad.numpy(), dk=tk.grad.numpy(), dv=tv.grad.numpy(),
               dgate=None if tg is None else tg.grad.numpy(),
               out=out.detach().numpy(), out_c=out_c.detach().numpy(), out_s=out_s.detach().numpy(),
               q2k_idx=fwd["q2k_idx"], q2k_num=fwd["q2k_num"], gap=fwd["gap"],
               max_abs_dot=fwd["max_abs_dot"], lse=sparse_row_lse2(q, k, fwd["q2k_idx"], block))
    return res
