"""Seeded synthetic Q/K/V/gate tensors for video sparse attention workloads.

Recipe (one CPU ``torch.Generator`` per workload, seeded once):

* draw order is Q, K, V, then gate logits;
* every tensor is drawn as float32 N(0, 1) with ``torch.randn`` and rounded to
  bfloat16 (round-to-nearest-even, torch's ``.to(torch.bfloat16)``);
* the gate is ``sigmoid(logits)`` evaluated in float32, then rounded to bf16,
  so the gate handed to the method is already squashed into (0, 1);
* varlen workloads draw each sequence in order (its Q, K, V, gate) and place
  it at its block-aligned offset in zero-filled packed tensors: sequence ``s``
  starts at slot ``64 * (sum of block counts of sequences before s)``; a
  sequence's partial last block occupies a full 64-slot block whose tail
  stays zero.

Dense tensors are laid out ``[B, H, S, D]``; packed ones ``[H, slots, D]``
(gates ``[B, H, S]`` and ``[H, slots]``).  The sizes follow the workloads the
pages measure and test: the H3-like combine shape of "[perf] avoid
full-sequence materialization in VSA coarse/sparse combine" (Performance:
56 heads, head dim 128, 15488 tokens, block 64) and the varlen cases listed
under Test plan in "[kernel] Add varlen support for block-sparse attention".
The real activations those pages used are not available; N(0, 1) stands in.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

BLOCK = 64


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a bf16 (or fp32) CPU tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


@dataclass
class DenseInputs:
    q: torch.Tensor  # [B,H,Sq,D] bf16
    k: torch.Tensor  # [B,H,Skv,D] bf16
    v: torch.Tensor  # [B,H,Skv,D] bf16
    gate: Optional[torch.Tensor]  # [B,H,Sq] bf16 or None
    topk: int
    name: str = ""

    @property
    def shape(self):
        B, H, Sq, D = self.q.shape
        return B, H, Sq, self.k.shape[2], D


@dataclass
class VarlenInputs:
    q: torch.Tensor  # [H, block*sum(nQ), D] bf16, block-padded, zero padding
    k: torch.Tensor  # [H, block*sum(nKV), D]
    v: torch.Tensor
    gate: Optional[torch.Tensor]  # [H, block*sum(nQ)] or None
    seqlens_q: List[int]
    seqlens_kv: List[int]
    topk: List[int]  # requested per-sequence top-k (before any clamping)
    name: str = ""
    per_seq: List[Dict[str, torch.Tensor]] = field(default_factory=list)
    block: int = BLOCK  # slots per block (the VSA block size)

    @property
    def heads(self) -> int:
        return self.q.shape[0]

    @property
    def head_dim(self) -> int:
        return self.q.shape[2]


def _bf16_randn(gen: torch.Generator, shape) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)


def _bf16_gate(gen: torch.Generator, shape) -> torch.Tensor:
    logits = torch.randn(*shape, generator=gen, dtype=torch.float32)
    return torch.sigmoid(logits).to(torch.bfloat16)


def dense_inputs(B: int, H: int, S: int, D: int, topk: int, seed: int,
                 gated: bool = False, S_kv: Optional[int] = None,
                 name: str = "") -> DenseInputs:
    S_kv = S if S_kv is None else S_kv
    gen = torch.Generator().manual_seed(seed)
    q = _bf16_randn(gen, (B, H, S, D))
    k = _bf16_randn(gen, (B, H, S_kv, D))
    v = _bf16_randn(gen, (B, H, S_kv, D))
    gate = _bf16_gate(gen, (B, H, S)) if gated else None
    return DenseInputs(q, k, v, gate, topk, name)


def varlen_inputs(seqlens_q: List[int], seqlens_kv: Optional[List[int]], H: int,
                  D: int, topk: List[int], seed: int, gated: bool = False,
                  name: str = "", block: int = BLOCK) -> VarlenInputs:
    seqlens_kv = list(seqlens_q) if seqlens_kv is None else list(seqlens_kv)
    assert len(seqlens_q) == len(seqlens_kv) == len(topk)
    nq = [_ceil_div(s, block) for s in seqlens_q]
    nkv = [_ceil_div(s, block) for s in seqlens_kv]
    q = torch.zeros(H, block * sum(nq), D, dtype=torch.bfloat16)
    k = torch.zeros(H, block * sum(nkv), D, dtype=torch.bfloat16)
    v = torch.zeros_like(k)
    gate = torch.zeros(H, block * sum(nq), dtype=torch.bfloat16) if gated else None
    gen = torch.Generator().manual_seed(seed)
    per_seq = []
    oq = okv = 0
    for s, (sq, skv) in enumerate(zip(seqlens_q, seqlens_kv)):
        qs = _bf16_randn(gen, (H, sq, D))
        ks = _bf16_randn(gen, (H, skv, D))
        vs = _bf16_randn(gen, (H, skv, D))
        gs = _bf16_gate(gen, (H, sq)) if gated else None
        q[:, oq:oq + sq] = qs
        k[:, okv:okv + skv] = ks
        v[:, okv:okv + skv] = vs
        if gated:
            gate[:, oq:oq + sq] = gs
        per_seq.append({"q": qs, "k": ks, "v": vs, "gate": gs})
        oq += block * nq[s]
        okv += block * nkv[s]
    return VarlenInputs(q, k, v, gate, list(seqlens_q), seqlens_kv, list(topk),
                        name, per_seq, block)


def output_grad(shape, seed: int) -> torch.Tensor:
    """Seeded output gradient for backward workloads: N(0, 1) in float32 from
    its own generator, rounded to bf16."""
    gen = torch.Generator().manual_seed(seed)
    return _bf16_randn(gen, shape)


def full_gate(shape, seed: int) -> torch.Tensor:
    """Seeded gate with one value per (token, head, d): sigmoid of N(0, 1)
    logits, rounded to bf16 (the per-token gate's recipe, one more axis)."""
    gen = torch.Generator().manual_seed(seed)
    return _bf16_gate(gen, shape)


# ---------------------------------------------------------------------------
# Named workloads.  Seeds are 1000 + the workload's number.
# ---------------------------------------------------------------------------

def _frac_topk(n_kv_blocks: int, frac: float) -> int:
    return int(math.ceil(frac * n_kv_blocks - 1e-9))


_VARLEN_MANY_Q_BLOCKS = [32 + 16 * i for i in range(8)]  # 32, 48, ..., 144

WORKLOADS = {
    # 1: tiny, oracle in well under a second
    "tiny": dict(kind="dense", B=1, H=1, S=256, D=64, topk=2, gated=False, seed=1001),
    # 2: top-k equal to every block, i.e. dense attention
    "dense_equiv": dict(kind="dense", B=2, H=4, S=1024, D=128, topk=16, gated=False,
                        seed=1002),
    # 3: three packed sequences of 5, 9 and 14 blocks, the last ending in a
    #    40-token partial block; top-k = ceil(0.25 * KV blocks)
    "varlen_small": dict(kind="varlen", H=16, D=128, gated=False, seed=1003, topk_frac=0.25,
                         seqlens_q=[5 * 64, 9 * 64, 13 * 64 + 40],
                         seqlens_kv=[5 * 64, 9 * 64, 13 * 64 + 40],
                         topk=[_frac_topk(n, 0.25) for n in (5, 9, 14)]),
    # 4: the large video-DiT shape, 242 blocks, top-k = ceil(0.20 * 242) = 49, gated
    "large": dict(kind="dense", B=1, H=56, S=15488, D=128, topk=_frac_topk(242, 0.20),
                  gated=True, seed=1004),
    # the shape of the pages' listed benchmark command (batch 1, 16 heads,
    # head_dim 128, 49152 query tokens, top-64 of 768 blocks), ungated
    "pages_bench_49k": dict(kind="dense", B=1, H=16, S=49152, D=128, topk=64, gated=False, seed=1006),
    # 5: eight packed sequences, Q blocks 32..144 step 16, KV = Q + 8 blocks,
    #    top-k = ceil(0.20 * KV blocks), gated
    "varlen_many": dict(kind="varlen", H=24, D=128, gated=True, seed=1005, topk_frac=0.20,
                        seqlens_q=[64 * n for n in _VARLEN_MANY_Q_BLOCKS],
                        seqlens_kv=[64 * (n + 8) for n in _VARLEN_MANY_Q_BLOCKS],
                        topk=[_frac_topk(n + 8, 0.20) for n in _VARLEN_MANY_Q_BLOCKS]),
}


def workload(name: str, heads: Optional[int] = None, block: int = BLOCK):
    """Build a named workload; ``heads`` optionally overrides H (same seed/recipe).
    ``block`` (packed workloads): the same sequences in VSA blocks of 128 or
    256 slots, the per-sequence top-k the same fraction of the VSA blocks."""
    cfg = dict(WORKLOADS[name])
    if heads is not None:
        cfg["H"] = heads
    if cfg["kind"] == "dense":
        if block != BLOCK:
            raise ValueError("dense workloads take the block size at the problem, not here")
        return dense_inputs(cfg["B"], cfg["H"], cfg["S"], cfg["D"], cfg["topk"],
                            cfg["seed"], cfg["gated"], name=name)
    topk = cfg["topk"]
    if block != BLOCK:
        topk = [_frac_topk(_ceil_div(s, block), cfg["topk_frac"]) for s in cfg["seqlens_kv"]]
    return varlen_inputs(cfg["seqlens_q"], cfg["seqlens_kv"], cfg["H"], cfg["D"],
                         topk, cfg["seed"], cfg["gated"], name=name, block=block)


# ---------------------------------------------------------------------------
# Inputs with exact ties among the block-level scores.
#
# Every value is a small integer (uniform in {-2, ..., 2}) times a power of
# two (1/4 for queries, 1 for keys, 1/8 for values), which bf16 holds
# exactly.  KV blocks (VSA blocks of ``block`` tokens) are copies of a few
# seeded integer patterns, and some are all zero, so that many KV blocks of a
# sequence have bitwise-equal contents: every query block then sees exactly
# equal scores for them, and a top-k boundary inside such a group has several
# correct answers unless a tie rule decides.  With whole blocks (or partial
# blocks of a power-of-two size) the block means are multiples of a power of
# two and every dot product of means is exact in float64 in any summation
# order.  Only layout and random draws happen here.
# ---------------------------------------------------------------------------

TIED_Q_UNIT, TIED_K_UNIT, TIED_V_UNIT = 0.25, 1.0, 0.125


def _int_values(gen: torch.Generator, shape, unit: float = 1.0) -> torch.Tensor:
    return (torch.randint(-2, 3, tuple(shape), generator=gen).to(torch.float32) * unit).to(torch.bfloat16)


def _tied_kv(gen: torch.Generator, H: int, S_kv: int, D: int, block: int, n_patterns: int,
             zero_frac: float) -> torch.Tensor:
    """[H, S_kv, D]: VSA block j of head h is pattern[h, c(h, j)] or zero."""
    nb = _ceil_div(S_kv, block)
    pats = _int_values(gen, (H, n_patterns, block, D), TIED_K_UNIT)
    choice = torch.randint(0, n_patterns, (H, nb), generator=gen)
    zero = torch.rand(H, nb, generator=gen) < zero_frac
    out = torch.zeros(H, nb * block, D, dtype=torch.bfloat16)
    for h in range(H):
        for j in range(nb):
            if not bool(zero[h, j]):
                out[h, j * block:(j + 1) * block] = pats[h, int(choice[h, j])]
    return out[:, :S_kv].contiguous()


def tied_dense_inputs(B: int, H: int, S: int, D: int, topk: int, seed: int, gated: bool = False,
                      S_kv: Optional[int] = None, block: int = BLOCK, n_patterns: int = 3,
                      zero_frac: float = 0.2, name: str = "tied") -> DenseInputs:
    """Dense ``[B, H, S, D]`` inputs whose KV blocks repeat (see above).  Keys
    and values share the block pattern choice, so equal key blocks also carry
    equal values."""
    S_kv = S if S_kv is None else S_kv
    gen = torch.Generator().manual_seed(seed)
    q = _int_values(gen, (B, H, S, D), TIED_Q_UNIT)
    k = torch.stack([_tied_kv(gen, H, S_kv, D, block, n_patterns, zero_frac) for _ in range(B)])
    v = _int_values(gen, (B, H, S_kv, D), TIED_V_UNIT)
    gate = _bf16_gate(gen, (B, H, S)) if gated else None
    return DenseInputs(q, k, v, gate, topk, name)


def tied_varlen_inputs(seqlens_q: List[int], seqlens_kv: Optional[List[int]], H: int, D: int,
                       topk: List[int], seed: int, gated: bool = False, block: int = BLOCK,
                       n_patterns: int = 3, zero_frac: float = 0.2, name: str = "tied_varlen") -> VarlenInputs:
    """Packed inputs (block-aligned, zero padding) whose sequences' KV blocks
    repeat as in ``tied_dense_inputs``."""
    seqlens_kv = list(seqlens_q) if seqlens_kv is None else list(seqlens_kv)
    nq = [_ceil_div(s, block) for s in seqlens_q]
    nkv = [_ceil_div(s, block) for s in seqlens_kv]
    q = torch.zeros(H, block * sum(nq), D, dtype=torch.bfloat16)
    k = torch.zeros(H, block * sum(nkv), D, dtype=torch.bfloat16)
    v = torch.zeros_like(k)
    gate = torch.zeros(H, block * sum(nq), dtype=torch.bfloat16) if gated else None
    gen = torch.Generator().manual_seed(seed)
    per_seq = []
    oq = okv = 0
    for s, (sq, skv) in enumerate(zip(seqlens_q, seqlens_kv)):
        qs = _int_values(gen, (H, sq, D), TIED_Q_UNIT)
        ks = _tied_kv(gen, H, skv, D, block, n_patterns, zero_frac)
        vs = _int_values(gen, (H, skv, D), TIED_V_UNIT)
        gs = _bf16_gate(gen, (H, sq)) if gated else None
        q[:, oq:oq + sq] = qs
        k[:, okv:okv + skv] = ks
        v[:, okv:okv + skv] = vs
        if gated:
            gate[:, oq:oq + sq] = gs
        per_seq.append({"q": qs, "k": ks, "v": vs, "gate": gs})
        oq += block * nq[s]
        okv += block * nkv[s]
    return VarlenInputs(q, k, v, gate, list(seqlens_q), seqlens_kv, list(topk), name, per_seq, block)
