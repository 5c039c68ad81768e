"""Plain, slow fp64 CPU oracle for the forward pass of video sparse attention (VSA).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it.

What it computes is the plain definition of the method, in float64, one
step at a time, in the order the pages describe:

1. cut Q, K and V into 64-token blocks; block ``i`` holds the rows
   ``[64 i, 64 i + size_i)`` of its sequence (a partial last block has
   ``size_i < 64``);
2. pool every block to the mean of its valid rows (the "block means" of the
   compression branch);
3. coarse attention: scaled dot-product softmax attention of the pooled
   queries over all pooled keys/values of the same sequence, giving one coarse
   output row per query block (kept at block resolution);
4. top-k routing: for every query block the ``min(topk, n_kv_blocks)`` KV
   blocks with the largest coarse scores (``q2k_idx``, stored ascending) and
   their count (``q2k_num``);
5. block-sparse attention: every valid query token attends, with softmax over
   the valid tokens of its query block's selected KV blocks only;
6. combine: ``out = out_c * gate + out_s`` with ``out_c`` broadcast over the
   tokens of its block (``out_c + out_s`` when there is no gate);
7. varlen: several sequences packed block-aligned into one tensor, each
   routed over its own KV blocks, indices rebased to global block offsets.

Sources (page title, section):

* "[perf] avoid full-sequence materialization in VSA coarse/sparse combine":
  Problem (the compression branch's per-block coarse output, the combine
  ``out_c * compress_attn_weight + out_s``), Change (coarse output kept at
  block resolution and broadcast over the intra-block axis), Correctness
  (top-k selection), Notes (block means).
* "[chore] release fastvideo-kernel 0.3.0": Block-sparse / VSA attention
  improvements (``block_sparse_attn_from_indices(q, k, v, q2k_idx, q2k_num,
  variable_block_sizes)``, varlen with ``cu_seqlens_q`` / ``cu_seqlens_kv``
  and mismatched Q/KV lengths).
* "[kernel] Add varlen support for block-sparse attention": Summary / How it
  works (block-aligned packing, 64 slots per block, rebasing of ``q2k_idx``
  to global block offsets, one launch), Test plan (packed equals
  per-sequence).

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):

* the pool divides by the number of valid tokens of the block;
* Q, K and V are all pooled; the coarse softmax uses the same 1/sqrt(D)
  scale as the fine attention;
* the top-k key is the raw pooled dot product ``Qc . Kc`` (a positive scale
  and the softmax keep its order); ties go to the lower block index; the
  selected indices are stored ascending; ``topk`` larger than the number of
  KV blocks is clamped; unused varlen slots hold -1;
* padded query rows of a block-padded tensor produce 0;
* the gate arrives already squashed (no sigmoid here); it is per token and
  head (``[.., S]``, broadcast over D) or full (``[.., S, D]``).

Parity pins: every function here is checked in ``tests/test_oracle_pins.py``
against closed forms, a library routine (dense softmax attention), brute
force over subsets, and invariances; see that file for the list.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 64


# ---------------------------------------------------------------------------
# Block metadata (step 1)
# ---------------------------------------------------------------------------

def block_sizes(seqlen: int, block: int = BLOCK) -> List[int]:
    """Valid-token count of each block of a sequence of ``seqlen`` tokens.

    Every block is ``block`` tokens except a partial last one ("[kernel] Add
    varlen support for block-sparse attention", Summary: each block occupies
    64 slots; review thread: per-block variable sizes).
    """
    if seqlen <= 0:
        raise ValueError("sequence length must be positive")
    n = -(-seqlen // block)
    return [block] * (n - 1) + [seqlen - block * (n - 1)]


# ---------------------------------------------------------------------------
# Stages 2-6 on one head of one sequence
# ---------------------------------------------------------------------------

def pool(x: np.ndarray, sizes: Sequence[int], block: int = BLOCK) -> np.ndarray:
    """Block means: row ``i`` is the mean of the valid rows of block ``i``.

    ``x`` is ``[slots, D]`` with block ``i`` at rows ``[block*i, block*i + sizes[i])``
    ("[perf] avoid full-sequence materialization ...", Notes: block means).
    """
    out = np.empty((len(sizes), x.shape[1]), dtype=np.float64)
    for i, n in enumerate(sizes):
        out[i] = x[block * i: block * i + n].astype(np.float64).mean(axis=0)
    return out


def coarse(qc: np.ndarray, kc: np.ndarray, vc: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Coarse attention over pooled blocks.

    Returns ``(dots, out_c)``: ``dots[i, j] = qc[i] . kc[j]`` (the raw score the
    routing ranks) and ``out_c[i] = sum_j softmax_j(dots[i] / sqrt(D)) vc[j]``,
    one row per query block ("[perf] avoid full-sequence materialization ...",
    Problem and Change: the compression branch's per-block coarse output).
    """
    d = qc.shape[1]
    dots = qc @ kc.T
    logits = dots / math.sqrt(d)
    logits = logits - logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    p = w / w.sum(axis=1, keepdims=True)
    return dots, p @ vc


def select_topk(dots_row: np.ndarray, topk: int) -> Tuple[List[int], float]:
    """Top-k routing for one query block.

    Orders the KV blocks by decreasing score, lower index first on equal
    scores, keeps the first ``min(topk, n)``, and returns them ascending,
    together with the gap between the last kept and the first dropped score
    (``inf`` when nothing is dropped).  ("[perf] avoid full-sequence
    materialization ...", Correctness: top-k selection; "[chore] release
    fastvideo-kernel 0.3.0", Block-sparse / VSA: q2k_idx / q2k_num.)
    """
    if topk < 1:
        raise ValueError("topk must be >= 1")
    n = dots_row.shape[0]
    kk = min(topk, n)
    # np.lexsort sorts by the last key first: primary -score, secondary index.
    order = np.lexsort((np.arange(n), -dots_row))
    chosen = sorted(int(j) for j in order[:kk])
    gap = float(dots_row[order[kk - 1]] - dots_row[order[kk]]) if kk < n else math.inf
    return chosen, gap


def sparse_block(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray,
                 kv_sizes: Sequence[int], idx: Sequence[int],
                 block: int = BLOCK) -> np.ndarray:
    """Attention of the valid query rows of one block over its selected KV blocks.

    Keys/values are the valid rows of the blocks listed in ``idx``; the softmax
    runs over exactly those tokens ("[chore] release fastvideo-kernel 0.3.0",
    Block-sparse / VSA: block_sparse_attn_from_indices).
    """
    d = q_rows.shape[1]
    keys = np.concatenate([k[block * j: block * j + kv_sizes[j]] for j in idx])
    vals = np.concatenate([v[block * j: block * j + kv_sizes[j]] for j in idx])
    s = (q_rows @ keys.T) / math.sqrt(d)
    s = s - s.max(axis=1, keepdims=True)
    w = np.exp(s)
    p = w / w.sum(axis=1, keepdims=True)
    return p @ vals


def combine(out_c_row: np.ndarray, out_s_rows: np.ndarray,
            gate_rows: Optional[np.ndarray]) -> np.ndarray:
    """``out_c * gate + out_s`` with the coarse row broadcast over the block's
    tokens; ``out_c + out_s`` without a gate ("[perf] avoid full-sequence
    materialization ...", Problem and Change).

    ``gate_rows`` is ``[n]`` (one value per token, broadcast over D) or ``[n, D]``.
    """
    if gate_rows is None:
        return out_c_row[None, :] + out_s_rows
    g = gate_rows[:, None] if gate_rows.ndim == 1 else gate_rows
    return out_c_row[None, :] * g + out_s_rows


# ---------------------------------------------------------------------------
# Dense batches: q [B,H,Sq,D], k/v [B,H,Skv,D]
# ---------------------------------------------------------------------------

def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def vsa_forward(q, k, v, topk: int, gate=None,
                blocks: Optional[Sequence[Tuple[int, int, int]]] = None,
                block: int = BLOCK) -> Dict[str, np.ndarray]:
    """VSA forward over a dense ``[B, H, S, D]`` batch (each batch item is one sequence).

    ``gate`` is ``None``, ``[B, H, Sq]`` or ``[B, H, Sq, D]``.  With ``blocks``
    (a list of ``(b, h, i)``) the sparse/combine stages run only for those
    query blocks and the other output rows are NaN; the coarse stage and the
    routing always run for every block.  ``block`` is the VSA block size: 64,
    or 128 / 256 ("[chore] release fastvideo-kernel 0.3.0", Block-sparse / VSA
    attention improvements: 256-token KV blocks; "[perf] avoid full-sequence
    materialization ...", Change: the 64/128/256 dispatch) - pooling, routing
    and the sparse attention all work on blocks of that many tokens.

    Returns ``out``, ``out_s`` (``[B,H,Sq,D]``), ``out_c`` (``[B,H,nQ,D]``),
    ``q2k_idx`` (``[B,H,nQ,min(topk,nKV)]``, int32, ascending), ``q2k_num``
    (``[B,H,nQ]``), ``gap`` (``[B,H,nQ]``, the routing margin in raw-dot units)
    and ``max_abs_dot`` (``[B,H]``).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    qs, ks = block_sizes(Sq, block), block_sizes(Skv, block)
    nq, nkv = len(qs), len(ks)
    kk = min(topk, nkv)
    out_c = np.empty((B, H, nq, D))
    idx = np.empty((B, H, nq, kk), dtype=np.int32)
    num = np.full((B, H, nq), kk, dtype=np.int32)
    gap = np.empty((B, H, nq))
    maxdot = np.empty((B, H))
    for b in range(B):
        for h in range(H):
            qc, kc, vc = pool(q[b, h], qs, block), pool(k[b, h], ks, block), pool(v[b, h], ks, block)
            dots, out_c[b, h] = coarse(qc, kc, vc)
            maxdot[b, h] = np.abs(dots).max()
            for i in range(nq):
                sel, gap[b, h, i] = select_topk(dots[i], topk)
                idx[b, h, i] = sel
    gate = None if gate is None else _f64(gate)
    want = ([(b, h, i) for b in range(B) for h in range(H) for i in range(nq)]
            if blocks is None else list(blocks))
    fill = 0.0 if blocks is None else np.nan
    out_s = np.full((B, H, Sq, D), fill)
    out = np.full((B, H, Sq, D), fill)
    for b, h, i in want:
        lo, n = block * i, qs[i]
        rows = sparse_block(q[b, h, lo:lo + n], k[b, h], v[b, h], ks, idx[b, h, i], block)
        out_s[b, h, lo:lo + n] = rows
        g = None if gate is None else gate[b, h, lo:lo + n]
        out[b, h, lo:lo + n] = combine(out_c[b, h, i], rows, g)
    return dict(out=out, out_s=out_s, out_c=out_c, q2k_idx=idx, q2k_num=num,
                gap=gap, max_abs_dot=maxdot)


# ---------------------------------------------------------------------------
# Varlen: block-padded packed q [H, 64*sum nQ, D], k/v [H, 64*sum nKV, D]
# ---------------------------------------------------------------------------

def varlen_metadata(seqlens_q: Sequence[int], seqlens_kv: Sequence[int], block: int = BLOCK):
    """Per-sequence block counts, cumulative block offsets and per-block sizes."""
    qsz = [block_sizes(s, block) for s in seqlens_q]
    ksz = [block_sizes(s, block) for s in seqlens_kv]
    cu_q = np.concatenate([[0], np.cumsum([len(x) for x in qsz])]).astype(np.int64)
    cu_kv = np.concatenate([[0], np.cumsum([len(x) for x in ksz])]).astype(np.int64)
    return qsz, ksz, cu_q, cu_kv


def vsa_forward_varlen(q, k, v, seqlens_q: Sequence[int], seqlens_kv: Sequence[int],
                       topk: Sequence[int], gate=None,
                       blocks: Optional[Sequence[Tuple[int, int]]] = None,
                       block: int = BLOCK) -> Dict[str, np.ndarray]:
    """VSA forward over block-padded packed sequences, in one pass over the packed arrays.

    Sequence ``s`` occupies query blocks ``[cu_q[s], cu_q[s+1])`` and KV blocks
    ``[cu_kv[s], cu_kv[s+1])``; block ``g`` of the packed tensor starts at slot
    ``64 g``.  Routing for a query block ranks only its own sequence's KV
    blocks and the stored indices are global KV block numbers
    ("[kernel] Add varlen support for block-sparse attention", How it works).

    ``gate`` is ``None``, ``[H, slots_q]`` or ``[H, slots_q, D]``.  With
    ``blocks`` (a list of ``(h, global_q_block)``) only those blocks get sparse
    outputs; others are NaN.  Padded query slots hold 0 in ``out``/``out_s``.

    Returns ``out``, ``out_s`` (``[H, slots_q, D]``), ``out_c``
    (``[H, nQ_total, D]``), ``q2k_idx`` (``[H, nQ_total, max_k]`` int32, -1 past
    ``q2k_num``), ``q2k_num``, ``gap``, ``max_abs_dot`` (``[H, num_seqs]``).
    With ``block`` = 128 or 256 every VSA block occupies that many slots
    (reading of the 256-token variable-block-size variants of "[chore]
    release fastvideo-kernel 0.3.0", Block-sparse / VSA attention
    improvements, with the packing of "[kernel] Add varlen support ...").
    """
    qsz, ksz, _, _ = varlen_metadata(seqlens_q, seqlens_kv, block)
    return forward_packed_blocks(q, k, v, qsz, ksz, topk, gate, blocks, block)


def forward_packed_blocks(q, k, v, qsz: Sequence[Sequence[int]], ksz: Sequence[Sequence[int]],
                          topk: Sequence[int], gate=None,
                          blocks: Optional[Sequence[Tuple[int, int]]] = None,
                          block: int = BLOCK) -> Dict[str, np.ndarray]:
    """The packed forward of ``vsa_forward_varlen`` for arbitrary per-block
    valid-token counts: sequence ``s`` has query blocks of ``qsz[s]`` valid
    tokens and KV blocks of ``ksz[s]`` valid tokens, each block at the start
    of its own 64 slots (the layout the pages' ``variable_block_sizes``
    describe; a partial block need not be the last one).  ``block``: slots
    per block, the VSA block size."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    H, _, D = q.shape
    cu_q = np.concatenate([[0], np.cumsum([len(x) for x in qsz])]).astype(np.int64)
    cu_kv = np.concatenate([[0], np.cumsum([len(x) for x in ksz])]).astype(np.int64)
    ns = len(qsz)
    nq_tot = int(cu_q[-1])
    kk = [min(topk[s], len(ksz[s])) for s in range(ns)]
    max_k = max(kk)
    out_c = np.empty((H, nq_tot, D))
    idx = np.full((H, nq_tot, max_k), -1, dtype=np.int32)
    num = np.empty((H, nq_tot), dtype=np.int32)
    gap = np.empty((H, nq_tot))
    maxdot = np.empty((H, ns))
    seq_of = np.empty(nq_tot, dtype=np.int64)
    for s in range(ns):
        q0, k0 = block * cu_q[s], block * cu_kv[s]
        qspan, kspan = block * len(qsz[s]), block * len(ksz[s])
        seq_of[cu_q[s]:cu_q[s + 1]] = s
        for h in range(H):
            qc = pool(q[h, q0:q0 + qspan], qsz[s], block)
            kc = pool(k[h, k0:k0 + kspan], ksz[s], block)
            vc = pool(v[h, k0:k0 + kspan], ksz[s], block)
            dots, oc = coarse(qc, kc, vc)
            maxdot[h, s] = np.abs(dots).max()
            for i in range(len(qsz[s])):
                g = cu_q[s] + i
                out_c[h, g] = oc[i]
                sel, gap[h, g] = select_topk(dots[i], topk[s])
                idx[h, g, :kk[s]] = np.asarray(sel) + cu_kv[s]
                num[h, g] = kk[s]
    gate = None if gate is None else _f64(gate)
    # global per-block sizes, indexed by global block number
    qsz_g = [n for x in qsz for n in x]
    ksz_g = [n for x in ksz for n in x]
    want = ([(h, g) for h in range(H) for g in range(nq_tot)] if blocks is None
            else list(blocks))
    out_s = np.zeros_like(q) if blocks is None else np.full(q.shape, np.nan)
    out = np.zeros_like(q) if blocks is None else np.full(q.shape, np.nan)
    for h, g in want:
        lo, n = block * g, qsz_g[g]
        sel = idx[h, g, :num[h, g]]
        rows = sparse_block(q[h, lo:lo + n], k[h], v[h], ksz_g, sel, block)
        out_s[h, lo:lo + block] = 0.0
        out[h, lo:lo + block] = 0.0
        out_s[h, lo:lo + n] = rows
        gr = None if gate is None else gate[h, lo:lo + n]
        out[h, lo:lo + n] = combine(out_c[h, g], rows, gr)
    return dict(out=out, out_s=out_s, out_c=out_c, q2k_idx=idx, q2k_num=num,
                gap=gap, max_abs_dot=maxdot, seq_of_block=seq_of)


def tie_free(gap: np.ndarray, max_abs_dot: float, rel: float = 1e-12) -> Tuple[bool, float, int]:
    """Whether every routing decision has a margin above ``rel * max|dot|``.

    Returns ``(ok, min_gap, n_rows_at_or_below_threshold)``.  On tie-free
    inputs the selected set does not depend on the order in which a dot
    product is summed, so exact index parity is a meaningful requirement.
    """
    tau = rel * float(max_abs_dot)
    finite = gap[np.isfinite(gap)]
    if finite.size == 0:
        return True, math.inf, 0
    bad = int((finite <= tau).sum())
    return bad == 0, float(finite.min()), bad
