"""Exact routing rule on integer-valued inputs (test code, not the oracle).

For inputs whose values are small multiples of a power of two (the tied
workloads of ``synth``), block sums are exact integers after scaling, so the
ranking quantity of the routing, the dot product of two block means, can be
compared exactly with Python integers: within one query block's row,
``Qc[i] . Kc[j]`` orders like ``(sum_Q[i] . sum_K[j]) * (L / size_j)`` for any
common multiple ``L`` of the KV block sizes.  The expected selection is then
the first ``min(k, n)`` blocks in the order (larger score first, lower index
first on equal scores), reported ascending; this is the tie reading of the
routing ("[perf] avoid full-sequence materialization in VSA coarse/sparse
combine", Correctness: the top-k selection) written with integers, with no
floating point and no shared code with the oracle.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np


def _int_sums(x: np.ndarray, sizes: Sequence[int], block: int, unit: float) -> List[np.ndarray]:
    """Per block: the sum of its valid rows, divided by ``unit`` (exact integers)."""
    out = []
    for i, n in enumerate(sizes):
        s = x[block * i: block * i + n].sum(axis=0) / unit
        r = np.rint(s)
        assert np.array_equal(r, s), "inputs are not multiples of the unit"
        out.append([int(t) for t in r])
    return out


def expected_routing(q: np.ndarray, k: np.ndarray, q_sizes: Sequence[int], kv_sizes: Sequence[int],
                     topk: int, block: int, unit_q: float, unit_k: float) -> Tuple[np.ndarray, np.ndarray]:
    """Routing of one sequence on one head ([slots, D] float arrays holding
    exact small values): (indices [nq, min(topk, nkv)] ascending, integer
    score keys [nq, nkv])."""
    sq = _int_sums(q, q_sizes, block, unit_q)
    sk = _int_sums(k, kv_sizes, block, unit_k)
    L = 1
    for n in kv_sizes:
        L = L * n // math.gcd(L, n)
    nkv = len(kv_sizes)
    kk = min(topk, nkv)
    idx = np.zeros((len(q_sizes), kk), dtype=np.int64)
    keys = np.zeros((len(q_sizes), nkv), dtype=object)
    for i, a in enumerate(sq):
        row = [sum(x * y for x, y in zip(a, sk[j])) * (L // kv_sizes[j]) for j in range(nkv)]
        keys[i] = row
        order = sorted(range(nkv), key=lambda j: (-row[j], j))
        idx[i] = sorted(order[:kk])
    return idx, keys


def check_selection(sel: Sequence[int], row_keys: Sequence[int]) -> None:
    """``sel`` is a valid top-k of ``row_keys`` under the tie rule: every
    selected key >= every unselected key, and among keys equal to the
    smallest selected one the selected indices are the lowest ones."""
    sel = [int(j) for j in sel]
    assert sel == sorted(sel) and len(set(sel)) == len(sel), "indices not strictly ascending"
    uns = [j for j in range(len(row_keys)) if j not in set(sel)]
    if not uns:
        return
    lo = min(row_keys[j] for j in sel)
    assert lo >= max(row_keys[j] for j in uns), "an unselected block scores above a selected one"
    tied_sel = [j for j in sel if row_keys[j] == lo]
    tied_uns = [j for j in uns if row_keys[j] == lo]
    if tied_uns:
        assert max(tied_sel) < min(tied_uns), "a tie at the threshold went to a higher index"


def count_threshold_ties(keys_row: Sequence[int], kk: int) -> int:
    """How many blocks share the k-th largest key (more than the number
    still to be chosen there means the tie rule decides the row)."""
    s = sorted(keys_row, reverse=True)
    if kk >= len(s):
        return 0
    t = s[kk - 1]
    return sum(1 for x in keys_row if x == t)


def rule_decides(keys_row: Sequence[int], kk: int) -> bool:
    """True when the k-th and (k+1)-th largest keys are equal."""
    s = sorted(keys_row, reverse=True)
    return kk < len(s) and s[kk - 1] == s[kk]
