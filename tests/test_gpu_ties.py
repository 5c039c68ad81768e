"""GPU routing under exact coarse-score ties.

The inputs (``synth.tied_dense_inputs`` / ``tied_varlen_inputs``) are
integer-valued and their KV blocks repeat or are all zero, so many rows have
several KV blocks with bitwise-equal scores at the top-k boundary and only
the tie reading (equal scores go to the lower block index, indices stored
ascending) makes the answer unique.  Block means and their dot products are
exact in float64 on both sides in any summation order, so the GPU's
``q2k_idx`` must equal the oracle's exactly, and it is also checked against
the integer rule of ``tests/tie_rule.py`` row by row (a valid selection, ties
at the threshold to the lowest indices).  The select kernel keeps up to 4, 16
or 64 keys per lane depending on the KV block count; the cases reach all
three.  ("[perf] avoid full-sequence materialization in VSA coarse/sparse
combine", Correctness: top-k selection unchanged.)
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_common as G
from tests import numerics as N
from tests import tie_rule as TR
from tests.numerics import f64

pytestmark = pytest.mark.gpu


def _check_rows(gpu_idx, gpu_num, keys, kk, rebase=0):
    decided = 0
    for i in range(len(keys)):
        n = int(gpu_num[i])
        assert n == kk, f"row {i}: q2k_num {n}, want {kk}"
        sel = [int(j) - rebase for j in gpu_idx[i][:n]]
        TR.check_selection(sel, list(keys[i]))
        assert all(int(j) == -1 for j in gpu_idx[i][n:]), "unused slots must hold -1"
        decided += TR.rule_decides(list(keys[i]), kk)
    return decided


DENSE = [
    # (B, H, Sq, Skv, D, topk, block, gate, n_patterns, zero_frac, bshd)
    (1, 3, 64 * 20, 64 * 20, 128, 5, 64, "token", 3, 0.2, False),        # 4 keys per lane
    (2, 2, 64 * 12 + 32, 64 * 17 + 32, 64, 4, 64, None, 3, 0.2, False),  # 32-token last blocks
    (1, 2, 64 * 6, 64 * 300, 64, 37, 64, "token", 4, 0.2, False),        # 16 keys per lane
    (1, 1, 64 * 3, 64 * 1100, 64, 200, 64, None, 5, 0.1, False),         # 64 keys per lane
    (1, 2, 64 * 16, 64 * 16, 128, 7, 64, None, 1, 0.5, False),           # two distinct scores per row
    (1, 2, 128 * 9, 128 * 11, 128, 3, 128, "token", 3, 0.2, True),       # 128-token blocks, [B,S,H,D]
    (1, 2, 256 * 5, 256 * 7 + 128, 64, 2, 256, "token", 2, 0.3, False),  # 256-token blocks
]


@pytest.mark.parametrize("B,H,Sq,Skv,D,topk,block,gate,npat,zf,bshd", DENSE)
def test_dense_ties(B, H, Sq, Skv, D, topk, block, gate, npat, zf, bshd):
    G.note(f"case dense ties B={B} H={H} Sq={Sq} Skv={Skv} D={D} topk={topk} block={block} "
           f"gate={gate} patterns={npat} zero={zf} bshd={bshd}")
    inp = synth.tied_dense_inputs(B, H, Sq, D, topk, seed=900 + Sq + Skv, gated=gate is not None,
                                  S_kv=Skv, block=block, n_patterns=npat, zero_frac=zf)
    gpu = G.run_dense_stages(inp, block_size=block, bshd=bshd)
    ref = G.oracle_dense(inp, block=block)
    G.assert_indices_equal(gpu["q2k_idx"], gpu["q2k_num"], ref)
    qs, ks = oracle.block_sizes(Sq, block), oracle.block_sizes(Skv, block)
    kk = min(topk, len(ks))
    decided = rows = 0
    gi, gn = gpu["q2k_idx"].numpy(), gpu["q2k_num"].numpy()
    for b in range(B):
        for h in range(H):
            want, keys = TR.expected_routing(f64(inp.q[b, h]), f64(inp.k[b, h]), qs, ks, topk, block,
                                             synth.TIED_Q_UNIT, synth.TIED_K_UNIT)
            assert np.array_equal(gi[b, h], want)
            decided += _check_rows(gi[b, h], gn[b, h], keys, kk)
            rows += len(qs)
    G.note(f"  rows decided by the tie rule: {decided} of {rows}")
    assert decided > 0
    N.check_out_c(f64(gpu["out_c"]), ref["out_c"])
    N.check_sparse(f64(gpu["out_s"]), ref["out_s"])
    N.check_out(f64(gpu["out"]), ref["out"])
    N.check_out(f64(gpu["out_fused"]), ref["out"], "out (fused combine)")


VARLEN = [
    # (seqlens_q, seqlens_kv, topk, H, D, block)
    ([64 * 7, 64 * 12 + 32, 64 * 30], [64 * 9, 64 * 12 + 32, 64 * 25], [2, 4, 9], 2, 128, 64),
    ([64 * 3, 64 * 5], [64 * 280, 64 * 40], [50, 6], 2, 64, 64),   # one sequence past 256 KV blocks
    ([128 * 5, 128 * 8 + 64], [128 * 6, 128 * 8 + 64], [2, 3], 2, 128, 128),
]


@pytest.mark.parametrize("sq,skv,topk,H,D,block", VARLEN)
def test_varlen_ties(sq, skv, topk, H, D, block):
    G.note(f"case varlen ties q={sq} kv={skv} topk={topk} H={H} D={D} block={block}")
    inp = synth.tied_varlen_inputs(sq, skv, H, D, topk, seed=950 + len(sq) + block, gated=True, block=block)
    gpu = G.run_varlen_stages(inp)
    ref = G.oracle_varlen(inp)
    G.assert_indices_equal(gpu["q2k_idx"], gpu["q2k_num"], ref)
    _, _, cu_q, cu_kv = oracle.varlen_metadata(sq, skv, block)
    gi, gn = gpu["q2k_idx"].numpy(), gpu["q2k_num"].numpy()
    decided = 0
    for s in range(len(sq)):
        qs, ks = oracle.block_sizes(sq[s], block), oracle.block_sizes(skv[s], block)
        kk = min(topk[s], len(ks))
        for h in range(H):
            per = inp.per_seq[s]
            want, keys = TR.expected_routing(f64(per["q"][h]), f64(per["k"][h]), qs, ks, topk[s], block,
                                             synth.TIED_Q_UNIT, synth.TIED_K_UNIT)
            rows = slice(int(cu_q[s]), int(cu_q[s + 1]))
            assert np.array_equal(gi[h, rows, :kk], want + cu_kv[s])
            decided += _check_rows(gi[h, rows], gn[h, rows], keys, kk, rebase=int(cu_kv[s]))
    G.note(f"  rows decided by the tie rule: {decided}")
    assert decided > 0
    N.check_out_c(f64(gpu["out_c"]), ref["out_c"])
    N.check_out(f64(gpu["out"]), ref["out"])
    N.check_out(f64(gpu["out_fused"]), ref["out"], "out (fused combine)")
