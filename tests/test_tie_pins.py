"""CPU pins of the routing's tie reading and of the tie-free margin check.

* ``oracle.tie_free`` on hand-built margin arrays (values at, below and above
  the threshold, infinite margins, an empty row set);
* the oracle's routing on inputs with exact score ties (integer-valued
  blocks that repeat, all-zero blocks) equals the integer rule of
  ``tests/tie_rule.py``, which ranks exact integer keys with no floating
  point, for dense problems (VSA blocks of 64, 128 and 256 tokens, a
  32-token last block) and packed ones;
* those inputs do put ties at the top-k boundary (so the GPU tie test
  exercises the rule), and the integer rule itself rejects a planted
  higher-index tie break.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from tests import tie_rule as TR
from tests.numerics import f64


def test_tie_free_hand_built():
    # threshold = 1e-12 * max|dot| = 2e-12 here
    ok, mn, bad = oracle.tie_free(np.array([math.inf, 3e-12, 0.5]), 2.0)
    assert ok and mn == 3e-12 and bad == 0
    ok, mn, bad = oracle.tie_free(np.array([2e-12, 0.1, 1e-13]), 2.0)
    assert not ok and mn == 1e-13 and bad == 2  # at and below the threshold both count
    ok, mn, bad = oracle.tie_free(np.array([0.0, 1.0]), 1.0)
    assert not ok and mn == 0.0 and bad == 1
    ok, mn, bad = oracle.tie_free(np.array([math.inf, math.inf]), 5.0)
    assert ok and mn == math.inf and bad == 0
    ok, mn, bad = oracle.tie_free(np.zeros((0,)), 1.0)
    assert ok and bad == 0
    # the relative threshold scales with the largest dot and with rel
    assert oracle.tie_free(np.array([1e-9]), 1e3)[0] is False
    assert oracle.tie_free(np.array([1e-9]), 1e3, rel=1e-13)[0] is True
    # multi-dimensional margin arrays are taken as a whole
    g = np.array([[0.5, math.inf], [1e-3, 0.0]])
    ok, mn, bad = oracle.tie_free(g, 1.0)
    assert not ok and mn == 0.0 and bad == 1


def _dense_rule(inp, block):
    B, H, Sq, Skv, D = inp.shape
    qs, ks = oracle.block_sizes(Sq, block), oracle.block_sizes(Skv, block)
    out = np.zeros((B, H, len(qs), min(inp.topk, len(ks))), dtype=np.int64)
    keys = {}
    for b in range(B):
        for h in range(H):
            out[b, h], keys[b, h] = TR.expected_routing(
                f64(inp.q[b, h]), f64(inp.k[b, h]), qs, ks, inp.topk, block,
                synth.TIED_Q_UNIT, synth.TIED_K_UNIT)
    return out, keys


DENSE_CASES = [
    # (B, H, Sq, Skv, D, topk, block)
    (1, 3, 64 * 20, 64 * 20, 64, 5, 64),
    (2, 2, 64 * 12 + 32, 64 * 17 + 32, 64, 4, 64),   # 32-token last blocks
    (1, 2, 128 * 9, 128 * 11, 64, 3, 128),
    (1, 2, 256 * 5, 256 * 7 + 128, 64, 2, 256),
]


@pytest.mark.parametrize("B,H,Sq,Skv,D,topk,block", DENSE_CASES)
def test_oracle_routing_on_ties_equals_integer_rule(B, H, Sq, Skv, D, topk, block):
    inp = synth.tied_dense_inputs(B, H, Sq, D, topk, seed=500 + Sq, S_kv=Skv, block=block)
    ref = oracle.vsa_forward(f64(inp.q), f64(inp.k), f64(inp.v), topk, blocks=[], block=block)
    want, keys = _dense_rule(inp, block)
    assert np.array_equal(ref["q2k_idx"], want)
    decided = 0
    for (b, h), kb in keys.items():
        for i in range(kb.shape[0]):
            TR.check_selection(ref["q2k_idx"][b, h, i], list(kb[i]))
            decided += TR.rule_decides(list(kb[i]), ref["q2k_idx"].shape[-1])
    # the inputs really put ties at the boundary in many rows
    assert decided >= 0.3 * sum(kb.shape[0] for kb in keys.values()), decided


def test_oracle_varlen_routing_on_ties_equals_integer_rule():
    sq = [64 * 7, 64 * 12 + 32, 64 * 30]
    skv = [64 * 9, 64 * 12 + 32, 64 * 25]
    topk = [2, 4, 9]
    inp = synth.tied_varlen_inputs(sq, skv, 2, 64, topk, seed=77)
    ref = oracle.vsa_forward_varlen(f64(inp.q), f64(inp.k), f64(inp.v), sq, skv, topk, blocks=[])
    _, _, cu_q, cu_kv = oracle.varlen_metadata(sq, skv)
    decided = rows = 0
    for s in range(3):
        qs, ks = oracle.block_sizes(sq[s]), oracle.block_sizes(skv[s])
        for h in range(2):
            per = inp.per_seq[s]
            want, keys = TR.expected_routing(f64(per["q"][h]), f64(per["k"][h]), qs, ks, topk[s], 64,
                                             synth.TIED_Q_UNIT, synth.TIED_K_UNIT)
            kk = want.shape[1]
            got = ref["q2k_idx"][h, cu_q[s]:cu_q[s + 1]]
            assert np.array_equal(got[:, :kk], want + cu_kv[s])
            assert (got[:, kk:] == -1).all()
            for i in range(len(qs)):
                decided += TR.rule_decides(list(keys[i]), kk)
                rows += 1
    assert decided >= 0.3 * rows


def test_integer_rule_rejects_higher_index_ties():
    keys = [5, 3, 3, 3, 1]
    TR.check_selection([0, 1, 2], keys)
    with pytest.raises(AssertionError):
        TR.check_selection([0, 2, 3], keys)
    with pytest.raises(AssertionError):
        TR.check_selection([0, 1, 4], keys)  # a lower score chosen over a higher one
    with pytest.raises(AssertionError):
        TR.check_selection([1, 0, 2], keys)  # not ascending
    assert TR.rule_decides(keys, 2) and not TR.rule_decides(keys, 1)
    assert TR.count_threshold_ties(keys, 3) == 3
