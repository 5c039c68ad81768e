"""Checks that pin the fp64 oracle to facts outside itself.

Each ``pin_*`` function raises ``AssertionError`` when the oracle disagrees
with a closed form, a library routine, a brute-force search, or an
invariance of the method.  ``test_oracle_pins.py`` runs them on the real
oracle and, to show they have teeth, on copies of it with one plausible
mistake planted (a dropped scale, a wrong divisor, a reversed tie-break, a
transposed operand, a missing rebase, ...).

The pages print no worked numerical example, so no value here is quoted from
them; every expected value is derived by hand in the docstring next to it,
or comes from an independent routine (torch's scaled_dot_product_attention
and avg_pool1d, itertools.combinations).
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import torch

import oracle.tiles as TL
import oracle.vsa_backward as BW
import oracle.vsa_oracle as O

RNG_SEED = 20261203


def _rng(extra=0):
    return np.random.default_rng(RNG_SEED + extra)


def _sdpa(q, k, v):
    """Textbook softmax(q k^T / sqrt(D)) v via torch's fp64 CPU routine."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).numpy()


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def pin_block_sizes():
    assert O.block_sizes(256) == [64] * 4
    assert O.block_sizes(13 * 64 + 40) == [64] * 13 + [40]
    assert O.block_sizes(1) == [1]
    assert O.block_sizes(64) == [64]
    try:
        O.block_sizes(0)
    except ValueError:
        pass
    else:
        raise AssertionError("zero-length sequence must be rejected")


def pin_pool_partial_block():
    """Block 0 full with rows 0..63 (mean 31.5); block 1 partial with rows
    valued 1, 2, 3 (mean 2).  A divisor of 64 for the partial block would give
    6/64 instead of 2."""
    d = 4
    x = np.zeros((128, d))
    x[:64] = np.arange(64)[:, None]
    x[64:67] = np.array([1.0, 2.0, 3.0])[:, None]
    x[67:] = 1e9  # padding rows must never be read
    m = O.pool(x, [64, 3])
    assert np.array_equal(m[0], np.full(d, 31.5)), m[0]
    assert np.array_equal(m[1], np.full(d, 2.0)), m[1]


def pin_two_token_closed_form():
    """One partial block of 2 tokens, D = 64 (scale 1/8).

    q0 = (8 ln 3, 0, ...), k0 = e0, k1 = 0 -> logits ln 3 and 0 -> weights 3/4
    and 1/4, so out_s[0] = 0.75 v0 + 0.25 v1.  q1 = 0 -> weights 1/2, 1/2.
    With a single block the coarse softmax has one key: out_c = Vc[0] =
    (v0 + v1) / 2, and routing must pick block 0.  Gate 0.5 per token:
    out = 0.5 out_c + out_s.
    """
    D = 64
    q = np.zeros((1, 1, 2, D)); k = np.zeros((1, 1, 2, D)); v = np.zeros((1, 1, 2, D))
    q[0, 0, 0, 0] = 8.0 * math.log(3.0)
    k[0, 0, 0, 0] = 1.0
    v[0, 0, 0, 1] = 4.0
    v[0, 0, 1, 2] = 8.0
    gate = np.full((1, 1, 2), 0.5)
    r = O.vsa_forward(q, k, v, topk=3, gate=gate)
    want_s0 = np.zeros(D); want_s0[1] = 3.0; want_s0[2] = 2.0
    want_s1 = np.zeros(D); want_s1[1] = 2.0; want_s1[2] = 4.0
    want_c = np.zeros(D); want_c[1] = 2.0; want_c[2] = 4.0
    assert np.allclose(r["out_s"][0, 0, 0], want_s0, atol=1e-14, rtol=0)
    assert np.allclose(r["out_s"][0, 0, 1], want_s1, atol=1e-14, rtol=0)
    assert np.allclose(r["out_c"][0, 0, 0], want_c, atol=1e-14, rtol=0)
    assert r["q2k_idx"].tolist() == [[[[0]]]] and r["q2k_num"].tolist() == [[[1]]]
    assert np.allclose(r["out"][0, 0, 0], 0.5 * want_c + want_s0, atol=1e-14, rtol=0)
    assert np.allclose(r["out"][0, 0, 1], 0.5 * want_c + want_s1, atol=1e-14, rtol=0)


def _two_block_case(D=128):
    """Q: one full block, every row (a, 0, ...), a = sqrt(D) ln 3.  K block 0
    rows e0, K block 1 zero.  V block 0 rows all 1.0 in column 5, V block 1
    rows all 1.0 in column 9.  Coarse dots: a and 0 -> coarse weights 3/4 and
    1/4 -> out_c = 0.75 e5 + 0.25 e9.  Fine logits: ln 3 for the 64 tokens of
    block 0, 0 for the 64 of block 1 -> the same 3/4 : 1/4 split."""
    a = math.sqrt(D) * math.log(3.0)
    q = np.zeros((1, 1, 64, D)); q[..., 0] = a
    k = np.zeros((1, 1, 128, D)); k[0, 0, :64, 0] = 1.0
    v = np.zeros((1, 1, 128, D)); v[0, 0, :64, 5] = 1.0; v[0, 0, 64:, 9] = 1.0
    return q, k, v


def pin_coarse_and_routing_closed_form():
    q, k, v = _two_block_case()
    want = np.zeros(128); want[5] = 0.75; want[9] = 0.25
    r = O.vsa_forward(q, k, v, topk=2)
    assert np.allclose(r["out_c"][0, 0, 0], want, atol=1e-14, rtol=0)
    assert np.allclose(r["out_s"][0, 0], want[None, :], atol=1e-14, rtol=0)
    assert np.allclose(r["out"][0, 0], 2 * want[None, :], atol=1e-14, rtol=0)
    assert r["q2k_idx"][0, 0, 0].tolist() == [0, 1]
    r1 = O.vsa_forward(q, k, v, topk=1)
    assert r1["q2k_idx"][0, 0, 0].tolist() == [0]  # block 0 has the larger score
    e5 = np.zeros(128); e5[5] = 1.0
    assert np.allclose(r1["out_s"][0, 0], e5[None, :], atol=1e-14, rtol=0)
    assert np.allclose(r1["out_c"][0, 0, 0], want, atol=1e-14, rtol=0)  # coarse stays dense


def pin_combine_closed_form():
    """out_c row (1, 2), out_s rows (10, 20), (30, 40); gate (0.5, 2):
    out = (10.5, 21), (32, 44).  Ungated adds: (11, 22), (31, 42).  A full
    [n, D] gate equal to (0.5, 3) per column on row 0 gives (10.5, 26)."""
    oc = np.array([1.0, 2.0])
    os_ = np.array([[10.0, 20.0], [30.0, 40.0]])
    assert np.array_equal(O.combine(oc, os_, np.array([0.5, 2.0])),
                          np.array([[10.5, 21.0], [32.0, 44.0]]))
    assert np.array_equal(O.combine(oc, os_, None), np.array([[11.0, 22.0], [31.0, 42.0]]))
    assert np.array_equal(O.combine(oc, os_[:1], np.array([[0.5, 3.0]])),
                          np.array([[10.5, 26.0]]))


# ---------------------------------------------------------------------------
# routing: brute force and tie rule
# ---------------------------------------------------------------------------

def pin_topk_bruteforce():
    """For distinct scores the selected set is the unique k-subset with the
    largest score sum; checked against every subset."""
    rng = _rng(1)
    for n, k in [(4, 2), (6, 3), (8, 3), (9, 5), (7, 1), (5, 5)]:
        for _ in range(20):
            row = rng.standard_normal(n)
            best = max(itertools.combinations(range(n), k), key=lambda c: row[list(c)].sum())
            sel, gap = O.select_topk(row, k)
            assert sel == sorted(best), (row, k, sel, best)
            s = np.sort(row)[::-1]
            want_gap = s[k - 1] - s[k] if k < n else math.inf
            assert gap == want_gap


def pin_topk_ties_and_order():
    """Equal scores go to the lower block index; output is ascending; topk is
    clamped to the number of blocks; topk < 1 is an error."""
    assert O.select_topk(np.array([1.0, 3.0, 3.0, 2.0]), 2)[0] == [1, 2]
    assert O.select_topk(np.array([5.0, 5.0, 1.0]), 1)[0] == [0]
    assert O.select_topk(np.array([1.0, 2.0, 2.0, 2.0]), 2)[0] == [1, 2]
    assert O.select_topk(np.array([0.0, 9.0, 1.0, 8.0]), 2)[0] == [1, 3]
    assert O.select_topk(np.array([4.0, 1.0, 3.0]), 3)[0] == [0, 1, 2]
    assert O.select_topk(np.array([4.0, 1.0, 3.0]), 10)[0] == [0, 1, 2]
    assert O.select_topk(np.array([2.0, 2.0]), 1)[1] == 0.0
    try:
        O.select_topk(np.array([1.0]), 0)
    except ValueError:
        pass
    else:
        raise AssertionError("topk < 1 must be rejected")


def pin_selection_property(seed=3):
    """On a random batch every row's selected minimum >= unselected maximum."""
    rng = _rng(seed)
    q = rng.standard_normal((2, 2, 64 * 9 - 13, 64))
    k = rng.standard_normal((2, 2, 64 * 7 - 5, 64))
    v = rng.standard_normal(k.shape)
    r = O.vsa_forward(q, k, v, topk=3, blocks=[])
    for b, h, i in itertools.product(range(2), range(2), range(9)):
        qc = O.pool(q[b, h], O.block_sizes(q.shape[2]))
        kc = O.pool(k[b, h], O.block_sizes(k.shape[2]))
        dots = qc @ kc.T  # (check only: the ranking quantity)
        sel = r["q2k_idx"][b, h, i]
        uns = np.setdiff1d(np.arange(7), sel)
        assert dots[i, sel].min() >= dots[i, uns].max()
        assert list(sel) == sorted(sel)


# ---------------------------------------------------------------------------
# reduction to dense attention (library routine)
# ---------------------------------------------------------------------------

def pin_dense_equivalence(seed=4):
    """topk = all blocks: out_s is textbook attention over the whole sequence,
    including a ragged tail and Sq != Skv; out_c is textbook attention over
    pooled tensors, the pooling done by torch's avg_pool1d (full blocks)."""
    rng = _rng(seed)
    for (B, H, Sq, Skv, D) in [(2, 3, 256, 256, 64), (1, 2, 200, 333, 128), (1, 1, 64, 64, 128)]:
        q = rng.standard_normal((B, H, Sq, D))
        k = rng.standard_normal((B, H, Skv, D))
        v = rng.standard_normal((B, H, Skv, D))
        r = O.vsa_forward(q, k, v, topk=10 ** 6)
        assert np.allclose(r["out_s"], _sdpa(q, k, v), atol=1e-12, rtol=0)
        if Sq % 64 == 0 and Skv % 64 == 0:
            def ap(x):
                t = torch.from_numpy(x).reshape(B * H, x.shape[2], D).transpose(1, 2)
                return torch.nn.functional.avg_pool1d(t, 64).transpose(1, 2).reshape(
                    B, H, -1, D).numpy()
            assert np.allclose(r["out_c"], _sdpa(ap(q), ap(k), ap(v)), atol=1e-12, rtol=0)


def pin_single_block(seed=5):
    """S <= 64: one block, routing {0}, out_c = Vc[0] exactly (softmax over a
    single key is 1), out_s = dense attention over <= 64 tokens."""
    rng = _rng(seed)
    for S in (64, 37, 1):
        q = rng.standard_normal((1, 2, S, 64))
        k = rng.standard_normal((1, 2, S, 64))
        v = rng.standard_normal((1, 2, S, 64))
        r = O.vsa_forward(q, k, v, topk=4)
        assert r["q2k_idx"].reshape(-1).tolist() == [0, 0]
        assert np.allclose(r["out_c"][:, :, 0], v.mean(axis=2), atol=1e-15, rtol=0)
        assert np.allclose(r["out_s"], _sdpa(q, k, v), atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------
# invariances
# ---------------------------------------------------------------------------

def _rand_dense(seed, B=1, H=2, nq=6, nkv=7, D=64, tail=0):
    rng = _rng(seed)
    q = rng.standard_normal((B, H, 64 * nq - tail, D))
    k = rng.standard_normal((B, H, 64 * nkv, D))
    v = rng.standard_normal((B, H, 64 * nkv, D))
    g = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, 64 * nq - tail))))
    return q, k, v, g


def pin_permute_within_kv_block(seed=6):
    q, k, v, g = _rand_dense(seed)
    r0 = O.vsa_forward(q, k, v, 3, g)
    perm = np.concatenate([64 * j + _rng(seed + 100 + j).permutation(64) for j in range(7)])
    r1 = O.vsa_forward(q, k[:, :, perm], v[:, :, perm], 3, g)
    assert np.array_equal(r0["q2k_idx"], r1["q2k_idx"])
    assert np.allclose(r0["out"], r1["out"], atol=1e-12, rtol=0)


def pin_permute_kv_blocks(seed=7):
    q, k, v, g = _rand_dense(seed)
    bperm = _rng(seed + 1).permutation(7)  # new block j holds old block bperm[j]
    tok = np.concatenate([64 * bperm[j] + np.arange(64) for j in range(7)])
    r0 = O.vsa_forward(q, k, v, 3, g)
    r1 = O.vsa_forward(q, k[:, :, tok], v[:, :, tok], 3, g)
    inv = np.argsort(bperm)  # old block o is now at inv[o]
    mapped = np.sort(inv[r0["q2k_idx"]], axis=-1)
    assert np.array_equal(mapped, r1["q2k_idx"])
    assert np.allclose(r0["out"], r1["out"], atol=1e-12, rtol=0)


def pin_linear_in_v(seed=8):
    q, k, v, g = _rand_dense(seed, tail=17)
    v2 = _rng(seed + 1).standard_normal(v.shape)
    a = O.vsa_forward(q, k, v, 2, g)
    b = O.vsa_forward(q, k, v2, 2, g)
    c = O.vsa_forward(q, k, v + 2.0 * v2, 2, g)
    assert np.allclose(c["out"], a["out"] + 2.0 * b["out"], atol=1e-12, rtol=0)
    assert np.allclose(c["out_c"], a["out_c"] + 2.0 * b["out_c"], atol=1e-12, rtol=0)


def pin_gate_special_values(seed=9):
    q, k, v, g = _rand_dense(seed, tail=30)
    un = O.vsa_forward(q, k, v, 3, None)
    one = O.vsa_forward(q, k, v, 3, np.ones_like(g))
    zero = O.vsa_forward(q, k, v, 3, np.zeros_like(g))
    assert np.array_equal(un["out"], one["out"])
    assert np.array_equal(zero["out"], zero["out_s"])
    per_tok = O.vsa_forward(q, k, v, 3, g)
    full = O.vsa_forward(q, k, v, 3, np.repeat(g[..., None], q.shape[-1], axis=-1))
    assert np.array_equal(per_tok["out"], full["out"])


# ---------------------------------------------------------------------------
# varlen: packed equals per-sequence
# ---------------------------------------------------------------------------

def _pack(seqs, key, H, D, lens, block=64):
    n = [-(-s // block) for s in lens]
    out = np.zeros((H, block * sum(n)) + ((D,) if key != "gate" else ()))
    o = 0
    for s, x in enumerate(seqs):
        out[:, o:o + lens[s]] = x[key]
        o += block * n[s]
    return out


def pin_varlen_matches_per_sequence(seed=10):
    rng = _rng(seed)
    H, D = 3, 64
    lens_q = [5 * 64, 9 * 64, 13 * 64 + 40, 64, 1]
    lens_kv = [6 * 64, 9 * 64, 14 * 64 - 7, 64, 130]
    topk = [2, 3, 4, 1, 5]
    seqs = []
    for sq, skv in zip(lens_q, lens_kv):
        seqs.append(dict(q=rng.standard_normal((H, sq, D)), k=rng.standard_normal((H, skv, D)),
                         v=rng.standard_normal((H, skv, D)),
                         gate=1 / (1 + np.exp(-rng.standard_normal((H, sq))))))
    qp, kp, vp = (_pack(seqs, x, H, D, lens_q if x == "q" else lens_kv) for x in "qkv")
    gp = _pack(seqs, "gate", H, D, lens_q)
    r = O.vsa_forward_varlen(qp, kp, vp, lens_q, lens_kv, topk, gp)
    oq = nq_acc = nkv_acc = 0
    for s, x in enumerate(seqs):
        ref = O.vsa_forward(x["q"][None], x["k"][None], x["v"][None], topk[s], x["gate"][None])
        nq = -(-lens_q[s] // 64)
        nkv = -(-lens_kv[s] // 64)
        kk = min(topk[s], nkv)
        sl = slice(oq, oq + lens_q[s])
        assert np.array_equal(r["out"][:, sl], ref["out"][0]), s
        assert np.array_equal(r["out_c"][:, nq_acc:nq_acc + nq], ref["out_c"][0]), s
        got = r["q2k_idx"][:, nq_acc:nq_acc + nq]
        assert np.array_equal(got[..., :kk], ref["q2k_idx"][0] + nkv_acc), s
        assert (got[..., kk:] == -1).all()
        assert (r["q2k_num"][:, nq_acc:nq_acc + nq] == kk).all()
        pad = slice(oq + lens_q[s], oq + 64 * nq)
        assert (r["out"][:, pad] == 0).all() and (r["out_s"][:, pad] == 0).all()
        oq += 64 * nq
        nq_acc += nq
        nkv_acc += nkv


def pin_varlen_large_blocks_matches_per_sequence(seed=24):
    """Packed sequences with VSA blocks of 128 and 256 tokens (each block
    128 / 256 slots): the separate packed path equals the dense path run on
    each sequence alone with the same block size, bit for bit, including
    rebased indices, partial blocks and zero padding slots; a single
    sequence packed alone equals the dense forward."""
    rng = _rng(seed)
    H, D = 2, 32
    for block in (128, 256):
        lens_q = [3 * block, block + 37, 1, 2 * block - 5]
        lens_kv = [2 * block + 9, block + 37, 70, 3 * block]
        topk = [2, 1, 3, 2]
        seqs = []
        for sq, skv in zip(lens_q, lens_kv):
            seqs.append(dict(q=rng.standard_normal((H, sq, D)), k=rng.standard_normal((H, skv, D)),
                             v=rng.standard_normal((H, skv, D)),
                             gate=1 / (1 + np.exp(-rng.standard_normal((H, sq))))))
        qp, kp, vp = (_pack(seqs, x, H, D, lens_q if x == "q" else lens_kv, block) for x in "qkv")
        gp = _pack(seqs, "gate", H, D, lens_q, block)
        r = O.vsa_forward_varlen(qp, kp, vp, lens_q, lens_kv, topk, gp, block=block)
        oq = nq_acc = nkv_acc = 0
        for s, x in enumerate(seqs):
            ref = O.vsa_forward(x["q"][None], x["k"][None], x["v"][None], topk[s], x["gate"][None], block=block)
            nq, nkv = -(-lens_q[s] // block), -(-lens_kv[s] // block)
            kk = min(topk[s], nkv)
            assert np.array_equal(r["out"][:, oq:oq + lens_q[s]], ref["out"][0]), (block, s)
            assert np.array_equal(r["out_c"][:, nq_acc:nq_acc + nq], ref["out_c"][0]), (block, s)
            got = r["q2k_idx"][:, nq_acc:nq_acc + nq]
            assert np.array_equal(got[..., :kk], ref["q2k_idx"][0] + nkv_acc), (block, s)
            assert (got[..., kk:] == -1).all()
            pad = slice(oq + lens_q[s], oq + block * nq)
            assert (r["out"][:, pad] == 0).all() and (r["out_s"][:, pad] == 0).all()
            oq += block * nq
            nq_acc += nq
            nkv_acc += nkv
    q, k, v, g = _rand_dense(seed + 1, B=1, H=2, nq=9, nkv=9, tail=11)
    d = O.vsa_forward(q, k, v, 2, g, block=256)
    r = O.vsa_forward_varlen(q[0], k[0], v[0], [q.shape[2]], [k.shape[2]], [2], g[0], block=256)
    n = q.shape[2]
    assert np.array_equal(r["out"][:, :n], d["out"][0])
    assert np.array_equal(r["q2k_idx"], d["q2k_idx"][0])


def pin_single_sequence_varlen_equals_dense(seed=11):
    q, k, v, g = _rand_dense(seed, B=1, H=2, nq=5, nkv=5, tail=0)
    d = O.vsa_forward(q, k, v, 2, g)
    r = O.vsa_forward_varlen(q[0], k[0], v[0], [q.shape[2]], [k.shape[2]], [2], g[0])
    assert np.array_equal(r["out"], d["out"][0])
    assert np.array_equal(r["q2k_idx"], d["q2k_idx"][0])


# ---------------------------------------------------------------------------
# magnitude sanity (statistics of N(0,1) inputs)
# ---------------------------------------------------------------------------

def pin_magnitudes(seed=12):
    """With N(0,1) inputs and D = 128 the fine logits are ~N(0,1); the output
    of attention over n tokens then has variance E[e^{2s}] / (n E[e^s]^2) =
    e / n, n = 64 k.  Pooled tensors have variance 1/64 per entry, so the
    coarse logits are ~0 and out_c averages nKV pooled values: variance 1/S."""
    rng = _rng(seed)
    H, nb, D, topk = 4, 24, 128, 6
    S = 64 * nb
    q, k, v = (rng.standard_normal((1, H, S, D)) for _ in range(3))
    r = O.vsa_forward(q, k, v, topk, blocks=[(0, h, i) for h in range(H) for i in range(0, nb, 4)])
    os_ = r["out_s"][np.isfinite(r["out_s"])]
    rms_s = math.sqrt(np.mean(os_ ** 2))
    assert abs(rms_s / math.sqrt(math.e / (64 * topk)) - 1) < 0.15, rms_s
    rms_c = math.sqrt(np.mean(r["out_c"] ** 2))
    assert abs(rms_c * math.sqrt(S) - 1) < 0.15, rms_c


# ---------------------------------------------------------------------------
# 3-D tile partition ("[kernel] Extract VSA utility functions into
# fastvideo_kernel", Summary / Design decisions)
# ---------------------------------------------------------------------------

TILE_CASES = [((4, 4, 4), (4, 4, 4)), ((5, 6, 7), (4, 4, 4)), ((3, 9, 2), (4, 4, 4)),
              ((8, 4, 12), (4, 4, 4)), ((6, 10, 5), (2, 4, 8)), ((1, 1, 130), (1, 1, 64)),
              ((9, 1, 1), (8, 1, 1)),
              # tiles of the 128/256-token variants (blocks of 128 and 256 slots)
              ((9, 10, 11), (4, 4, 8)), ((5, 9, 17), (4, 8, 8)), ((3, 7, 7), (3, 5, 7)),
              ((1, 1, 300), (1, 1, 256))]


def _slots_per_tile(vol):
    # 64 slots up to 64 tokens, else the next power of two (128 or 256)
    return 64 * 2 ** max(0, math.ceil(math.log2(vol / 64)))


def pin_tile_partition_by_sorting():
    """Tile order from an independent construction: tile number of every
    token from its coordinates, then a stable sort by (tile, t, h, w); sizes by
    counting; padded slot = (slots per tile) * tile + rank inside the tile."""
    for (T, H, W), (tt, th, tw) in TILE_CASES:
        m = TL.tile_partition(T, H, W, (tt, th, tw))
        t, h, w = np.unravel_index(np.arange(T * H * W), (T, H, W))
        n_h, n_w = -(-H // th), -(-W // tw)
        tile_of = ((t // tt) * n_h + h // th) * n_w + w // tw
        fwd = np.lexsort((w, h, t, tile_of))
        assert np.array_equal(m["tile_partition_indices"], fwd), (T, H, W)
        sizes = np.bincount(tile_of, minlength=-(-T // tt) * n_h * n_w)
        assert np.array_equal(m["variable_block_sizes"], sizes)
        first = np.concatenate([[0], np.cumsum(sizes)[:-1]])
        tiles_in_order = tile_of[fwd]
        rank = np.arange(len(fwd)) - first[tiles_in_order]
        assert np.array_equal(m["non_pad_index"], _slots_per_tile(tt * th * tw) * tiles_in_order + rank)
        assert np.array_equal(m["reverse_tile_partition_indices"][fwd], np.arange(len(fwd)))
        assert sizes.sum() == T * H * W and sizes.max() <= tt * th * tw


def pin_tile_closed_forms():
    """Grids that are multiples of the tile: every tile is full; a 1 x 1 x N
    grid with 1 x 1 x 64 tiles is the identity order with 64-token blocks."""
    m = TL.tile_partition(8, 8, 12, (4, 4, 4))
    assert (m["variable_block_sizes"] == 64).all() and len(m["variable_block_sizes"]) == 2 * 2 * 3
    # first tile: t, h, w in 0..3, raster inside
    want0 = [(t * 8 + h) * 12 + w for t in range(4) for h in range(4) for w in range(4)]
    assert list(m["tile_partition_indices"][:64]) == want0
    m = TL.tile_partition(1, 1, 200, (1, 1, 64))
    assert np.array_equal(m["tile_partition_indices"], np.arange(200))
    assert list(m["variable_block_sizes"]) == O.block_sizes(200)
    assert np.array_equal(m["non_pad_index"], np.arange(200))
    # the same with 256-token tiles: 256-slot blocks, still the identity
    m = TL.tile_partition(1, 1, 700, (1, 1, 256))
    assert np.array_equal(m["tile_partition_indices"], np.arange(700))
    assert list(m["variable_block_sizes"]) == [256, 256, 188]
    assert np.array_equal(m["non_pad_index"], np.arange(700))
    # a full 4 x 8 x 8 grid is one tile of 256 tokens in raster order
    m = TL.tile_partition(4, 8, 8, (4, 8, 8))
    assert list(m["variable_block_sizes"]) == [256]
    assert np.array_equal(m["tile_partition_indices"], np.arange(256))


def pin_tile_gather_scatter_roundtrip(seed=13):
    rng = np.random.default_rng(seed)
    for (T, H, W), tile in TILE_CASES[:5] + TILE_CASES[7:10]:
        x = rng.standard_normal((2, T * H * W, 3))
        y = TL.tile_gather(x, (T, H, W), tile)
        m = TL.tile_partition(T, H, W, tile)
        pad = np.ones(y.shape[1], dtype=bool)
        pad[m["non_pad_index"]] = False
        assert (y[:, pad] == 0).all()
        assert np.array_equal(TL.tile_scatter(y, (T, H, W), tile), x)


def pin_video_forward_1d_equals_dense(seed=14):
    """A 1 x 1 x S grid in 1 x 1 x b tiles is the dense forward with VSA blocks
    of b tokens on the raster sequence (same blocks, same order), b = 64, 128,
    256."""
    rng = np.random.default_rng(seed)
    for b, S in ((64, 64 * 5 + 23), (128, 128 * 4 + 23), (256, 256 * 3 + 100)):
        D = 16
        q, k, v = (rng.standard_normal((2, 3, S, D)) for _ in range(3))
        gate = rng.uniform(0, 1, (2, 3, S))
        dense = O.vsa_forward(q, k, v, 3, gate, block=b)
        vid = TL.vsa_forward_video(q, k, v, (1, 1, S), 3, gate, tile=(1, 1, b))
        assert np.allclose(vid["out_raster"], dense["out"], rtol=1e-12, atol=1e-13), b
        nq = len(O.block_sizes(S, b))
        idx = vid["q2k_idx"].reshape(3, 2, nq, 3) - (np.arange(2) * nq)[None, :, None, None]
        assert np.array_equal(idx.transpose(1, 0, 2, 3), dense["q2k_idx"]), b


def pin_video_forward_tile_equivariance(seed=15):
    """Permuting the tokens inside every tile of the input permutes the output
    the same way and changes nothing else (the pool, the routing and the
    softmax over a block do not see the order of its tokens)."""
    rng = np.random.default_rng(seed)
    grid, tile = (5, 6, 7), (4, 4, 4)
    S, D = 5 * 6 * 7, 8
    q, k, v = (rng.standard_normal((1, 2, S, D)) for _ in range(3))
    m = TL.tile_partition(*grid, tile)
    fwd, sizes = m["tile_partition_indices"], m["variable_block_sizes"]
    perm = np.arange(S)  # raster index -> raster index it takes its token from
    p0 = 0
    for n in sizes:
        members = fwd[p0:p0 + n]
        perm[members] = members[rng.permutation(n)]
        p0 += n
    a = TL.vsa_forward_video(q, k, v, grid, 3, tile=tile)
    b = TL.vsa_forward_video(q[:, :, perm], k[:, :, perm], v[:, :, perm], grid, 3, tile=tile)
    assert np.array_equal(a["q2k_idx"], b["q2k_idx"])
    assert np.allclose(a["out_raster"][:, :, perm], b["out_raster"], rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# backward ("[kernel] Add varlen support for block-sparse attention", Test
# plan: backward; "[chore] release fastvideo-kernel 0.3.0": forward and
# backward of the block-sparse attention)
# ---------------------------------------------------------------------------

def _t64(x, grad=False):
    return torch.tensor(np.asarray(x, dtype=np.float64), dtype=torch.float64, requires_grad=grad)


def pin_backward_forward_matches_oracle(seed=16):
    """The differentiable restatement computes the oracle's forward."""
    rng = np.random.default_rng(seed)
    B, H, S, D = 2, 2, 64 * 3 + 21, 8
    q, k, v = (rng.standard_normal((B, H, S, D)) for _ in range(3))
    for gate in (None, rng.uniform(0, 1, (B, H, S)), rng.uniform(0, 1, (B, H, S, D))):
        ref = O.vsa_forward(q, k, v, 2, gate)
        out, out_c, out_s = BW.forward_torch(_t64(q), _t64(k), _t64(v), None if gate is None else _t64(gate),
                                             ref["q2k_idx"])
        assert np.allclose(out.detach().numpy(), ref["out"], rtol=1e-12, atol=1e-13)
        assert np.allclose(out_c.detach().numpy(), ref["out_c"], rtol=1e-12, atol=1e-13)
        assert np.allclose(out_s.detach().numpy(), ref["out_s"], rtol=1e-12, atol=1e-13)


def pin_backward_gradcheck(seed=17):
    """Gradients of the restatement against finite differences (routing fixed)."""
    rng = np.random.default_rng(seed)
    B, H, S, D = 1, 1, 64 + 6, 3
    q, k, v = (rng.standard_normal((B, H, S, D)) for _ in range(3))
    gate = rng.uniform(0.2, 0.8, (B, H, S))
    idx = O.vsa_forward(q, k, v, 1, gate)["q2k_idx"]
    w = _t64(rng.standard_normal((B, H, S, D)))
    f = lambda a, b_, c, g: (BW.forward_torch(a, b_, c, g, idx)[0] * w).sum()
    assert torch.autograd.gradcheck(f, (_t64(q, True), _t64(k, True), _t64(v, True), _t64(gate, True)),
                                    eps=1e-6, atol=1e-7, rtol=1e-5)


def pin_backward_dense_equivalence(seed=18):
    """top-k = every block: the sparse branch's gradients are those of
    dense softmax attention (torch's scaled_dot_product_attention, float64)
    and the coarse branch's those of dense attention on the block means."""
    rng = np.random.default_rng(seed)
    B, H, S, D = 1, 2, 64 * 3, 8
    q, k, v = (rng.standard_normal((B, H, S, D)) for _ in range(3))
    w = rng.standard_normal((B, H, S, D))
    wc = rng.standard_normal((B, H, 3, D))
    idx = O.vsa_forward(q, k, v, 3)["q2k_idx"]
    tq, tk, tv = _t64(q, True), _t64(k, True), _t64(v, True)
    _, out_c, out_s = BW.forward_torch(tq, tk, tv, None, idx)
    ((out_s * _t64(w)).sum() + (out_c * _t64(wc)).sum()).backward()
    rq, rk, rv = _t64(q, True), _t64(k, True), _t64(v, True)
    ref_s = torch.nn.functional.scaled_dot_product_attention(rq, rk, rv)
    pool = lambda x: torch.nn.functional.avg_pool1d(x.reshape(B * H, S, D).transpose(1, 2), 64).transpose(1, 2).reshape(B, H, 3, D)
    ref_c = torch.nn.functional.scaled_dot_product_attention(pool(rq), pool(rk), pool(rv))
    ((ref_s * _t64(w)).sum() + (ref_c * _t64(wc)).sum()).backward()
    for a, b_ in ((tq, rq), (tk, rk), (tv, rv)):
        assert np.allclose(a.grad.numpy(), b_.grad.numpy(), rtol=1e-10, atol=1e-12)


def pin_backward_large_blocks(seed=23):
    """VSA blocks of 128 tokens: the restatement reproduces the oracle's
    forward (ragged last block, token gate); its gradients match finite
    differences; with every block selected they are those of torch's dense
    attention on the tokens and on the 128-token means (avg_pool1d), and the
    row log-sum-exp is scipy's over the dense scores."""
    from scipy.special import logsumexp
    rng = np.random.default_rng(seed)
    B, H, S, D = 1, 2, 128 * 2 + 37, 8
    q, k, v = (rng.standard_normal((B, H, S, D)) for _ in range(3))
    gate = rng.uniform(0, 1, (B, H, S))
    ref = O.vsa_forward(q, k, v, 2, gate, block=128)
    out, out_c, out_s = BW.forward_torch(_t64(q), _t64(k), _t64(v), _t64(gate), ref["q2k_idx"], 128)
    assert np.allclose(out.detach().numpy(), ref["out"], rtol=1e-12, atol=1e-13)
    assert np.allclose(out_c.detach().numpy(), ref["out_c"], rtol=1e-12, atol=1e-13)

    Sg, Dg = 128 + 6, 3
    qg, kg, vg = (rng.standard_normal((1, 1, Sg, Dg)) for _ in range(3))
    gg = rng.uniform(0.2, 0.8, (1, 1, Sg))
    idx = O.vsa_forward(qg, kg, vg, 1, gg, block=128)["q2k_idx"]
    w = _t64(rng.standard_normal((1, 1, Sg, Dg)))
    f = lambda a, b_, c, g: (BW.forward_torch(a, b_, c, g, idx, 128)[0] * w).sum()
    assert torch.autograd.gradcheck(f, (_t64(qg, True), _t64(kg, True), _t64(vg, True), _t64(gg, True)),
                                    eps=1e-6, atol=1e-7, rtol=1e-5)

    S3 = 128 * 3
    q, k, v = (rng.standard_normal((B, H, S3, D)) for _ in range(3))
    w, wc = rng.standard_normal((B, H, S3, D)), rng.standard_normal((B, H, 3, D))
    idx = O.vsa_forward(q, k, v, 3, block=128)["q2k_idx"]
    tq, tk, tv = _t64(q, True), _t64(k, True), _t64(v, True)
    _, out_c, out_s = BW.forward_torch(tq, tk, tv, None, idx, 128)
    ((out_s * _t64(w)).sum() + (out_c * _t64(wc)).sum()).backward()
    rq, rk, rv = _t64(q, True), _t64(k, True), _t64(v, True)
    ref_s = torch.nn.functional.scaled_dot_product_attention(rq, rk, rv)
    pool = lambda x: torch.nn.functional.avg_pool1d(x.reshape(B * H, S3, D).transpose(1, 2), 128).transpose(1, 2).reshape(B, H, 3, D)
    ref_c = torch.nn.functional.scaled_dot_product_attention(pool(rq), pool(rk), pool(rv))
    ((ref_s * _t64(w)).sum() + (ref_c * _t64(wc)).sum()).backward()
    for a, b_ in ((tq, rq), (tk, rk), (tv, rv)):
        assert np.allclose(a.grad.numpy(), b_.grad.numpy(), rtol=1e-10, atol=1e-12)
    dense = logsumexp(np.einsum("bhsd,bhtd->bhst", q, k) / math.sqrt(D), axis=-1) / math.log(2.0)
    assert np.allclose(BW.sparse_row_lse2(q, k, idx, 128), dense, rtol=1e-13, atol=1e-12)


def pin_lse_dense_equivalence(seed=19):
    """Every block selected: the row log-sum-exp is scipy's logsumexp of the
    dense scaled scores, in base 2."""
    from scipy.special import logsumexp
    rng = np.random.default_rng(seed)
    B, H, S, D = 1, 2, 64 * 2 + 9, 16
    q, k = rng.standard_normal((B, H, S, D)), rng.standard_normal((B, H, S, D))
    idx = O.vsa_forward(q, k, k, 3)["q2k_idx"]
    ref = logsumexp(np.einsum("bhsd,bhtd->bhst", q, k) / math.sqrt(D), axis=-1) / math.log(2.0)
    assert np.allclose(BW.sparse_row_lse2(q, k, idx), ref, rtol=1e-13, atol=1e-12)


def pin_lse_reproduces_sparse_output(seed=20):
    """The probabilities exp2(s log2(e) / sqrt(D) - lse) over each row's
    selected tokens give the oracle's sparse output (top-k 2 of 4 blocks,
    ragged last block)."""
    rng = np.random.default_rng(seed)
    B, H, S, D = 1, 2, 64 * 3 + 30, 8
    q, k, v = (rng.standard_normal((B, H, S, D)) for _ in range(3))
    ref = O.vsa_forward(q, k, v, 2)
    lse = BW.sparse_row_lse2(q, k, ref["q2k_idx"])
    sizes = O.block_sizes(S)
    for b in range(B):
        for h in range(H):
            for i, n in enumerate(sizes):
                toks = np.concatenate([np.arange(64 * j, 64 * j + sizes[j]) for j in ref["q2k_idx"][b, h, i]])
                rows = slice(64 * i, 64 * i + n)
                s_ = q[b, h, rows] @ k[b, h, toks].T
                p = np.exp2(s_ * (1.0 / math.log(2.0)) / math.sqrt(D) - lse[b, h, rows][:, None])
                assert np.allclose(p.sum(axis=1), 1.0, rtol=1e-12)
                assert np.allclose(p @ v[b, h, toks], ref["out_s"][b, h, rows], rtol=1e-11, atol=1e-12)


def pin_large_blocks_dense_equivalence(seed=21):
    """VSA blocks of 128 and 256 tokens with top-k = every block: out_s is
    textbook attention over the whole sequence and out_c attention over the
    means of 128 / 256 consecutive tokens (torch's avg_pool1d)."""
    rng = _rng(seed)
    for block, (B, H, S, D) in ((128, (1, 2, 512, 32)), (256, (2, 1, 512, 16))):
        q, k, v = (rng.standard_normal((B, H, S, D)) for _ in range(3))
        r = O.vsa_forward(q, k, v, topk=10 ** 6, block=block)
        assert r["q2k_idx"].shape == (B, H, S // block, S // block)
        assert np.allclose(r["out_s"], _sdpa(q, k, v), atol=1e-12, rtol=0)

        def ap(x):
            t = torch.from_numpy(x).reshape(B * H, S, D).transpose(1, 2)
            return torch.nn.functional.avg_pool1d(t, block).transpose(1, 2).reshape(B, H, -1, D).numpy()
        assert np.allclose(r["out_c"], _sdpa(ap(q), ap(k), ap(v)), atol=1e-12, rtol=0)


def pin_large_blocks_by_duplication(seed=22):
    """A 128-token VSA block made of two copies of the same 64 tokens has the
    mean of those 64 tokens, and softmax over doubled keys equals softmax over
    the keys once: VSA with 128-token blocks on such a sequence equals VSA with
    64-token blocks on the undoubled one, token for token (routing, coarse
    output, sparse output).  The ragged last block of 20 tokens is doubled too
    (a 40-token last VSA block): every key then appears exactly twice, so the
    softmax weights are those of the undoubled sequence."""
    rng = _rng(seed)
    B, H, L, D = 1, 2, 64 * 5 + 20, 16
    base = [rng.standard_normal((B, H, L, D)) for _ in range(3)]
    sizes = O.block_sizes(L, 64)

    def double(x):  # every 64-token block (and the ragged one) twice in a row
        parts = []
        for i, n in enumerate(sizes):
            blk = x[:, :, 64 * i: 64 * i + n]
            parts += [blk, blk]
        return np.concatenate(parts, axis=2)
    q2, k2, v2 = (double(x) for x in base)
    for topk in (2, 3):
        small = O.vsa_forward(*base, topk=topk, block=64)
        big = O.vsa_forward(q2, k2, v2, topk=topk, block=128)
        assert np.array_equal(big["q2k_idx"], small["q2k_idx"])
        assert np.allclose(big["out_c"], small["out_c"], rtol=1e-12, atol=1e-13)
        out_small = double(small["out"])
        assert np.allclose(big["out"], out_small, rtol=1e-11, atol=1e-12)


ALL_PINS = [
    pin_block_sizes, pin_pool_partial_block, pin_two_token_closed_form,
    pin_coarse_and_routing_closed_form, pin_combine_closed_form, pin_topk_bruteforce,
    pin_topk_ties_and_order, pin_selection_property, pin_dense_equivalence,
    pin_single_block, pin_permute_within_kv_block, pin_permute_kv_blocks,
    pin_linear_in_v, pin_gate_special_values, pin_varlen_matches_per_sequence,
    pin_single_sequence_varlen_equals_dense, pin_magnitudes,
    pin_tile_partition_by_sorting, pin_tile_closed_forms, pin_tile_gather_scatter_roundtrip,
    pin_video_forward_1d_equals_dense, pin_video_forward_tile_equivariance,
    pin_backward_forward_matches_oracle, pin_backward_gradcheck, pin_backward_dense_equivalence,
    pin_lse_dense_equivalence, pin_lse_reproduces_sparse_output,
    pin_large_blocks_dense_equivalence, pin_large_blocks_by_duplication,
    pin_backward_large_blocks, pin_varlen_large_blocks_matches_per_sequence,
]
