"""The oracle against its pins, and the pins against planted oracle mistakes.

The mistakes are planted in the oracle, on the CPU (never in GPU code): each
variant below is a plausible slip in writing the method down, and at least one
pin must reject it.
"""
import math

import numpy as np
import torch
import pytest

import oracle.tiles as TL
import oracle.vsa_backward as BW
import oracle.vsa_oracle as O
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------

def _sparse_no_scale(q_rows, k, v, kv_sizes, idx, block=64):
    keys = np.concatenate([k[block * j: block * j + kv_sizes[j]] for j in idx])
    vals = np.concatenate([v[block * j: block * j + kv_sizes[j]] for j in idx])
    s = q_rows @ keys.T
    w = np.exp(s - s.max(axis=1, keepdims=True))
    return (w / w.sum(axis=1, keepdims=True)) @ vals


def _pool_div64(x, sizes, block=64):
    return np.stack([x[block * i: block * i + n].sum(axis=0) / block for i, n in enumerate(sizes)])


def _pool_reads_padding(x, sizes, block=64):
    return np.stack([x[block * i: block * i + block].mean(axis=0) for i, _ in enumerate(sizes)])


def _coarse_no_scale(qc, kc, vc):
    dots = qc @ kc.T
    w = np.exp(dots - dots.max(axis=1, keepdims=True))
    return dots, (w / w.sum(axis=1, keepdims=True)) @ vc


def _coarse_transposed(qc, kc, vc):
    # probabilities transposed before the value product (raises on non-square)
    dots = qc @ kc.T
    lg = dots / math.sqrt(qc.shape[1])
    w = np.exp(lg - lg.max(axis=1, keepdims=True))
    return dots, (w / w.sum(axis=1, keepdims=True)).T @ vc


def _coarse_softmax_wrong_axis(qc, kc, vc):
    dots = qc @ kc.T
    lg = dots / math.sqrt(qc.shape[1])
    w = np.exp(lg - lg.max(axis=0, keepdims=True))
    return dots, (w / w.sum(axis=0, keepdims=True)) @ vc


def _topk_high_index_ties(row, topk):
    n = row.shape[0]
    kk = min(topk, n)
    order = np.lexsort((-np.arange(n), -row))
    gap = float(row[order[kk - 1]] - row[order[kk]]) if kk < n else math.inf
    return sorted(int(j) for j in order[:kk]), gap


def _topk_unsorted(row, topk):
    n = row.shape[0]
    kk = min(topk, n)
    order = np.lexsort((np.arange(n), -row))
    gap = float(row[order[kk - 1]] - row[order[kk]]) if kk < n else math.inf
    return [int(j) for j in order[:kk]], gap


def _topk_smallest(row, topk):
    return _orig_select(-row, topk)


def _combine_gate_on_sparse(out_c_row, out_s_rows, gate_rows):
    if gate_rows is None:
        return out_c_row[None, :] + out_s_rows
    g = gate_rows[:, None] if gate_rows.ndim == 1 else gate_rows
    return out_c_row[None, :] + g * out_s_rows


def _combine_drops_coarse(out_c_row, out_s_rows, gate_rows):
    return out_s_rows + 0.0 * out_c_row[None, :]


_orig_select = O.select_topk
_orig_varlen = O.vsa_forward_varlen


def _varlen_no_rebase(*a, **kw):
    r = _orig_varlen(*a, **kw)
    cu_kv = O.varlen_metadata(a[3], a[4])[3]
    idx = r["q2k_idx"].copy()
    for s in range(len(cu_kv) - 1):
        rows = r["seq_of_block"] == s
        sub = idx[:, rows]
        sub[sub >= 0] -= cu_kv[s]
        idx[:, rows] = sub
    r["q2k_idx"] = idx
    return r


_tile_partition_ok = TL.tile_partition


def _tiles_local_order_w_slowest(T, H, W, tile=(4, 4, 4)):
    tt, th, tw = tile
    m = _tile_partition_ok(T, H, W, tile)
    fwd = []
    for bt in range(-(-T // tt)):
        for bh in range(-(-H // th)):
            for bw in range(-(-W // tw)):
                for lw in range(min(tw, W - bw * tw)):
                    for lh in range(min(th, H - bh * th)):
                        for lt in range(min(tt, T - bt * tt)):
                            fwd.append(((bt * tt + lt) * H + (bh * th + lh)) * W + (bw * tw + lw))
    m["tile_partition_indices"] = np.asarray(fwd)
    m["reverse_tile_partition_indices"] = np.argsort(fwd)
    return m


def _tiles_unpadded(T, H, W, tile=(4, 4, 4)):
    m = _tile_partition_ok(T, H, W, tile)
    m["non_pad_index"] = np.arange(len(m["non_pad_index"]))
    return m


def _tiles_reverse_is_forward(T, H, W, tile=(4, 4, 4)):
    m = _tile_partition_ok(T, H, W, tile)
    m["reverse_tile_partition_indices"] = m["tile_partition_indices"].copy()
    return m


def _tiles_64_slots(T, H, W, tile=(4, 4, 4)):
    # every tile padded to 64 slots whatever its size (overlapping slots for
    # tiles of more than 64 tokens)
    m = _tile_partition_ok(T, H, W, tile)
    sizes = m["variable_block_sizes"]
    first = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    tile_of = np.repeat(np.arange(len(sizes)), sizes)
    m["non_pad_index"] = 64 * tile_of + (np.arange(len(tile_of)) - first[tile_of])
    return m


_forward_torch_ok = BW.forward_torch
_lse_ok = BW.sparse_row_lse2


def _bw_gate_on_sparse(q, k, v, gate, idx, block=64):
    out, out_c, out_s = _forward_torch_ok(q, k, v, None, idx, block)
    if gate is None:
        return out, out_c, out_s
    g = gate[..., None] if gate.dim() == 3 else gate
    blk = torch.arange(q.shape[2]) // block
    return out_c[:, :, blk] + out_s * g, out_c, out_s


def _bw_value_detached(q, k, v, gate, idx, block=64):
    # gradient stops at v in the sparse branch (a slip in the restatement)
    return _forward_torch_ok(q, k, v.detach(), gate, idx, block)


def _lse_natural_log(q, k, idx, block=64):
    # natural log instead of base 2
    return _lse_ok(q, k, idx, block) * math.log(2.0)


def _lse_unscaled(q, k, idx, block=64):
    # scores without the 1 / sqrt(D) factor
    return _lse_ok(np.asarray(q) * math.sqrt(np.asarray(q).shape[-1]), k, idx, block)


def _lse_max_only(q, k, idx, block=64):
    # the row max of the scaled scores taken for the log-sum-exp
    q, k = np.asarray(q, dtype=np.float64), np.asarray(k, dtype=np.float64)
    B, H, Sq, D = q.shape
    qs, ks = O.block_sizes(Sq), O.block_sizes(k.shape[2])
    out = np.empty((B, H, Sq))
    for b in range(B):
        for h in range(H):
            for i, n in enumerate(qs):
                keys = np.concatenate([k[b, h, 64 * j: 64 * j + ks[j]] for j in idx[b, h, i]])
                s_ = q[b, h, 64 * i: 64 * i + n] @ keys.T / math.sqrt(D)
                out[b, h, 64 * i: 64 * i + n] = s_.max(axis=1) / math.log(2.0)
    return out


_orig_block_sizes = O.block_sizes
_orig_pool = O.pool
_orig_sparse_block = O.sparse_block


def _block_sizes_always_64(seqlen, block=64):
    # the block parameter ignored when splitting a sequence
    return _orig_block_sizes(seqlen, 64)


def _pool_stride_64(x, sizes, block=64):
    # blocks of `block` tokens averaged, but located 64 rows apart
    return _orig_pool(x, sizes, 64)


def _sparse_stride_64(q_rows, k, v, kv_sizes, idx, block=64):
    # selected KV blocks located 64 rows apart whatever the block size
    return _orig_sparse_block(q_rows, k, v, kv_sizes, idx, 64)


_orig_packed = O.forward_packed_blocks


def _packed_slots_64(q, k, v, qsz, ksz, topk, gate=None, blocks=None, block=64):
    # packed VSA blocks located 64 slots apart whatever their size; the sizes
    # are cut to 64 so that the slip runs instead of raising
    cut = lambda sz: [[min(n, 64) for n in x] for x in sz]
    return _orig_packed(q, k, v, cut(qsz), cut(ksz), topk, gate, blocks, 64)


def _bw_blocks_64(q, k, v, gate, idx, block=64):
    # the restatement ignores the VSA block size (pools and attends 64-token blocks)
    return _forward_torch_ok(q, k, v, gate, idx, 64)


MISTAKES = {
    "sparse_scale_dropped": ("sparse_block", _sparse_no_scale),
    "pool_divides_by_64": ("pool", _pool_div64),
    "pool_reads_padding": ("pool", _pool_reads_padding),
    "coarse_scale_dropped": ("coarse", _coarse_no_scale),
    "coarse_transposed_operand": ("coarse", _coarse_transposed),
    "coarse_softmax_wrong_axis": ("coarse", _coarse_softmax_wrong_axis),
    "topk_ties_to_higher_index": ("select_topk", _topk_high_index_ties),
    "topk_not_ascending": ("select_topk", _topk_unsorted),
    "topk_picks_smallest": ("select_topk", _topk_smallest),
    "combine_gate_on_sparse": ("combine", _combine_gate_on_sparse),
    "combine_drops_coarse": ("combine", _combine_drops_coarse),
    "varlen_indices_not_rebased": ("vsa_forward_varlen", _varlen_no_rebase),
    "tiles_local_order_w_slowest": ("tiles.tile_partition", _tiles_local_order_w_slowest),
    "tiles_not_padded": ("tiles.tile_partition", _tiles_unpadded),
    "tiles_reverse_is_forward": ("tiles.tile_partition", _tiles_reverse_is_forward),
    "tiles_always_64_slots": ("tiles.tile_partition", _tiles_64_slots),
    "backward_gate_on_sparse": ("backward.forward_torch", _bw_gate_on_sparse),
    "backward_value_detached": ("backward.forward_torch", _bw_value_detached),
    "lse_natural_log": ("backward.sparse_row_lse2", _lse_natural_log),
    "lse_unscaled": ("backward.sparse_row_lse2", _lse_unscaled),
    "lse_max_only": ("backward.sparse_row_lse2", _lse_max_only),
    "block_sizes_ignore_block": ("block_sizes", _block_sizes_always_64),
    "pool_blocks_64_apart": ("pool", _pool_stride_64),
    "sparse_blocks_64_apart": ("sparse_block", _sparse_stride_64),
    "backward_ignores_block_size": ("backward.forward_torch", _bw_blocks_64),
    "packed_blocks_64_slots_apart": ("forward_packed_blocks", _packed_slots_64),
}


def _some_pin_fails():
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin()
        except Exception:  # a pin that raises rejects the planted mistake
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, bad = MISTAKES[name]
    mod = O
    if attr.startswith("tiles."):
        mod, attr = TL, attr.split(".", 1)[1]
    elif attr.startswith("backward."):
        mod, attr = BW, attr.split(".", 1)[1]
    monkeypatch.setattr(mod, attr, bad)
    failed = _some_pin_fails()
    assert failed, f"no pin rejects the planted mistake {name}"
