"""CPU tests of libvsa's host side: exported symbols, metadata, workspace sizing
and every validation error.  No kernel is launched: every call here fails
validation before any HIP call (fake device addresses are never touched)."""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import oracle
from video_sparse_attention_amd import _abi
from video_sparse_attention_amd._abi import VsaMetaSizes, VsaProblem

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vsa.h")


@pytest.fixture(scope="module")
def lib():
    return _abi.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vsa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("vsa_build_metadata", "vsa_workspace_size", "vsa_forward", "vsa_forward_varlen",
              "vsa_coarse_topk", "vsa_sparse_attn_from_indices", "vsa_sparse_attn_combine", "vsa_combine",
              "vsa_status_string", "vsa_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (vsa_\w+)", out))
    assert set(declared_functions()) <= exported
    assert set(_abi.SIGNATURES) == set(declared_functions())


def test_status_strings(lib):
    for code in range(-9, 1):
        s = lib.vsa_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.vsa_status_string(-99).decode() == "unknown status"
    assert b"gfx950" in lib.vsa_version()


# ---------------------------------------------------------------------------
# metadata
# ---------------------------------------------------------------------------

def _meta(lib, sq, skv, topk, block=64):
    n = len(sq)
    arr = lambda xs: (ctypes.c_int32 * max(len(xs), 1))(*xs)
    sizes = VsaMetaSizes()
    rc = lib.vsa_build_metadata(n, arr(sq), None if skv is None else arr(skv), arr(topk), block,
                                ctypes.byref(sizes), None, None, None, None, None)
    if rc:
        return rc, sizes, None
    bufs = [(ctypes.c_int32 * (n + 1))(), (ctypes.c_int32 * (n + 1))(),
            (ctypes.c_int32 * sizes.total_q_blocks)(), (ctypes.c_int32 * sizes.total_kv_blocks)(),
            (ctypes.c_int32 * n)()]
    rc = lib.vsa_build_metadata(n, arr(sq), None if skv is None else arr(skv), arr(topk), block,
                                ctypes.byref(sizes), *bufs)
    return rc, sizes, [list(b) for b in bufs]


@pytest.mark.parametrize("block", [64, 128, 256])
@pytest.mark.parametrize("sq,skv,topk", [
    ([320, 576, 872], None, [2, 3, 4]),
    ([64 * n for n in range(32, 145, 16)], [64 * (n + 8) for n in range(32, 145, 16)],
     [8, 12, 15, 18, 21, 24, 28, 31]),
    ([1, 65, 130], [200, 1, 64], [5, 1, 1]),
])
def test_metadata_matches_oracle(lib, sq, skv, topk, block):
    rc, sizes, (cu_q, cu_kv, bs_q, bs_kv, tk) = _meta(lib, sq, skv, topk, block)
    assert rc == 0
    skv_ = sq if skv is None else skv
    qsz, ksz, ocu_q, ocu_kv = oracle.varlen_metadata(sq, skv_, block)
    assert cu_q == list(ocu_q) and cu_kv == list(ocu_kv)
    assert bs_q == [n for x in qsz for n in x] and bs_kv == [n for x in ksz for n in x]
    assert tk == [min(t, len(k)) for t, k in zip(topk, ksz)]
    assert sizes.total_q_blocks == ocu_q[-1] and sizes.total_kv_blocks == ocu_kv[-1]
    assert sizes.max_q_blocks == max(len(x) for x in qsz)
    assert sizes.max_kv_blocks == max(len(x) for x in ksz)
    assert sizes.max_topk == max(tk)
    assert sizes.q_slots == block * ocu_q[-1] and sizes.kv_slots == block * ocu_kv[-1]


def test_metadata_errors(lib):
    assert _meta(lib, [], None, [])[0] == _abi.VSA_ERR_SHAPE            # empty batch
    assert _meta(lib, [64, 0], None, [1, 1])[0] == _abi.VSA_ERR_SHAPE   # zero-length sequence
    assert _meta(lib, [64], [0], [1])[0] == _abi.VSA_ERR_SHAPE
    assert _meta(lib, [64, 64], None, [1, 0])[0] == _abi.VSA_ERR_TOPK   # topk < 1
    for bad in (32, 96, 512):
        assert _meta(lib, [64], None, [1], bad)[0] == _abi.VSA_ERR_UNSUPPORTED
    sizes = VsaMetaSizes()
    one = (ctypes.c_int32 * 1)(64)
    assert lib.vsa_build_metadata(1, None, None, one, 64, ctypes.byref(sizes),
                                  None, None, None, None, None) == _abi.VSA_ERR_NULL
    assert lib.vsa_build_metadata(1, one, None, one, 64, None, None, None, None, None, None) == _abi.VSA_ERR_NULL
    buf = (ctypes.c_int32 * 2)()
    assert lib.vsa_build_metadata(1, one, None, one, 64, ctypes.byref(sizes), buf, None, None, None,
                                  None) == _abi.VSA_ERR_NULL  # some outputs but not all
    assert lib.vsa_build_metadata(1, (ctypes.c_int32 * 1)(2 ** 31 - 1), None, one, 64, ctypes.byref(sizes),
                                  None, None, None, None, None) == _abi.VSA_ERR_SHAPE
    # 2^31 - 255 tokens fit in 64-slot blocks, not in 256-slot ones (2^31 slots)
    sz = VsaMetaSizes()
    L = (ctypes.c_int32 * 1)(2 ** 31 - 255)
    assert lib.vsa_build_metadata(1, L, None, one, 64, ctypes.byref(sz), None, None, None, None, None) == 0
    assert sz.q_slots == 2 ** 31 - 192
    assert lib.vsa_build_metadata(1, L, None, one, 256, ctypes.byref(sz), None, None, None, None,
                                  None) == _abi.VSA_ERR_SHAPE


# ---------------------------------------------------------------------------
# workspace
# ---------------------------------------------------------------------------

def dense(B=1, H=2, Sq=1000, Skv=1000, D=128, topk=3, bs=64):
    return VsaProblem(layout=0, heads=H, head_dim=D, block_size=bs, batch=B, seqlen_q=Sq,
                      seqlen_kv=Skv, topk=topk)


FAKE = 0x7f0000000000  # 256-aligned, never dereferenced


def bshd(B=1, H=2, Sq=1000, Skv=1000, D=128, topk=3, bs=64):
    return VsaProblem(layout=2, heads=H, head_dim=D, block_size=bs, batch=B, seqlen_q=Sq,
                      seqlen_kv=Skv, topk=topk)


def packed(num_seqs=2, nq=5, nkv=6, mq=3, mkv=4, mk=2, H=2, D=64, ptrs=True):
    p = [FAKE + 4096 * i for i in range(5)] if ptrs else [None] * 5
    return VsaProblem(layout=1, heads=H, head_dim=D, block_size=64, num_seqs=num_seqs,
                      total_q_blocks=nq, total_kv_blocks=nkv, max_q_blocks=mq, max_kv_blocks=mkv,
                      max_topk=mk, cu_blocks_q=p[0], cu_blocks_kv=p[1], block_sizes_q=p[2],
                      block_sizes_kv=p[3], topk_per_seq=p[4])


def packed_bs(bs):
    p = packed()
    p.block_size = bs
    return p


def test_workspace_is_block_resolution(lib):
    """The workspace never holds a full-sequence tensor: it is a bounded
    fraction of one [B,H,S,D] bf16 tensor, from block-resolution float64 pooled
    Q/K/V, the chunked block-level score matrix, the float32 coarse output and
    the routing indices."""
    sizes = []
    for S in (64 * 10, 64 * 100, 64 * 242, 64 * 4096):
        p = dense(B=1, H=56, Sq=S, Skv=S, D=128, topk=49)
        ws = lib.vsa_workspace_size(ctypes.byref(p))
        full = 56 * S * 128 * 2
        assert 0 < ws < 0.4 * full, (S, ws / full)
        sizes.append(ws)
    p = packed()
    assert lib.vsa_workspace_size(ctypes.byref(p)) > 0
    assert lib.vsa_workspace_size(ctypes.byref(dense(bs=32))) == 0


# ---------------------------------------------------------------------------
# validation errors of the compute entry points (no launch happens)
# ---------------------------------------------------------------------------

A = ctypes.c_void_p(FAKE)
B_ = ctypes.c_void_p(FAKE + (1 << 32))
C_ = ctypes.c_void_p(FAKE + (2 << 32))
O_ = ctypes.c_void_p(FAKE + (3 << 32))
W_ = ctypes.c_void_p(FAKE + (4 << 32))
G_ = ctypes.c_void_p(FAKE + (5 << 32))


def coarse(lib, p, q=A, k=B_, v=C_, oc=O_, idx=G_, num=G_, ws=W_, wsb=1 << 40):
    return lib.vsa_coarse_topk(ctypes.byref(p), q, k, v, oc, idx, num, ws, wsb, None)


def sparse(lib, p, q=A, k=B_, v=C_, idx=G_, num=G_, out=O_):
    return lib.vsa_sparse_attn_from_indices(ctypes.byref(p), q, k, v, idx, num, out, None)


def comb(lib, p, oc=C_, gate=G_, mode=1, st=None, out=O_):
    return lib.vsa_combine(ctypes.byref(p), oc, gate, mode, st, out, None)


def fused(lib, p, q=A, k=B_, v=C_, idx=G_, num=G_, oc=W_, gate=G_, mode=1, st=None, out=O_):
    return lib.vsa_sparse_attn_combine(ctypes.byref(p), q, k, v, idx, num, oc, gate, mode, st, out, None)


def fwd(lib, q=A, k=B_, v=C_, gate=None, mode=0, st=None, out=O_, B=1, H=2, Sq=1000, Skv=1000,
        D=128, bs=64, topk=3, ws=W_, wsb=1 << 40):
    return lib.vsa_forward(q, k, v, gate, mode, st, out, None, None, None, B, H, Sq, Skv, D, bs,
                           topk, ws, wsb, None)


E = _abi


@pytest.mark.parametrize("call,code", [
    (lambda L: coarse(L, dense(), q=None), E.VSA_ERR_NULL),
    (lambda L: coarse(L, dense(), oc=None), E.VSA_ERR_NULL),
    (lambda L: coarse(L, dense(), ws=None), E.VSA_ERR_WORKSPACE),
    (lambda L: coarse(L, dense(), wsb=100), E.VSA_ERR_WORKSPACE),
    (lambda L: coarse(L, dense(), ws=ctypes.c_void_p(FAKE + 64)), E.VSA_ERR_ALIGN),
    (lambda L: coarse(L, dense(), k=ctypes.c_void_p(FAKE + 2)), E.VSA_ERR_ALIGN),
    (lambda L: coarse(L, dense(bs=96)), E.VSA_ERR_UNSUPPORTED),
    (lambda L: coarse(L, dense(bs=512)), E.VSA_ERR_UNSUPPORTED),
    (lambda L: coarse(L, packed_bs(96)), E.VSA_ERR_UNSUPPORTED),
    (lambda L: coarse(L, packed_bs(128), wsb=100), E.VSA_ERR_WORKSPACE),
    (lambda L: coarse(L, dense(bs=128, Skv=128 * 4097)), E.VSA_ERR_UNSUPPORTED),
    (lambda L: train_fwd(L, dense(bs=128), lse=None), E.VSA_ERR_NULL),
    (lambda L: train_fwd(L, bshd(), out_s=O_), E.VSA_ERR_ALIAS),
    (lambda L: bwd(L, dense(bs=256), wsb=4096), E.VSA_ERR_WORKSPACE),
    (lambda L: bwd(L, bshd(bs=128), dk=DO_), E.VSA_ERR_ALIAS),
    (lambda L: bwd(L, packed_bs(32)), E.VSA_ERR_UNSUPPORTED),
    (lambda L: bwd(L, packed_bs(256), wsb=4096), E.VSA_ERR_WORKSPACE),
    (lambda L: L.vsa_forward_bshd(A, B_, C_, None, 0, None, O_, None, None, None, 1, 2, 1000, 1000, 128, 32, 3, W_,
                                  1 << 40, None), E.VSA_ERR_UNSUPPORTED),
    (lambda L: L.vsa_forward_bshd(A, B_, C_, None, 0, None, A, None, None, None, 1, 2, 1000, 1000, 128, 128, 3, W_,
                                  1 << 40, None), E.VSA_ERR_ALIAS),
    (lambda L: L.vsa_forward_bshd(A, B_, C_, G_, 1, None, O_, None, None, None, 1, 2, 1000, 1000, 128, 256, 3, W_,
                                  10, None), E.VSA_ERR_WORKSPACE),
    (lambda L: coarse(L, dense(D=96)), E.VSA_ERR_UNSUPPORTED),
    (lambda L: coarse(L, dense(topk=0)), E.VSA_ERR_TOPK),
    (lambda L: coarse(L, dense(B=0)), E.VSA_ERR_SHAPE),
    (lambda L: coarse(L, dense(H=0)), E.VSA_ERR_SHAPE),
    (lambda L: coarse(L, dense(Sq=0)), E.VSA_ERR_SHAPE),
    (lambda L: coarse(L, dense(Skv=0)), E.VSA_ERR_SHAPE),
    (lambda L: coarse(L, dense(Skv=64 * 4097)), E.VSA_ERR_UNSUPPORTED),
    (lambda L: coarse(L, packed(num_seqs=0)), E.VSA_ERR_SHAPE),
    (lambda L: coarse(L, packed(ptrs=False)), E.VSA_ERR_NULL),
    (lambda L: coarse(L, packed(nq=1, num_seqs=2)), E.VSA_ERR_SHAPE),
    (lambda L: coarse(L, packed(mq=9)), E.VSA_ERR_SHAPE),
    (lambda L: coarse(L, packed(mk=0)), E.VSA_ERR_TOPK),
    (lambda L: sparse(L, dense(), idx=None), E.VSA_ERR_NULL),
    (lambda L: sparse(L, dense(), out=ctypes.c_void_p(FAKE + 1000 * 128)), E.VSA_ERR_ALIAS),
    (lambda L: sparse(L, dense(), out=ctypes.c_void_p(FAKE + (1 << 32) + 4096)), E.VSA_ERR_ALIAS),
    (lambda L: sparse(L, dense(), out=ctypes.c_void_p(FAKE + (3 << 32) + 8)), E.VSA_ERR_ALIGN),
    (lambda L: comb(L, dense(), mode=3), E.VSA_ERR_GATE),
    (lambda L: comb(L, dense(), gate=None), E.VSA_ERR_NULL),
    (lambda L: comb(L, dense(), st=(ctypes.c_int64 * 3)(-1, 1, 1)), E.VSA_ERR_GATE),
    (lambda L: comb(L, dense(), st=(ctypes.c_int64 * 3)(2000, 0, 1)), E.VSA_ERR_GATE),
    (lambda L: comb(L, dense(), mode=2, st=(ctypes.c_int64 * 3)(8, 8, 12)), E.VSA_ERR_ALIGN),
    (lambda L: comb(L, dense(), gate=ctypes.c_void_p(FAKE + (5 << 32) + 1)), E.VSA_ERR_ALIGN),
    (lambda L: comb(L, dense(), gate=ctypes.c_void_p(FAKE + (3 << 32) + 64)), E.VSA_ERR_ALIAS),
    (lambda L: comb(L, dense(), oc=None), E.VSA_ERR_NULL),
    (lambda L: fused(L, dense(), oc=None), E.VSA_ERR_NULL),
    (lambda L: fused(L, dense(), idx=None), E.VSA_ERR_NULL),
    (lambda L: fused(L, dense(), mode=5), E.VSA_ERR_GATE),
    (lambda L: fused(L, dense(), gate=None), E.VSA_ERR_NULL),
    (lambda L: fused(L, dense(), out=B_), E.VSA_ERR_ALIAS),
    (lambda L: fused(L, dense(), gate=ctypes.c_void_p(FAKE + (3 << 32) + 64)), E.VSA_ERR_ALIAS),
    (lambda L: fused(L, dense(), oc=ctypes.c_void_p(FAKE + (4 << 32) + 4)), E.VSA_ERR_ALIGN),
    (lambda L: fused(L, dense(), mode=2, st=(ctypes.c_int64 * 3)(8, 8, 12)), E.VSA_ERR_ALIGN),
    (lambda L: fwd(L, out=A), E.VSA_ERR_ALIAS),
    (lambda L: fwd(L, mode=1, gate=ctypes.c_void_p(FAKE + (3 << 32) + 64)), E.VSA_ERR_ALIAS),
    (lambda L: fwd(L, wsb=10), E.VSA_ERR_WORKSPACE),
    (lambda L: fwd(L, mode=1, gate=None), E.VSA_ERR_NULL),
    (lambda L: fwd(L, B=0), E.VSA_ERR_SHAPE),
    (lambda L: fwd(L, topk=-1), E.VSA_ERR_TOPK),
    (lambda L: fwd(L, bs=32), E.VSA_ERR_UNSUPPORTED),
    (lambda L: L.vsa_forward_varlen(A, B_, C_, None, 0, None, O_, None, None, None,
                                    None, G_, G_, G_, G_, 1, 1, 1, 1, 1, 1, 2, 64, 64, W_,
                                    1 << 40, None), E.VSA_ERR_NULL),
    (lambda L: L.vsa_forward_varlen(A, B_, C_, None, 0, None, O_, None, None, None,
                                    G_, G_, G_, G_, G_, 0, 1, 1, 1, 1, 1, 2, 64, 64, W_,
                                    1 << 40, None), E.VSA_ERR_SHAPE),
])
def test_validation_errors(lib, call, code):
    rc = call(lib)
    assert rc == code, (rc, lib.vsa_last_error())
    assert lib.vsa_last_error()


# ---------------------------------------------------------------------------
# training entry points: validation and workspace (no launch happens)
# ---------------------------------------------------------------------------

def _fk(n):
    return ctypes.c_void_p(FAKE + (n << 32))


# distinct fake buffers, 4 GiB apart: q, k, v, out_c, ws, gate/idx, out_s, lse, dout, dq, dk, dv, dgate,
# and a forward workspace
OS_, LSE_, DO_, DQ_, DK_, DV_, DG_, FW_ = (_fk(n) for n in range(6, 14))


def train_fwd(lib, p, q=A, k=B_, v=C_, idx=G_, num=G_, oc=W_, gate=None, mode=0, st=None, out=O_, out_s=OS_,
              lse=LSE_):
    return lib.vsa_sparse_attn_combine_train(ctypes.byref(p), q, k, v, idx, num, oc, gate, mode, st, out, out_s,
                                             lse, None)


def bwd(lib, p, q=A, k=B_, v=C_, idx=G_, num=G_, oc=O_, gate=None, mode=0, st=None, out_s=OS_, lse=LSE_, dout=DO_,
        dq=DQ_, dk=DK_, dv=DV_, dgate=DG_, ws=W_, wsb=1 << 40):
    return lib.vsa_backward(ctypes.byref(p), q, k, v, idx, num, oc, gate, mode, st, out_s, lse, dout, dq, dk, dv,
                            dgate, ws, wsb, None)


def bwdp(lib, p, fws=FW_, fwsb=1 << 40, ws=W_, wsb=1 << 40, dq=DQ_, dout=DO_):
    return lib.vsa_backward_pooled(ctypes.byref(p), A, B_, C_, G_, G_, O_, None, 0, None, OS_, LSE_, dout, dq, DK_,
                                   DV_, DG_, fws, fwsb, ws, wsb, None)


@pytest.mark.parametrize("call,code", [
    (lambda L: bwdp(L, dense(), fws=None), E.VSA_ERR_WORKSPACE),
    (lambda L: bwdp(L, dense(), fwsb=4096), E.VSA_ERR_WORKSPACE),
    (lambda L: bwdp(L, dense(), fws=ctypes.c_void_p(FAKE + (13 << 32) + 16)), E.VSA_ERR_ALIGN),
    (lambda L: bwdp(L, dense(), dq=FW_), E.VSA_ERR_ALIAS),
    (lambda L: bwdp(L, dense(), ws=FW_), E.VSA_ERR_ALIAS),
    (lambda L: bwdp(L, dense(), dout=None), E.VSA_ERR_NULL),
    (lambda L: bwdp(L, dense(), ws=None), E.VSA_ERR_WORKSPACE),
    (lambda L: bwdp(L, dense(topk=0)), E.VSA_ERR_TOPK),
    (lambda L: train_fwd(L, dense(), out_s=None), E.VSA_ERR_NULL),
    (lambda L: train_fwd(L, dense(), lse=None), E.VSA_ERR_NULL),
    (lambda L: train_fwd(L, dense(), out_s=ctypes.c_void_p(FAKE + (6 << 32) + 8)), E.VSA_ERR_ALIGN),
    (lambda L: train_fwd(L, dense(), lse=ctypes.c_void_p(FAKE + (7 << 32) + 2)), E.VSA_ERR_ALIGN),
    (lambda L: train_fwd(L, dense(), out_s=O_), E.VSA_ERR_ALIAS),
    (lambda L: train_fwd(L, dense(), out_s=A), E.VSA_ERR_ALIAS),
    (lambda L: train_fwd(L, dense(), lse=ctypes.c_void_p(FAKE + (6 << 32) + 4096)), E.VSA_ERR_ALIAS),
    (lambda L: train_fwd(L, dense(), mode=1, gate=ctypes.c_void_p(FAKE + (6 << 32) + 64)), E.VSA_ERR_ALIAS),
    (lambda L: train_fwd(L, dense(), mode=4, gate=G_), E.VSA_ERR_GATE),
    (lambda L: bwd(L, dense(), dout=None), E.VSA_ERR_NULL),
    (lambda L: bwd(L, dense(), lse=None), E.VSA_ERR_NULL),
    (lambda L: bwd(L, dense(), dk=None), E.VSA_ERR_NULL),
    (lambda L: bwd(L, dense(), mode=1, gate=G_, dgate=None), E.VSA_ERR_NULL),
    (lambda L: bwd(L, dense(), mode=2, gate=G_, dgate=ctypes.c_void_p(FAKE + (12 << 32) + 2)), E.VSA_ERR_ALIGN),
    (lambda L: bwd(L, dense(), mode=1, gate=G_, dgate=ctypes.c_void_p(FAKE + (12 << 32) + 1)), E.VSA_ERR_ALIGN),
    (lambda L: bwd(L, dense(), dq=ctypes.c_void_p(FAKE + (9 << 32) + 8)), E.VSA_ERR_ALIGN),
    (lambda L: bwd(L, dense(), lse=ctypes.c_void_p(FAKE + (7 << 32) + 1)), E.VSA_ERR_ALIGN),
    (lambda L: bwd(L, dense(), dq=A), E.VSA_ERR_ALIAS),
    (lambda L: bwd(L, dense(), dk=DO_), E.VSA_ERR_ALIAS),
    (lambda L: bwd(L, dense(), dv=ctypes.c_void_p(FAKE + (10 << 32) + 4096)), E.VSA_ERR_ALIAS),
    (lambda L: bwd(L, dense(), dq=ctypes.c_void_p(FAKE + (7 << 32) + 64)), E.VSA_ERR_ALIAS),
    (lambda L: bwd(L, dense(), mode=2, gate=G_, dgate=DQ_), E.VSA_ERR_ALIAS),
    (lambda L: bwd(L, dense(), mode=1, gate=G_, dgate=ctypes.c_void_p(FAKE + (3 << 32) + 256)), E.VSA_ERR_ALIAS),
    (lambda L: bwd(L, dense(), ws=None), E.VSA_ERR_WORKSPACE),
    (lambda L: bwd(L, dense(), wsb=4096), E.VSA_ERR_WORKSPACE),
    (lambda L: bwd(L, dense(), ws=ctypes.c_void_p(FAKE + (4 << 32) + 16)), E.VSA_ERR_ALIGN),
    (lambda L: bwd(L, dense(D=80)), E.VSA_ERR_UNSUPPORTED),
    (lambda L: bwd(L, dense(topk=0)), E.VSA_ERR_TOPK),
    (lambda L: bwd(L, packed(ptrs=False)), E.VSA_ERR_NULL),
    (lambda L: bwd(L, dense(), mode=3, gate=G_), E.VSA_ERR_GATE),
])
def test_training_validation_errors(lib, call, code):
    rc = call(lib)
    assert rc == code, (rc, lib.vsa_last_error())
    assert lib.vsa_last_error()


def test_backward_workspace(lib):
    """The backward workspace holds block-resolution float64 data, the
    block-level coarse matrices and the inverse routing: a small fraction of
    one bf16 [B,H,S,D] tensor for long sequences."""
    for S in (64 * 10, 64 * 242, 64 * 1024):
        p = dense(B=1, H=56, Sq=S, Skv=S, D=128, topk=32)
        ws = lib.vsa_backward_workspace_size(ctypes.byref(p))
        nb = S // 64
        qb = 56 * nb
        floor = 8 * qb * 128 * 7 + 2 * 8 * qb * nb + 4 * qb * 128 + 4 * qb * nb + 4 * qb
        assert floor <= ws <= floor + 13 * 256, (S, ws, floor)
    assert lib.vsa_backward_workspace_size(ctypes.byref(packed())) > 0
    assert lib.vsa_backward_workspace_size(ctypes.byref(dense(bs=32))) == 0
    # VSA blocks of 128 / 256 tokens: the coarse data per VSA block, the row
    # statistics and the inverse lists per 64-token block; BSHD the same
    for bs in (128, 256):
        S = 64 * 242
        nb64, nbv = S // 64, -(-S // bs)
        qb64, qbv = 56 * nb64, 56 * nbv
        floor = 8 * qbv * 128 * 7 + 2 * 8 * qbv * nbv + 4 * qb64 * 128 + 4 * qb64 * nb64 + 4 * qb64
        for p in (dense(B=1, H=56, Sq=S, Skv=S, D=128, topk=32, bs=bs),
                  bshd(B=1, H=56, Sq=S, Skv=S, D=128, topk=32, bs=bs)):
            ws = lib.vsa_backward_workspace_size(ctypes.byref(p))
            assert floor <= ws <= floor + 13 * 256, (bs, ws, floor)
    # packed with VSA blocks of 128 / 256 tokens: Nq = 5, Nkv = 6 VSA blocks,
    # at most 3 / 4 per sequence, H = 2, D = 64
    for bs in (64, 128, 256):
        r = bs // 64
        nq, nkv, mq, mkv, H, D = 5, 6, 3, 4, 2, 64
        floor = (8 * H * (3 * nq + 4 * nkv) * D + 2 * 8 * 2 * H * mq * mkv
                 + 4 * H * nq * r * 128 + 4 * H * nkv * r * mq * r + 4 * H * nkv * r)
        ws = lib.vsa_backward_workspace_size(ctypes.byref(packed_bs(bs)))
        assert floor <= ws <= floor + 13 * 256, (bs, ws, floor)


def test_layout_maps_on_cpu(tmp_path):
    """Compile and run the host-only check of the attention kernel's index maps
    (bijections, bounds, MFMA k-slot relabelling, LDS bank model, XCD remap)."""
    exe = tmp_path / "layout_check"
    src = os.path.join(ROOT, "tests", "cpp", "layout_check.hip")
    inc = [f"-I{os.path.join(ROOT, 'video_sparse_attention_amd', 'csrc')}",
           f"-I{os.path.join(ROOT, 'include')}"]
    subprocess.run(["hipcc", "-O1", "-std=c++17", *inc, src, "-o", str(exe)], check=True,
                   capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "layout checks passed" in r.stdout


# ---------------------------------------------------------------------------
# 3-D tile partition (host side)
# ---------------------------------------------------------------------------

TILE_CASES = [((4, 4, 4), (4, 4, 4)), ((5, 6, 7), (4, 4, 4)), ((3, 9, 2), (4, 4, 4)),
              ((8, 4, 12), (4, 4, 4)), ((6, 10, 5), (2, 4, 8)), ((1, 1, 130), (1, 1, 64)),
              ((9, 1, 1), (8, 1, 1)), ((13, 17, 11), (4, 4, 4)),
              # 128/256-token tiles (blocks of 128 and 256 slots)
              ((9, 10, 11), (4, 4, 8)), ((5, 9, 17), (4, 8, 8)), ((3, 7, 7), (3, 5, 7)),
              ((1, 1, 300), (1, 1, 256)), ((8, 16, 24), (4, 8, 8))]


@pytest.mark.parametrize("grid,tile", TILE_CASES)
def test_tile_partition_matches_oracle(lib, grid, tile):
    import oracle.tiles as TL
    import video_sparse_attention_amd as vsa
    got = vsa.tile_partition(*grid, tile)
    want = TL.tile_partition(*grid, tile)
    for key in want:
        assert np.array_equal(got[key].numpy(), want[key]), key


@pytest.mark.parametrize("grid,tile", TILE_CASES[:4] + TILE_CASES[8:])
def test_tile_metadata_is_packed_layout(lib, grid, tile):
    import oracle.tiles as TL
    import video_sparse_attention_amd as vsa
    m = vsa.vsa_build_tile_metadata(3, grid, 7, tile)
    sizes = TL.tile_partition(*grid, tile)["variable_block_sizes"]
    n = len(sizes)
    bs = TL.tile_block(tile)
    assert m.block_size == bs == vsa.tile_block(tile)
    assert m.sizes.q_slots == m.sizes.kv_slots == 3 * n * bs
    assert m.sizes.num_seqs == 3 and m.sizes.total_q_blocks == 3 * n == m.sizes.total_kv_blocks
    assert m.cu_blocks_q.tolist() == [0, n, 2 * n, 3 * n] == m.cu_blocks_kv.tolist()
    assert np.array_equal(m.block_sizes_q.numpy(), np.tile(sizes, 3))
    assert np.array_equal(m.block_sizes_kv.numpy(), np.tile(sizes, 3))
    assert m.topk.tolist() == [min(7, n)] * 3 and m.sizes.max_topk == min(7, n)


def test_noalloc_rejects_problems_past_its_scratch(lib):
    """vsa_forward_noalloc checks the problem's workspace against its fixed
    per-device scratch array before any device call (so this runs without a
    GPU); NULL tensors never get that far."""
    assert lib.vsa_noalloc_scratch_bytes() == 96 << 20
    E = _abi
    # 56 heads x 4096 blocks: far more than 96 MiB of block-level workspace
    rc = lib.vsa_forward_noalloc(None, None, None, None, 0, None, None, None, None, None,
                                 1, 56, 64 * 4096, 64 * 4096, 128, 64, 49, None)
    assert rc == E.VSA_ERR_WORKSPACE
    assert "scratch" in lib.vsa_last_error().decode()
    # invalid problems are rejected as by vsa_forward
    rc = lib.vsa_forward_noalloc(None, None, None, None, 0, None, None, None, None, None,
                                 1, 2, 64, 64, 128, 32, 1, None)
    assert rc == E.VSA_ERR_UNSUPPORTED


def test_video_forward_reuses_device_tile_metadata(lib):
    """The video forward keeps one device copy of the tile metadata per
    (videos, grid, top-k, tile, device): a second forward of the same shape
    builds and copies nothing."""
    import video_sparse_attention_amd.binding as BD
    a = BD._cached_tile_metadata(2, (5, 8, 8), 3, (4, 4, 4), "cpu")
    b = BD._cached_tile_metadata(2, (5, 8, 8), 3, (4, 4, 4), "cpu")
    c = BD._cached_tile_metadata(2, (5, 8, 8), 4, (4, 4, 4), "cpu")
    assert a is b and c is not a
    assert a.cu_blocks_q.data_ptr() == b.cu_blocks_q.data_ptr()
    assert c.topk.tolist() == [4, 4] and a.topk.tolist() == [3, 3]


def test_tile_errors(lib):
    nt = ctypes.c_int32(0)
    E = _abi
    assert lib.vsa_tile_partition(4, 4, 4, 4, 4, 4, None, None, None, None, None) == E.VSA_ERR_NULL
    assert lib.vsa_tile_partition(0, 4, 4, 4, 4, 4, ctypes.byref(nt), None, None, None, None) == E.VSA_ERR_SHAPE
    assert lib.vsa_tile_partition(4, 4, 4, 8, 8, 8, ctypes.byref(nt), None, None, None, None) == E.VSA_ERR_SHAPE
    assert lib.vsa_tile_partition(4, 4, 4, 1, 1, 257, ctypes.byref(nt), None, None, None, None) == E.VSA_ERR_SHAPE
    assert lib.vsa_tile_partition(4, 4, 4, 4, 8, 8, ctypes.byref(nt), None, None, None, None) == 0
    assert lib.vsa_tile_partition(4, 4, 4, 4, 0, 4, ctypes.byref(nt), None, None, None, None) == E.VSA_ERR_SHAPE
    sizes = _abi.VsaMetaSizes()
    assert lib.vsa_build_tile_metadata(0, 4, 4, 4, 4, 4, 4, 1, ctypes.byref(sizes),
                                       None, None, None, None, None) == E.VSA_ERR_SHAPE
    assert lib.vsa_build_tile_metadata(1, 4, 4, 4, 4, 4, 4, 0, ctypes.byref(sizes),
                                       None, None, None, None, None) == E.VSA_ERR_TOPK
    assert lib.vsa_build_tile_metadata(1, 4, 4, 4, 4, 4, 4, 1, None,
                                       None, None, None, None, None) == E.VSA_ERR_NULL
    assert lib.vsa_build_tile_metadata(1, 64, 64, 68, 4, 4, 4, 1, ctypes.byref(sizes),
                                       None, None, None, None, None) == E.VSA_ERR_UNSUPPORTED
    # gather / scatter validation (fake device addresses are never touched)
    g = lambda *a: lib.vsa_tile_gather(*a)
    assert g(None, O_, 1, 2, 4, 4, 4, 4, 4, 4, 128, None) == E.VSA_ERR_NULL
    assert g(A, ctypes.c_void_p(FAKE + 8), 1, 2, 4, 4, 4, 4, 4, 4, 128, None) in (E.VSA_ERR_ALIGN, E.VSA_ERR_ALIAS)
    assert g(A, ctypes.c_void_p(FAKE + (3 << 32) + 8), 1, 2, 4, 4, 4, 4, 4, 4, 128, None) == E.VSA_ERR_ALIGN
    assert g(A, ctypes.c_void_p(FAKE + 4096), 1, 2, 4, 4, 4, 4, 4, 4, 128, None) == E.VSA_ERR_ALIAS
    assert g(A, O_, 0, 2, 4, 4, 4, 4, 4, 4, 128, None) == E.VSA_ERR_SHAPE
    assert g(A, O_, 1, 2, 4, 4, 4, 4, 4, 4, 0, None) == E.VSA_ERR_SHAPE
    assert g(A, O_, 1, 2, 4, 4, 4, 3, 10, 9, 128, None) == E.VSA_ERR_SHAPE  # 270-token tile
    assert lib.vsa_tile_scatter(A, ctypes.c_void_p(FAKE + 2), 1, 2, 4, 4, 4, 4, 4, 4, 1, None) == E.VSA_ERR_ALIAS
    assert lib.vsa_tile_scatter(A, ctypes.c_void_p(FAKE + (3 << 32) + 1), 1, 2, 4, 4, 4, 4, 4, 4, 1,
                                None) == E.VSA_ERR_ALIGN


def test_missing_library_fails_loudly(tmp_path):
    """With no libvsa.so at the configured path, the first entry point raises
    ImportError naming the missing library: there is no CPU or PyTorch
    fallback on the product path."""
    code = (
        "import video_sparse_attention_amd as vsa\n"
        "p = vsa.dense_problem(1, 1, 64, 64, 64, 1)\n"
        "try:\n"
        "    vsa.vsa_workspace_size(p)\n"
        "except ImportError as e:\n"
        "    print('IMPORT-ERROR:', e)\n"
        "else:\n"
        "    print('NO-ERROR')\n")
    env = dict(os.environ, VSA_LIBRARY=str(tmp_path / "absent" / "libvsa.so"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "IMPORT-ERROR:" in r.stdout and "libvsa.so not found" in r.stdout, r.stdout + r.stderr[-2000:]


def test_packed_problem_keeps_its_metadata_arrays_alive():
    """A packed problem holds raw addresses of its metadata's arrays; built
    from a temporary VarlenMeta it must keep those arrays alive itself."""
    import gc
    import video_sparse_attention_amd as vsa
    p = vsa.vsa_build_metadata([100, 300, 5], topk=[1, 2, 1], device="cpu").problem(2, 64)
    gc.collect()
    d = p._device_arrays
    assert p.cu_blocks_q == d["cu_blocks_q"].data_ptr() and p.cu_blocks_kv == d["cu_blocks_kv"].data_ptr()
    assert p.block_sizes_q == d["block_sizes_q"].data_ptr() and p.topk_per_seq == d["topk"].data_ptr()
    assert d["cu_blocks_q"].tolist() == [0, 2, 7, 8]
    assert d["block_sizes_q"].tolist() == [64, 36, 64, 64, 64, 64, 44, 5]
