"""ctypes declarations of the libvsa C ABI (include/vsa.h).  No arithmetic here."""
from __future__ import annotations

import ctypes
import os

# VSA_LIBRARY names another build of the same library (the host-sanitizer
# build of the CPU tests); by default the in-tree libvsa.so is loaded.
LIB_PATH = os.environ.get("VSA_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "lib", "libvsa.so")

VSA_OK = 0
VSA_ERR_NULL = -1
VSA_ERR_UNSUPPORTED = -2
VSA_ERR_TOPK = -3
VSA_ERR_SHAPE = -4
VSA_ERR_GATE = -5
VSA_ERR_WORKSPACE = -6
VSA_ERR_ALIGN = -7
VSA_ERR_ALIAS = -8
VSA_ERR_HIP = -9

VSA_LAYOUT_DENSE = 0
VSA_LAYOUT_PACKED = 1
VSA_LAYOUT_BSHD = 2
VSA_GATE_NONE = 0
VSA_GATE_TOKEN = 1
VSA_GATE_FULL = 2

i32 = ctypes.c_int32
i64 = ctypes.c_int64
vp = ctypes.c_void_p
sz = ctypes.c_size_t


class VsaProblem(ctypes.Structure):
    _fields_ = [
        ("layout", i32), ("heads", i32), ("head_dim", i32), ("block_size", i32),
        ("batch", i32), ("seqlen_q", i32), ("seqlen_kv", i32), ("topk", i32),
        ("num_seqs", i32), ("total_q_blocks", i32), ("total_kv_blocks", i32),
        ("max_q_blocks", i32), ("max_kv_blocks", i32), ("max_topk", i32),
        ("cu_blocks_q", vp), ("cu_blocks_kv", vp), ("block_sizes_q", vp),
        ("block_sizes_kv", vp), ("topk_per_seq", vp),
    ]


class VsaMetaSizes(ctypes.Structure):
    _fields_ = [
        ("num_seqs", i32), ("total_q_blocks", i32), ("total_kv_blocks", i32),
        ("max_q_blocks", i32), ("max_kv_blocks", i32), ("max_topk", i32),
        ("q_slots", i64), ("kv_slots", i64),
    ]


P_PROBLEM = ctypes.POINTER(VsaProblem)

# name -> (restype, argtypes); the exported symbols of include/vsa.h
SIGNATURES = {
    "vsa_build_metadata": (i32, [i32, vp, vp, vp, i32, ctypes.POINTER(VsaMetaSizes), vp, vp, vp, vp, vp]),
    "vsa_workspace_size": (sz, [P_PROBLEM]),
    "vsa_coarse_topk": (i32, [P_PROBLEM, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
    "vsa_sparse_attn_from_indices": (i32, [P_PROBLEM, vp, vp, vp, vp, vp, vp, vp]),
    "vsa_sparse_attn_combine": (i32, [P_PROBLEM, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp]),
    "vsa_combine": (i32, [P_PROBLEM, vp, vp, i32, vp, vp, vp]),
    "vsa_sparse_attn_combine_train": (i32, [P_PROBLEM, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp]),
    "vsa_backward_workspace_size": (sz, [P_PROBLEM]),
    "vsa_backward": (i32, [P_PROBLEM, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp,
                           vp, vp, vp, vp, vp, sz, vp]),
    "vsa_backward_pooled": (i32, [P_PROBLEM, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp,
                                  vp, vp, vp, vp, vp, sz, vp, sz, vp]),
    "vsa_forward": (i32, [vp, vp, vp, vp, i32, vp, vp, vp, vp, vp,
                          i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]),
    "vsa_forward_noalloc": (i32, [vp, vp, vp, vp, i32, vp, vp, vp, vp, vp,
                                  i32, i32, i32, i32, i32, i32, i32, vp]),
    "vsa_noalloc_scratch_bytes": (sz, []),
    "vsa_forward_bshd": (i32, [vp, vp, vp, vp, i32, vp, vp, vp, vp, vp,
                               i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]),
    "vsa_forward_varlen": (i32, [vp, vp, vp, vp, i32, vp, vp, vp, vp, vp,
                                 vp, vp, vp, vp, vp,
                                 i32, i32, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]),
    "vsa_tile_partition": (i32, [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]),
    "vsa_build_tile_metadata": (i32, [i32, i32, i32, i32, i32, i32, i32, i32,
                                      ctypes.POINTER(VsaMetaSizes), vp, vp, vp, vp, vp]),
    "vsa_tile_gather": (i32, [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, vp]),
    "vsa_tile_scatter": (i32, [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, vp]),
    "vsa_status_string": (ctypes.c_char_p, [i32]),
    "vsa_last_error": (ctypes.c_char_p, []),
    "vsa_version": (ctypes.c_char_p, []),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libvsa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"libvsa.so not found at {path}: build it first "
            "(python -m video_sparse_attention_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class VsaError(RuntimeError):
    def __init__(self, status: int, detail: str, where: str):
        self.status = status
        self.detail = detail
        super().__init__(f"{where}: {detail or 'error'} (status {status})")


def check(status: int, where: str) -> None:
    if status != VSA_OK:
        lib = load()
        detail = (lib.vsa_last_error() or b"").decode()
        raise VsaError(status, detail or lib.vsa_status_string(status).decode(), where)
