"""vsa_forward_noalloc (the forward whose workspace is the library's
per-device scratch array) against vsa_forward with a caller-provided
workspace, through the C ABI: two calls in a row, the second on a smaller
problem, each bitwise equal to vsa_forward on the same inputs (the same
kernels run in the same order), plus the routing against the oracle."""
import numpy as np
import pytest
import torch

import synth
import video_sparse_attention_amd as vsa
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


def _pair(inp, gate):
    q, k, v = (t.to(G.DEV) for t in (inp.q, inp.k, inp.v))
    g = None if gate is None else gate.to(G.DEV)
    ref = vsa.vsa_forward(q, k, v, inp.topk, g, return_aux=True)
    got = vsa.vsa_forward_noalloc(q, k, v, inp.topk, g, return_aux=True)
    torch.cuda.synchronize()
    for name, a, b in zip(("out", "out_c", "q2k_idx", "q2k_num"), got, ref):
        assert torch.equal(a.cpu(), b.cpu()), f"{name} differs from vsa_forward"
    return got


def test_noalloc_two_calls_match_vsa_forward():
    big = synth.dense_inputs(1, 8, 64 * 100 + 13, 128, 7, seed=3100, gated=True)
    small = synth.dense_inputs(2, 3, 64 * 20 + 5, 64, 4, seed=3101)
    G.note(f"case noalloc: big {big.shape} then small {small.shape}")
    assert vsa.vsa_workspace_size(vsa.dense_problem(*big.shape, big.topk)) <= vsa.vsa_noalloc_scratch_bytes()
    _pair(big, big.gate)
    full_gate = synth.full_gate(small.q.shape, 3102)
    out, out_c, idx, num = _pair(small, full_gate)
    ref = G.oracle_dense(synth.DenseInputs(small.q, small.k, small.v, full_gate, small.topk), blocks=[])
    G.assert_tie_free(ref)
    G.assert_indices_equal(idx.cpu(), num.cpu(), ref)
    assert np.isfinite(out.float().cpu().numpy()).all()
