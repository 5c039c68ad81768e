"""GPU parity at the full sizes of the large workloads, in the launch
configuration the benchmark times: every routing index and every coarse
output row is compared with the oracle, and the token outputs on a seeded
sample of query blocks (the oracle evaluates those blocks one by one)."""
import numpy as np
import pytest

import synth
from tests import gpu_common as G
from tests import numerics as N

pytestmark = pytest.mark.gpu

N_SAMPLE = 48


def _whole_heads(H, nq, picks):
    """Every query block of the first and the last head, plus sampled ones."""
    blocks = {(0, h, i) for h in (0, H - 1) for i in range(nq)}
    blocks |= {(0, int(p) // nq, int(p) % nq) for p in picks}
    return sorted(blocks)


def _assert_finite(gpu):
    for key in ("out", "out_fused", "out_s", "out_c"):
        assert np.isfinite(N.f64(gpu[key])).all(), f"{key}: non-finite values"


def test_large_video_dit_shape():
    """B=1, H=56, D=128, S=15488 (242 blocks), top-49, gated: heads 0 and 55
    compared token for token in full, sampled blocks of the others."""
    inp = synth.workload("large")
    B, H, Sq, Skv, D = inp.shape
    nq = Sq // 64
    rng = np.random.default_rng(4)
    picks = rng.choice(H * nq, N_SAMPLE, replace=False)
    blocks = _whole_heads(H, nq, picks)
    G.note(f"case large: H={H} S={Sq} topk={inp.topk}, {len(blocks)} blocks")
    gpu = G.run_dense_stages(inp)
    _assert_finite(gpu)
    ref = G.oracle_dense(inp, blocks=blocks)
    G.assert_tie_free(ref)
    G.assert_indices_equal(gpu["q2k_idx"], gpu["q2k_num"], ref)
    N.check_out_c(N.f64(gpu["out_c"]), ref["out_c"])
    rel = N.check_sparse(N.f64(gpu["out_s"]), ref["out_s"])
    mx, mean = N.check_out(N.f64(gpu["out"]), ref["out"])
    N.check_out(N.f64(gpu["out_fused"]), ref["out"], "out (fused combine)")
    N.check_fused(N.f64(gpu["out_fused"]), N.f64(gpu["out"]), N.f64(gpu["out_s"]))
    G.note(f"  out max-abs {mx:.2e} mean-abs {mean:.2e}; sparse rel-rms {rel:.2e}")


def test_pages_benchmark_shape():
    """B=1, H=16, D=128, S=49152 (768 blocks), top-64, ungated: the shape of
    the pages' listed benchmark command (bench.py --workload pages_bench_49k).
    Its block-level score matrix (16 x 768 x 768 float64, 75.5 MB) fits the
    coarse stage's bound, so the coarse stage runs in one chunk.  Heads 0 and
    15 are compared token for token in full, sampled blocks of the others."""
    inp = synth.workload("pages_bench_49k")
    B, H, Sq, Skv, D = inp.shape
    nq = Sq // 64
    rng = np.random.default_rng(6)
    picks = rng.choice(H * nq, N_SAMPLE, replace=False)
    blocks = _whole_heads(H, nq, picks)
    G.note(f"case pages bench shape: H={H} S={Sq} topk={inp.topk}, {len(blocks)} blocks")
    gpu = G.run_dense_stages(inp)
    _assert_finite(gpu)
    ref = G.oracle_dense(inp, blocks=blocks)
    G.assert_tie_free(ref)
    G.assert_indices_equal(gpu["q2k_idx"], gpu["q2k_num"], ref)
    N.check_out_c(N.f64(gpu["out_c"]), ref["out_c"])
    N.check_sparse(N.f64(gpu["out_s"]), ref["out_s"])
    mx, mean = N.check_out(N.f64(gpu["out_fused"]), ref["out"], "out (fused combine)")
    G.note(f"  out max-abs {mx:.2e} mean-abs {mean:.2e}")


@pytest.mark.parametrize("block", [64, 128, 256])
def test_varlen_many_sequences(block):
    """8 packed sequences, Q blocks 32..144, KV = Q + 8 blocks (of 64 tokens),
    H=24, gated; also in VSA blocks of 128 and 256 slots with top-k 20 % of
    those (the benchmark's --block-size runs)."""
    inp = synth.workload("varlen_many", block=block)
    nq_tot = sum(-(-s // block) for s in inp.seqlens_q)
    rng = np.random.default_rng(5 + block)
    picks = rng.choice(inp.heads * nq_tot, N_SAMPLE, replace=False)
    blocks = [(int(p) // nq_tot, int(p) % nq_tot) for p in picks] + [(inp.heads - 1, nq_tot - 1)]
    G.note(f"case varlen_many block={block}: lens={inp.seqlens_q} topk={inp.topk}")
    gpu = G.run_varlen_stages(inp)
    ref = G.oracle_varlen(inp, blocks=blocks)
    G.assert_tie_free(ref)
    G.assert_indices_equal(gpu["q2k_idx"], gpu["q2k_num"], ref)
    N.check_out_c(N.f64(gpu["out_c"]), ref["out_c"])
    N.check_sparse(N.f64(gpu["out_s"]), ref["out_s"])
    mx, mean = N.check_out(N.f64(gpu["out"]), ref["out"])
    N.check_out(N.f64(gpu["out_fused"]), ref["out"], "out (fused combine)")
    N.check_fused(N.f64(gpu["out_fused"]), N.f64(gpu["out"]), N.f64(gpu["out_s"]))
    G.note(f"  out max-abs {mx:.2e} mean-abs {mean:.2e}")


def test_large_sparse_on_oracle_indices():
    """The sparse stage at full size fed the oracle's routing."""
    inp = synth.workload("large")
    B, H, Sq, Skv, D = inp.shape
    nq = Sq // 64
    rng = np.random.default_rng(6)
    picks = rng.choice(H * nq, 24, replace=False)
    blocks = [(0, int(p) // nq, int(p) % nq) for p in picks]
    ref = G.oracle_dense(inp, blocks=blocks)
    gpu = G.run_dense_stages(inp, idx_override=(ref["q2k_idx"], ref["q2k_num"]))
    N.check_sparse(N.f64(gpu["out_s"]), ref["out_s"])


def test_coarse_in_chunks():
    """3000 x 3000 query/KV blocks on two heads: the float64 score matrix
    (144 MB) exceeds the coarse stage's workspace bound (128 MiB), so it runs
    in two chunks of query blocks; every index row, every coarse row and
    sampled outputs are compared with the oracle."""
    S = 64 * 3000
    inp = synth.dense_inputs(1, 2, S, 64, 7, seed=2100, gated=True)
    nq = S // 64
    rng = np.random.default_rng(7)
    blocks = [(0, int(i) % 2, int(i) // 2) for i in rng.choice(2 * nq, 16, replace=False)]
    blocks += [(0, 0, 2795), (0, 1, 2796), (0, 1, nq - 1)]
    G.note(f"case chunked coarse: S={S} D=64 topk=7, {len(blocks)} sampled blocks")
    gpu = G.run_dense_stages(inp)
    ref = G.oracle_dense(inp, blocks=blocks)
    G.assert_tie_free(ref)
    G.assert_indices_equal(gpu["q2k_idx"], gpu["q2k_num"], ref)
    N.check_out_c(N.f64(gpu["out_c"]), ref["out_c"])
    N.check_sparse(N.f64(gpu["out_s"]), ref["out_s"])
    N.check_out(N.f64(gpu["out_fused"]), ref["out"], "out (fused combine)")


def test_packed_coarse_in_chunks():
    """Two packed sequences of 2100 and 1900 blocks on four heads: the
    per-sequence float64 score matrix (2 x 4 x 2100 rows of 2100, 141 MB)
    exceeds the coarse stage's bound (128 MiB), so the packed coarse stage
    runs in three chunks of query blocks.  Every index row and every coarse
    row is compared with the oracle's separate varlen path, and the token
    outputs of the blocks on both sides of each chunk boundary."""
    sq = [64 * 2100, 64 * 1900 + 17]
    topk = [3, 4]
    inp = synth.varlen_inputs(sq, None, 4, 64, topk, seed=2200, gated=True, name="packed_chunks")
    per_row = 2 * 4 * 2100 * 8
    C = (128 << 20) // per_row  # query blocks per chunk (bound 128 MiB above 1/8 of q's bytes)
    assert 2 * 4 * 2100 * 2100 * 8 > (128 << 20) and C < 2100
    nq_tot = 2100 + 1900
    edges = sorted({c + d for c in range(C, 2100, C) for d in (-1, 0)})
    blocks = [(h, g) for h in (0, 3) for g in edges] + [(h, 2100 + g) for h in (1, 2) for g in edges if g < 1900]
    blocks += [(3, nq_tot - 1), (0, 0), (2, 2099), (1, 2100)]
    G.note(f"case packed chunks: lens={sq} C={C} boundary rows {edges}")
    gpu = G.run_varlen_stages(inp)
    ref = G.oracle_varlen(inp, blocks=blocks)
    G.assert_tie_free(ref)
    G.assert_indices_equal(gpu["q2k_idx"], gpu["q2k_num"], ref)
    N.check_out_c(N.f64(gpu["out_c"]), ref["out_c"])
    N.check_sparse(N.f64(gpu["out_s"]), ref["out_s"])
    N.check_out(N.f64(gpu["out_fused"]), ref["out"], "out (fused combine)")
