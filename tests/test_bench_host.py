"""Host-side pieces of bench.py: the pair count behind the effective-FLOP
figure, and the refusal of more than one GPU."""
import subprocess
import sys

import numpy as np

import bench
import oracle


def test_pair_count_block64_is_nq_times_k():
    idx = np.tile(np.arange(5, dtype=np.int32), (1, 2, 7, 1))
    num = np.full((1, 2, 7), 5, dtype=np.int32)
    assert bench.pair_count(idx, num, 64 * 7 - 3, 64 * 9, 64) == 2 * 7 * 5


def test_pair_count_large_blocks_by_hand():
    # Sq = 300 (VSA blocks of 256: 256 + 44 tokens -> 4 + 1 query sub-blocks),
    # Skv = 600 (10 sub-blocks: VSA blocks of 4, 4, 2)
    idx = np.array([[[[0, 2], [2, 1]]]])
    num = np.array([[[2, 1]]])
    # block 0 (4 query sub-blocks): KV blocks 0 and 2 -> 4 + 2 sub-blocks
    # block 1 (1 query sub-block): only its first entry (block 2) -> 2
    assert bench.pair_count(idx, num, 300, 600, 256) == 4 * 6 + 1 * 2


def test_pair_count_matches_oracle_token_count():
    """Brute force: count 64-token (query, key) block pairs from the oracle's
    routing token by token."""
    rng = np.random.default_rng(3)
    Sq, Skv, block = 128 * 3 + 70, 128 * 4 + 5, 128
    q, k, v = (rng.standard_normal((1, 1, n, 16)) for n in (Sq, Skv, Skv))
    r = oracle.vsa_forward(q, k, v, topk=2, block=block)
    pairs = set()
    for qt in range(Sq):
        for J in r["q2k_idx"][0, 0, qt // block][: r["q2k_num"][0, 0, qt // block]]:
            for kt in range(block * J, min(block * (J + 1), Skv)):
                pairs.add((qt // 64, kt // 64))
    assert bench.pair_count(r["q2k_idx"], r["q2k_num"], Sq, Skv, block) == len(pairs)


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert p.returncode != 0 and "one GPU" in p.stderr
