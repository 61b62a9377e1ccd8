"""Host-side checks of bench.py: the algorithmic byte and flop counts its roofline divides by,
and its refusal to run on more than one GPU.  No GPU needed."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import meta as ometa  # noqa: E402
from tree_attention_draft_amd import workloads  # noqa: E402


def test_algorithmic_bytes_of_the_benchmark_batch_written_out():
    # B=64 requests, L=4096, N=33, 32 query / 8 kv heads, D=128, bf16: per request K and V
    # over the L + N visible keys, Q read and out written, fp32 LSE, int32 parents and the
    # prefix length
    T = 4096 + 33
    kv = T * 8 * 128 * 2 * 2
    q_out = 2 * 33 * 32 * 128 * 2
    lse = 33 * 32 * 4
    meta = 33 * 4 + 4
    assert bench.algorithmic_bytes([4096] * 64, 33, 32, 8, 128, 2) == 64 * (kv + q_out + lse + meta)
    assert bench.algorithmic_bytes([4096] * 64, 33, 32, 8, 128, 2) == 1_117_274_624


def test_algorithmic_bytes_counts_each_page_id_once():
    # paged: one int32 page id per page of the L + N keys, on top of the contiguous count
    plain = bench.algorithmic_bytes([100, 37], 5, 4, 2, 64, 2)
    paged = bench.algorithmic_bytes([100, 37], 5, 4, 2, 64, 2, paged_page=16)
    assert paged - plain == 4 * (-(-105 // 16) + -(-42 // 16))


def test_algorithmic_flops_match_a_count_over_the_oracle_mask():
    # 4 * D flops (two multiply-adds) per query head, per node, per key the node may see:
    # every prefix key plus the tree keys the oracle's ancestor mask allows
    rng = np.random.default_rng(7)
    trees = [workloads.random_tree(rng, 12, 4)[0] for _ in range(3)]
    L = [5, 0, 17]
    Hq, D = 3, 16
    metas = [ometa.build_from_paths(t, 0) for t in trees]
    brute = 0
    for m, Lb in zip(metas, L):
        for row in m["mask"]:
            brute += 4 * D * Hq * (Lb + sum(bool(x) for x in row))
    assert bench.algorithmic_flops(L, [m["depth"] for m in metas], Hq, D) == brute


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("flag", ["--steady-steps", "--steady-warmup"])
def test_steady_state_leg_flags_are_declared(flag):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and flag in r.stdout
