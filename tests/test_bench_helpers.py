"""Host-side checks of the benchmark's reporting helpers (no GPU)."""
import sys
import types

import numpy as np
import pytest
import torch

sys.argv = sys.argv[:1]
import bench  # noqa: E402


def test_spearman_matches_scipy_with_ties():
    from scipy.stats import spearmanr

    r = np.random.default_rng(3)
    a = r.random(40).round(2).tolist()
    b = (np.array(a) * 0.5 + r.random(40) * 0.3).round(2).tolist()
    assert bench._spearman(a, b) == pytest.approx(spearmanr(a, b).statistic, abs=1e-12)
    assert bench._spearman([1.0, 2.0], [2.0, 1.0]) is None


def test_agreement_stats_hand_example():
    c = [0.1, 0.6, 0.3, 0.55]   # C_struct >= 0.5: heads 1 and 3
    d = [0.05, 0.5, 0.4, 0.2]   # JSD distances
    st = bench.agreement_stats(c, d, 0.5, (0.1, 0.45))
    assert st["vs_heads_cstruct"] == 2
    # distance >= 0.1: heads 1, 2, 3 -> alike on 0, 1, 3
    assert st["agreement_at"][0.1] == pytest.approx(0.75)
    # distance >= 0.45: head 1 only -> alike on 0, 1, 2
    assert st["agreement_at"][0.45] == pytest.approx(0.75)
    # no threshold separates {1, 3} from {0, 2} (head 3's distance is below head 2's);
    # the first threshold reaching the best is the distance 0.2
    assert st["best_agreement"] == pytest.approx(0.75)
    assert st["best_tau_jsd"] == 0.2


def test_needle_recall_counts_listed_blocks_and_kept_columns():
    N, B = 4, 128
    # one sink head (0) of one KV group, needles at keys 130 (block 1) and 300 (block 2)
    x = types.SimpleNamespace(q=torch.zeros(1, N * B, 1), k=torch.zeros(1, N * B, 1), sink_heads=[0],
                              needle_pos={0: [130, 300]})
    count = torch.zeros(1, N, dtype=torch.int32)
    idx = torch.zeros(N * (N + 1) // 2, dtype=torch.int32)
    last = (N - 1) * N // 2
    count[0, N - 1] = 2
    idx[last:last + 2] = torch.tensor([1, 3])  # the last query block lists key blocks 1 and 3
    bufs = types.SimpleNamespace(blocks={"count": count, "idx": idx},
                                 cols=torch.tensor([[300, 0, 0, 0]], dtype=torch.int32),
                                 ncols=torch.tensor([1], dtype=torch.int32))
    assert bench.needle_recall(x, bufs, N, tokens=False) == pytest.approx(0.5)
    assert bench.needle_recall(x, bufs, N, tokens=True) == pytest.approx(1.0)


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_bench_refuses_more_than_one_gpu(gpus):
    """The layer is timed on one GPU; asking for more exits with status 2 and
    says so, before touching torch or a GPU."""
    import os
    import subprocess

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", gpus],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_record_matches_the_attention_kernel():
    """The HBM counters the bench line reports as `traffic` were taken on the
    attention kernel as committed (hash of attn.hip and common.h); after a
    kernel change they must be taken again, or the bench reports null."""
    import json
    import os

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    with open(os.path.join(root, "profiles", "sparse_attn_traffic.json")) as f:
        rec = json.load(f)
    assert rec["kernel_sha"] == bench.kernel_sha()
    assert rec["workload"] == "llama3.1-8b-512k"
    assert rec["hbm_bytes_per_launch"] == rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
    assert rec["hbm_bytes_per_launch"] > rec["algorithmic_bytes_per_launch"] > 0


@pytest.mark.parametrize("taken", ["two-block", "one-block", "one-block, runs of 16 blocks per XCD"])
def test_attn_schedule_reads_the_decision_words(taken):
    """The bench reports which attention kernel took a call's items from the
    decision words after the schedule sums: the two-block kernel runs when
    its pair passes the two-block test, a one-block kernel when its pair
    fails it ((1, 0) passes, (0, 1) fails)."""
    go_two, stop_two = (1, 0), (0, 1)
    go_one, stop_one = (0, 1), (1, 0)
    words = {"two-block": go_two + stop_one + stop_one,
             "one-block": stop_two + go_one + stop_one,
             "one-block, runs of 16 blocks per XCD": stop_two + stop_one + go_one}[taken]
    ws = torch.zeros(256, dtype=torch.uint8)
    ws[80:128] = torch.tensor(words, dtype=torch.int64).view(torch.uint8)
    assert bench.attn_schedule(torch, ws) == taken
    ws[80:128] = torch.tensor(go_two + go_one + stop_one, dtype=torch.int64).view(torch.uint8)
    assert bench.attn_schedule(torch, ws) == "unknown"
