"""The benchmark's byte accounting, pinned to the pages' Table 2 figure
(Pith review of "Kinetics: Rethinking Test-Time Scaling Laws", referee report,
major comment 1: Qwen3-32B holds 8 GB of KV cache per 32K-token sequence)."""
import json
import os

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "table2_kv_bytes.json")


def test_dense_bytes_per_token_match_table2():
    fx = json.load(open(GOLDEN))
    per_layer = bench.dense_kv_bytes_per_token(fx["num_kv_heads"], fx["head_dim"],
                                               fx["bytes_per_element"])
    assert per_layer * fx["layers"] * fx["tokens"] == fx["kv_bytes"]
    # the dense model's KV term over one 32K sequence of one layer is the same figure
    b = bench.algorithmic_bytes([fx["tokens"]], 64, fx["num_kv_heads"], fx["head_dim"], 64,
                                fx["bytes_per_element"])
    kv_only = b["dense"] - 4 * (fx["tokens"] // 16) - 2 * 64 * fx["head_dim"] * 2
    assert kv_only * fx["layers"] == fx["kv_bytes"]


def test_sparse_bytes_shrink_and_k_at_least_blocks_reads_everything():
    b = bench.algorithmic_bytes([32768] * 8, 64, 8, 128, 64, 2)
    assert b["step"] < b["dense"] / 10
    # centroid scan is 1/16 of the dense KV bytes for fp32 centroids and bf16 K+V
    scan = 8 * 8 * 4 * 128 * 2048
    assert 16 * scan == 8 * 8 * 2 * 32768 * 128 * 2
    full = bench.algorithmic_bytes([100], 4, 2, 64, 64, 2)  # 7 blocks < k
    kv_att = full["attend"] - 2 * (8 * 64 + 2 * 2 * 64 * 2)
    assert kv_att == 2 * 2 * 100 * 64 * 2


def test_exact_selected_tokens():
    import torch
    idx = torch.tensor([[[0, 6, -1]]], dtype=torch.int32)
    assert bench.selected_tokens(idx, [100]) == [[16 + 4]]


def test_local_window_bytes():
    # a window covering every block moves exactly the dense bytes
    lens = [37, 16, 1, 200]
    full = bench.algorithmic_bytes(lens, 8, 2, 128, 64, 2)
    assert full["local"] == full["dense"]
    # a window of w whole blocks moves w pages of K and V per unit, plus q/out and table
    w, r, D, e = 4, 4, 128, 2
    part = bench.algorithmic_bytes([1000], 8, 2, D, w, e)
    nb = (1000 + 15) // 16
    toks = 1000 - 16 * (nb - w)  # the last block holds 1000 - 16*62 = 8 tokens
    assert toks == 3 * 16 + 8
    assert part["local"] == 4 * w + 2 * (2 * r * D * e + 2 * toks * D * e)


def test_token_baseline_bytes():
    # every key once, plus the kept tokens' K and V (16k of them, or all of L)
    r, D, e, k = 4, 128, 2, 2
    out = bench.algorithmic_bytes([1000, 20], 8, 2, D, k, e)
    want = 4 * 63 + 4 * 2
    for L in (1000, 20):
        want += 2 * (2 * r * D * e + L * D * e + 2 * min(16 * k, L) * D * e)
    assert out["token"] == want


def test_bench_refuses_more_than_one_gpu():
    """The benchmark runs on one GPU; asking for more exits with a message before any GPU work."""
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_sketch_step_bytes():
    lens, hq, hkv, D, k, e = [1000, 20, 4000], 8, 2, 128, 16, 2
    sel = [[16 * k] * hkv, [20] * hkv, [16 * k] * hkv]
    step = bench.algorithmic_bytes(lens, hq, hkv, D, k, e, sel_tokens=sel)["step"]
    units = len(lens) * hkv
    nbs = [(L + 15) // 16 for L in lens]
    # the fp32-scan kernel: the step's bytes plus the rebuilt sketch row of each unit
    fp32 = bench.sketch_step_bytes(lens, hq, hkv, D, k, e, [[n] * hkv for n in nbs], sel,
                                   fp32_scan=True)
    assert fp32 == step + units * (D + 8)
    # the unit kernel: every fp32 row replaced by the block's sketch row, plus the
    # m candidates' fp32 rows
    m = [[3, 5], [0, 0], [40, 7]]
    unit = bench.sketch_step_bytes(lens, hq, hkv, D, k, e, m, sel)
    want = step + units * (D + 8)
    for n, mm in zip(nbs, m):
        for x in mm:
            want += n * (D + 8) - 4 * D * n + 4 * D * x
    assert unit == want
