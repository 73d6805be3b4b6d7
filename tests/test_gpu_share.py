"""The single-launch step at one GPU's share of a large serving batch.

Kinetics README, "Benchmark Block TopK Attention throughput": Qwen3-8B served at
batch 4096 with 32768-token contexts and 64 pages kept, split eight ways by
tensor parallelism, so one GPU holds one KV head and its four query heads of
every sequence.  The caches (69 GB) are drawn on the device; the step runs on
the whole batch, equals the three separate calls bit for bit on every unit, and
is checked against the oracle on sequences copied to the host from each 1024-
sequence window of the step's row prefix (first, last and window edges).
"""
import pytest
import torch

import block_top_sparse_btk_amd as btk
import oracle
import synth
from parity import CENTROID_TOL, check_indices, check_lse, check_outputs, max_abs, sum_factor

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SHARE = dict(batch=4096, num_q_heads=4, num_kv_heads=1, head_dim=128, context=32768, top_k=64,
             seed=8004)
SAMPLE = [0, 1, 1023, 1024, 2047, 2048, 3071, 3072, 4094, 4095, 777, 2999]


def _say(*a):
    print(*a, flush=True)


def test_one_gpu_share_b4096():
    _say(f"[share] drawing {SHARE} on the device")
    bt = synth.make_device_batch(device=DEV, name="qwen3-8b-share", **SHARE)
    prob = btk.make_problem(bt.q, bt.k_cache, bt.block_table)
    k = bt.top_k
    first = (bt.seq_lens - 1).to(torch.int32)
    cent = torch.zeros((bt.num_pages, bt.num_kv_heads, bt.head_dim), dtype=torch.float32,
                       device=DEV)
    btk.btk_centroid_update(bt.k_cache, bt.block_table, bt.seq_lens, cent, problem=prob)
    torch.cuda.synchronize()
    _say("[share] centroids built; three separate calls")
    ws1 = btk.new_workspace(prob, k, DEV)
    c1 = cent.clone()
    lse1 = torch.empty((bt.batch, bt.num_q_heads), device=DEV)
    out1, idx1 = btk.sparse_decode_step(bt.q, bt.k_cache, bt.v_cache, bt.block_table,
                                        bt.seq_lens, c1, k, ws1, first_pos=first, lse=lse1,
                                        problem=prob)
    torch.cuda.synchronize()
    del c1
    _say("[share] single launch, twice on one workspace")
    ws2 = btk.new_workspace(prob, k, DEV)
    for rep in range(2):
        c2 = cent.clone()
        lse2 = torch.empty_like(lse1)
        out2, idx2 = btk.btk_decode_step(bt.q, bt.k_cache, bt.v_cache, bt.block_table,
                                         bt.seq_lens, c2, k, ws2, first_pos=first, lse=lse2,
                                         problem=prob)
        torch.cuda.synchronize()
        assert torch.equal(idx2, idx1), rep
        assert torch.equal(out2, out1), rep
        assert torch.equal(lse2, lse1), rep
        assert torch.equal(c2, cent), rep  # full pages: the refreshed page is unchanged
        del c2
    assert btk.workspace_error_bits(ws1) == 0 and btk.workspace_error_bits(ws2) == 0
    _say(f"[share] step == separate calls on {bt.batch} units; oracle on {SAMPLE}")
    sub, pages = synth.extract(bt, SAMPLE)
    ora = oracle.sparse_step(sub.q, sub.k_cache, sub.v_cache, sub.block_table, sub.seq_lens, k)
    assert max_abs(cent[pages.to(DEV)].cpu(), ora["centroids"]) <= CENTROID_TOL
    sel = torch.tensor(SAMPLE)
    g_idx, g_out, g_lse = idx2.cpu()[sel], out2.cpu()[sel], lse2.cpu()[sel]
    st = check_indices(g_idx, ora["indices"], ora["scores"], sub.seq_lens, k,
                       sum_units=sum_factor(sub.group, sub.head_dim))
    check_outputs(g_out, ora["out"], sub.dtype, st["equal_mask"], sub.group)
    check_lse(g_lse, ora["lse"], sub.dtype, st["equal_mask"], sub.group)
    o_own, l_own, _ = oracle.attend(sub.q, sub.k_cache, sub.v_cache, sub.block_table,
                                    sub.seq_lens, g_idx)
    check_outputs(g_out, o_own, sub.dtype, what="step out on own indices")
    check_lse(g_lse, l_own, sub.dtype)
    _say(f"[share] ok: {st['units']} sampled units, {st['strict']} strict, "
         f"{st['differ']} differ near ties")
