"""The allocation-free single-launch step (btk_decode_step_noalloc): its scratch is
the library's own per-GPU device array.  Checked through the C ABI against
btk_decode_step (bit for bit: the same kernels on the same inputs) and against
the oracle under the parity rules, on calls in a row, the second with a smaller
problem, then the first again (the array keeps the previous call's contents)."""
import pytest
import torch

import block_top_sparse_btk_amd as btk
import oracle
import synth
from parity import check_indices, check_lse, check_outputs, sum_factor

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)


def _both(bt):
    d = bt.to(DEV)
    prob = btk.make_problem(d.q, d.k_cache, d.block_table)
    cent = oracle.centroids(bt.k_cache, bt.block_table, bt.seq_lens)
    L = bt.seq_lens.long()
    cent[bt.block_table[torch.arange(bt.batch), (L - 1) // 16].long()] = float("nan")  # stale
    first = (d.seq_lens - 1).to(torch.int32)
    ws = btk.new_workspace(prob, bt.top_k, DEV)
    c1, c2 = cent.to(DEV), cent.to(DEV)
    lse1 = torch.empty((bt.batch, bt.num_q_heads), device=DEV)
    lse2 = torch.full_like(lse1, float("nan"))
    out1, idx1 = btk.btk_decode_step(d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens, c1,
                                     bt.top_k, ws, first_pos=first, lse=lse1, problem=prob)
    out2, idx2 = btk.btk_decode_step_noalloc(d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                                             c2, bt.top_k, first_pos=first, lse=lse2,
                                             problem=prob)
    torch.cuda.synchronize()
    assert btk.workspace_error_bits(ws) == 0
    return (out1, idx1, lse1, c1), (out2, idx2, lse2, c2)


def test_noalloc_step_equals_the_workspace_step_on_calls_in_a_row():
    big = synth.make_config(3)
    small = synth.make_batch(name="noalloc-small", batch=5, num_q_heads=8, num_kv_heads=2,
                             head_dim=128, seq_lens=[1, 17, 300, 5000, 33], top_k=12, seed=91)
    for label, bt in (("config 3", big), ("smaller", small), ("config 3 again", big)):
        _say(f"[noalloc] {label}: B={bt.batch} Hkv={bt.num_kv_heads} k={bt.top_k}")
        ref, got = _both(bt)
        for x, y in zip(ref, got):
            assert torch.equal(x, y)
        ora = oracle.sparse_step(bt.q, bt.k_cache, bt.v_cache, bt.block_table, bt.seq_lens,
                                 bt.top_k)
        st = check_indices(got[1].cpu(), ora["indices"], ora["scores"], bt.seq_lens, bt.top_k,
                           sum_units=sum_factor(bt.group, bt.head_dim))
        check_outputs(got[0].cpu(), ora["out"], bt.dtype, st["equal_mask"], bt.group)
        check_lse(got[2].cpu(), ora["lse"], bt.dtype, st["equal_mask"], bt.group)
        _say(f"[noalloc]   ok near_tie={st['near_tie']} differ={st['differ']}")
