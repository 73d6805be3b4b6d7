"""The single-launch step does not depend on all of its workgroups being resident.

Every share of the scan is claimed before it is scored, by its own workgroup or,
if that one has not started, by workgroup 0 (dispatched first) or a workgroup
without phase-2 items; so no wait depends on a workgroup that is not running.
BTK_STEP_TEST_FLAGS=1 makes every owner leave its share unclaimed, which forces
that path from the host; results must not change.  Every kernel exits normally
in these tests (the second-stream kernel is an ordinary matrix product).
"""
import os

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


def _run_step(bt, d, prob, cent, ws, append=False):
    L = bt.seq_lens.long()
    first = (d.seq_lens - 1).to(torch.int32)
    c = cent.clone()
    lse = torch.empty((bt.batch, bt.num_q_heads), device=DEV)
    if append:
        page = bt.block_table[torch.arange(bt.batch), (L - 1) // 16].long()[:, None].to(DEV)
        slot = ((L - 1) % 16)[:, None].to(DEV)
        heads = torch.arange(bt.num_kv_heads, device=DEV)[None, :]
        kn = d.k_cache[page, heads, slot, :].contiguous()
        vn = d.v_cache[page, heads, :, slot].contiguous()
        kc, vc = d.k_cache.clone(), d.v_cache.clone()
        out, idx = btk.btk_decode_step_append(d.q, kn, vn, kc, vc, d.block_table, d.seq_lens, c,
                                              bt.top_k, ws, lse=lse, problem=prob)
    else:
        out, idx = btk.btk_decode_step(d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens, c,
                                       bt.top_k, ws, first_pos=first, lse=lse, problem=prob)
    return out, idx, lse, c


CASES = [("config3", dict(cfg=3)),
         ("ragged-small", dict(kw=dict(batch=5, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                       seq_lens=[1, 17, 300, 5000, 33], top_k=12, seed=31))),
         ("fp32-d64", dict(kw=dict(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64,
                                   seq_lens=[2000, 17, 640], top_k=9, seed=35,
                                   dtype=torch.float32))),
         # 2048 items: no workgroup is without items, so workgroup 0 claims every share
         ("no-idle-1024", dict(kw=dict(batch=1024, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                       seq_lens=[1 + (i * 7919) % 700 for i in range(1024)],
                                       top_k=8, seed=34))),
         # several row-prefix windows: taken-over shares lie in any of them
         ("windows-2500", dict(kw=dict(batch=2500, num_q_heads=4, num_kv_heads=1, head_dim=128,
                                       seq_lens=[1 + (i * 7919) % 300 for i in range(2500)],
                                       top_k=8, seed=38)))]


@pytest.mark.parametrize("append", [False, True], ids=["step", "step+append"])
@pytest.mark.parametrize("label,spec", CASES, ids=[c[0] for c in CASES])
def test_unclaimed_shares_are_taken_over(label, spec, append):
    """With every owner leaving its share unclaimed, workgroup 0 and the
    workgroups without items score all shares: indices, outputs, lse and
    centroids equal the normal step's bit for bit and the oracle's under the
    usual rules; the workspace serves normal launches afterwards."""
    bt = synth.make_config(spec["cfg"]) if "cfg" in spec else synth.make_batch(name=label,
                                                                               **spec["kw"])
    _say(f"[takeover] {label} append={append}")
    d = bt.to(DEV)
    prob = btk.make_problem(d.q, d.k_cache, d.block_table)
    cent = oracle.centroids(bt.k_cache, bt.block_table, bt.seq_lens).to(DEV)
    ws0 = btk.new_workspace(prob, bt.top_k, DEV)
    ref = _run_step(bt, d, prob, cent, ws0, append)
    torch.cuda.synchronize()
    assert btk.workspace_error_bits(ws0) == 0
    ws1 = btk.new_workspace(prob, bt.top_k, DEV)
    old = os.environ.get("BTK_STEP_TEST_FLAGS")
    os.environ["BTK_STEP_TEST_FLAGS"] = "1"
    try:
        got = [_run_step(bt, d, prob, cent, ws1, append) for _ in range(2)]
        torch.cuda.synchronize()
    finally:
        if old is None:
            del os.environ["BTK_STEP_TEST_FLAGS"]
        else:
            os.environ["BTK_STEP_TEST_FLAGS"] = old
    got.append(_run_step(bt, d, prob, cent, ws1, append))  # a normal launch after them
    torch.cuda.synchronize()
    assert btk.workspace_error_bits(ws1) == 0
    for g in got:
        for x, y in zip(g, ref):
            assert torch.equal(x, y)
    if bt.batch <= 64:
        ora = oracle.sparse_step(bt.q, bt.k_cache, bt.v_cache, bt.block_table, bt.seq_lens,
                                 bt.top_k)
        st = check_indices(got[0][1].cpu(), ora["indices"], ora["scores"], bt.seq_lens, bt.top_k,
                           sum_units=sum_factor(bt.group, bt.head_dim))
        check_outputs(got[0][0].cpu(), ora["out"], bt.dtype, st["equal_mask"], bt.group)
        check_lse(got[0][2].cpu(), ora["lse"], bt.dtype, st["equal_mask"], bt.group)
    _say("[takeover]   ok")


def test_step_beside_a_long_kernel_on_another_stream():
    """The step is launched while matrix products on a second stream hold much of
    the device, so some of its workgroups start late; results are unchanged."""
    bt = synth.make_config(3)
    _say("[beside] config 3 next to fp32 matrix products on a second stream")
    d = bt.to(DEV)
    prob = btk.make_problem(d.q, d.k_cache, d.block_table)
    cent = oracle.centroids(bt.k_cache, bt.block_table, bt.seq_lens).to(DEV)
    ws0 = btk.new_workspace(prob, bt.top_k, DEV)
    ref = _run_step(bt, d, prob, cent, ws0)
    torch.cuda.synchronize()
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    a = torch.randn(4096, 4096, device=DEV, generator=g)
    b = torch.randn(4096, 4096, device=DEV, generator=g)
    side = torch.cuda.Stream()
    ws1 = btk.new_workspace(prob, bt.top_k, DEV)
    results = []
    for rep in range(3):
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(8):
                c = a @ b
        results.append(_run_step(bt, d, prob, cent, ws1))
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
    assert torch.isfinite(c).all()
    assert btk.workspace_error_bits(ws1) == 0
    for r in results:
        for x, y in zip(r, ref):
            assert torch.equal(x, y)
    _say("[beside]   ok")
