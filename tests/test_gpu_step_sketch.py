"""btk_decode_step_sketch against btk_decode_step (bit for bit) and the oracle.

The sketched step reads 8-bit block sketches in place of the fp32 centroid rows
and scores only the blocks the sketch cannot rule out, so every case compares
its indices, outputs, lse and centroids with btk_decode_step's on the same
inputs, exactly, and with the oracle (centroids, the margin rule, outputs and
lse on equal selections, and every unit's output against the oracle's
attention over the step's own indices).  The sketch rows the step rebuilds for
the touched blocks must equal what btk_sketch_update writes from the updated
centroids.  Covered: the five workloads (the 32B sweep 8K-64K), ragged and edge
shapes (D=64, fp32, group 1 and 16, k >= n_b), 1024 and 3000 sequences (row
prefix windows), exact score ties, a sketch never built (every block a
candidate: the exact path over all blocks, beyond 1024 candidates the full
scan), invalid lengths and pages, and three decode steps in a row on one
sketch that only the step keeps current.
"""
import pytest
import torch

import block_top_sparse_btk_amd as btk
import oracle
import synth
from parity import (CENTROID_TOL, check_indices, check_lse, check_outputs, max_abs, n_blocks,
                    sum_factor)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)


CASES = [("config1", dict(cfg=1)), ("config2", dict(cfg=2)), ("config3", dict(cfg=3)),
         ("config4", dict(cfg=4)), ("config5-8k", dict(cfg=5, context=8192)),
         ("config5-16k", dict(cfg=5, context=16384)),
         ("config5-32k", dict(cfg=5, context=32768)),
         ("config5-64k", dict(cfg=5, context=65536)),
         ("ragged-small", dict(kw=dict(batch=5, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                       seq_lens=[1, 17, 300, 5000, 33], top_k=12, seed=31))),
         ("k-exceeds-blocks", dict(kw=dict(batch=3, num_q_heads=8, num_kv_heads=4, head_dim=128,
                                           seq_lens=[40, 200, 16], top_k=20, seed=38))),
         ("d64-group1", dict(kw=dict(batch=3, num_q_heads=4, num_kv_heads=4, head_dim=64,
                                     seq_lens=[100, 999, 64], top_k=5, seed=32))),
         ("group16-heavy", dict(kw=dict(batch=2, num_q_heads=32, num_kv_heads=2, head_dim=128,
                                        seq_lens=[1500, 999], top_k=12, seed=39,
                                        heavy_frac=0.1))),
         ("fp32-d128", dict(kw=dict(batch=2, num_q_heads=6, num_kv_heads=2, head_dim=128,
                                    seq_lens=[333, 1000], top_k=6, seed=33,
                                    dtype=torch.float32))),
         ("fp32-d64", dict(kw=dict(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64,
                                   seq_lens=[2000, 17, 640], top_k=9, seed=35,
                                   dtype=torch.float32))),
         ("batch-1024", dict(kw=dict(batch=1024, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                     seq_lens=[1 + (i * 7919) % 700 for i in range(1024)],
                                     top_k=8, seed=34))),
         ("windows-3000-hkv1", dict(kw=dict(batch=3000, num_q_heads=4, num_kv_heads=1,
                                            head_dim=128,
                                            seq_lens=[1 + (i * 7919) % 400 for i in range(3000)],
                                            top_k=8, seed=36))),
         # block tables wider than 2048 blocks, up to the unit kernel's 3072
         ("long-3072-blocks", dict(kw=dict(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                           seq_lens=[3072 * 16, 2049 * 16 + 3, 700], top_k=40,
                                           seed=40, max_blocks=3072))),
         ("long-2600-fp32-d64", dict(kw=dict(batch=2, num_q_heads=4, num_kv_heads=1,
                                             head_dim=64, seq_lens=[2600 * 16 - 9, 2100 * 16],
                                             top_k=17, seed=41, max_blocks=2601,
                                             dtype=torch.float32)))]

_CACHE = {}


def _batch(label, spec):
    key = label
    if key not in _CACHE:
        _CACHE.clear()  # one workload at a time in host memory
        if "cfg" in spec:
            _CACHE[key] = synth.make_config(spec["cfg"], context=spec.get("context"))
        else:
            _CACHE[key] = synth.make_batch(name=label, **spec["kw"])
    return _CACHE[key]


def _stale_centroids(bt):
    """The oracle's centroids with every newest token's page set to NaN (stale
    before the step, which recomputes it)."""
    full = oracle.centroids(bt.k_cache, bt.block_table, bt.seq_lens)
    stale = full.clone()
    L = bt.seq_lens.long()
    stale[bt.block_table[torch.arange(bt.batch), (L - 1) // 16].long()] = float("nan")
    return full, stale


def _run_both(d, prob, k, cent_a, cent_b, sketch, first, ws_a=None, ws_b=None, counts=None):
    """btk_decode_step on cent_a and btk_decode_step_sketch on cent_b / sketch."""
    ws_a = ws_a if ws_a is not None else btk.new_workspace(prob, k, DEV)
    ws_b = ws_b if ws_b is not None else btk.new_workspace(prob, k, DEV)
    lse_a = torch.full((d.batch, d.num_q_heads), float("nan"), device=DEV)
    lse_b = lse_a.clone()
    out_a, idx_a = btk.btk_decode_step(d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                                       cent_a, k, ws_a, first_pos=first, lse=lse_a, problem=prob)
    out_b, idx_b = btk.btk_decode_step_sketch(d.q, d.k_cache, d.v_cache, d.block_table,
                                              d.seq_lens, cent_b, sketch, k, ws_b,
                                              first_pos=first, lse=lse_b, cand_counts=counts,
                                              problem=prob)
    torch.cuda.synchronize()
    a = dict(idx=idx_a.cpu(), out=out_a.cpu(), lse=lse_a.cpu(), cent=cent_a.cpu(),
             err=btk.workspace_error_bits(ws_a))
    b = dict(idx=idx_b.cpu(), out=out_b.cpu(), lse=lse_b.cpu(), cent=cent_b.cpu(),
             err=btk.workspace_error_bits(ws_b))
    return a, b


def _assert_same(a, b, units=None):
    assert a["err"] == b["err"]
    assert torch.equal(a["idx"], b["idx"])
    if units is None:
        assert torch.equal(a["out"], b["out"]) and torch.equal(a["lse"], b["lse"])
    else:
        assert torch.equal(a["out"][units], b["out"][units])
        assert torch.equal(a["lse"][units], b["lse"][units])
    assert torch.equal(a["cent"], b["cent"])


def _check_counts(counts, bt, k):
    nb = torch.tensor(n_blocks(bt.seq_lens))[:, None].expand_as(counts)
    kb = torch.clamp(nb, max=k)
    keep_all = nb <= k
    assert (counts[keep_all] == 0).all()
    assert ((counts[~keep_all] >= kb[~keep_all]) & (counts[~keep_all] <= nb[~keep_all])).all()


# Which kernel the sketched step runs (BTK_STEP_TEST_FLAGS, read at each call):
# "auto" the library's choice (one workgroup per unit when the units fill the
# device, else the persistent kernel's fp32 scan, which rebuilds the touched
# blocks' sketch rows), "unit" the one-workgroup-per-unit kernel wherever its
# limits allow (small batches too; the Best-of-N and 32B cases exceed them),
# "persistent" never (the batches where auto takes the unit kernel).
MODES = {"auto": "0", "unit": "2", "persistent": "4"}
_UNIT_AUTO = {"config2", "config3", "batch-1024", "windows-3000-hkv1"}
MODE_CASES = ([(lab, sp, "auto") for lab, sp in CASES]
              + [(lab, sp, "unit") for lab, sp in CASES
                 if sp.get("cfg") not in (4, 5) and lab not in _UNIT_AUTO]
              + [(lab, sp, "persistent") for lab, sp in CASES if lab in _UNIT_AUTO])


@pytest.fixture
def kernel_mode(request, monkeypatch):
    mode = getattr(request, "param", "auto")
    monkeypatch.setenv("BTK_STEP_TEST_FLAGS", MODES[mode])
    return mode


@pytest.mark.parametrize("label,spec,kernel_mode", MODE_CASES,
                         ids=[f"{c[0]}-{c[2]}" for c in MODE_CASES], indirect=["kernel_mode"])
def test_sketch_step_equals_step_and_oracle(label, spec, kernel_mode):
    bt = _batch(label, spec)
    _say(f"[sketch-step] {label} ({kernel_mode})")
    d = bt.to(DEV)
    prob = btk.make_problem(d.q, d.k_cache, d.block_table)
    k = bt.top_k
    first = (d.seq_lens - 1).to(torch.int32)
    full, stale = _stale_centroids(bt)
    ws_s = btk.new_workspace(prob, k, DEV)
    # the sketch as a caller keeps it before the step: built from the centroids
    # as they were (the touched blocks' rows from the stale ones)
    sketch = btk.new_sketch(prob, DEV)
    btk.btk_sketch_update(stale.to(DEV), d.block_table, d.seq_lens, sketch, ws_s, problem=prob)
    counts = torch.full((bt.batch, bt.num_kv_heads), -7, dtype=torch.int32, device=DEV)
    ws_b = btk.new_workspace(prob, k, DEV)
    for rep in range(3):  # three launches in a row on one workspace and one sketch
        a, b = _run_both(d, prob, k, stale.to(DEV), stale.to(DEV), sketch, first, ws_b=ws_b,
                         counts=counts)
        assert a["err"] == 0
        _assert_same(a, b)
    _check_counts(counts.cpu(), bt, k)
    # the rebuilt rows equal what the sketch update writes from the new centroids
    ref = sketch.clone()
    btk.btk_sketch_update(b["cent"].to(DEV), d.block_table, d.seq_lens, ref, ws_s,
                          first_pos=first, problem=prob)
    torch.cuda.synchronize()
    assert torch.equal(ref, sketch)
    # and against the oracle
    assert max_abs(b["cent"], full) <= CENTROID_TOL
    ora = oracle.sparse_step(bt.q, bt.k_cache, bt.v_cache, bt.block_table, bt.seq_lens, k)
    st = check_indices(b["idx"], ora["indices"], ora["scores"], bt.seq_lens, k,
                       sum_units=sum_factor(bt.group, bt.head_dim))
    check_outputs(b["out"], ora["out"], bt.dtype, st["equal_mask"], bt.group)
    check_lse(b["lse"], ora["lse"], bt.dtype, st["equal_mask"], bt.group)
    o_own, l_own, _ = oracle.attend(bt.q, bt.k_cache, bt.v_cache, bt.block_table, bt.seq_lens,
                                    b["idx"])
    check_outputs(b["out"], o_own, bt.dtype, what="sketch step out on own indices")
    check_lse(b["lse"], l_own, bt.dtype)
    c = counts.cpu().float()
    _say(f"[sketch-step]   ok {label}: {st['units']} units, {st['strict']} strict, "
         f"candidates mean {c.mean():.1f} max {int(c.max())}")


@pytest.mark.parametrize("kernel_mode", ["auto", "unit"], indirect=True)
@pytest.mark.parametrize("top_k", [32, 64, 100])
def test_sketch_step_keeps_exact_ties(top_k, kernel_mode):
    """Runs of exactly tied scores: every tied block stays a candidate and the
    lowest indices win, as in the full step."""
    bt = synth.make_tie_batch(seq_lens=[700, 2000, 4096, 333, 1500, 8000], top_k=top_k, seed=41)
    d = bt.to(DEV)
    prob = btk.make_problem(d.q, d.k_cache, d.block_table)
    cent = torch.zeros((bt.num_pages, bt.num_kv_heads, bt.head_dim), device=DEV)
    ws = btk.new_workspace(prob, top_k, DEV)
    btk.btk_centroid_update(d.k_cache, d.block_table, d.seq_lens, cent, problem=prob)
    sketch = btk.new_sketch(prob, DEV)
    btk.btk_sketch_update(cent, d.block_table, d.seq_lens, sketch, ws, problem=prob)
    a, b = _run_both(d, prob, top_k, cent.clone(), cent.clone(), sketch, None)
    _assert_same(a, b)
    ora = oracle.sparse_step(bt.q, bt.k_cache, bt.v_cache, bt.block_table, bt.seq_lens, top_k)
    check_indices(b["idx"], ora["indices"], ora["scores"], bt.seq_lens, top_k,
                  sum_units=sum_factor(bt.group, bt.head_dim))


@pytest.mark.parametrize("label,spec,kernel_mode",
                         [CASES[2] + ("auto",), CASES[2] + ("persistent",), CASES[7] + ("auto",)],
                         ids=["config3", "config3-persistent", "config5-64k"],
                         indirect=["kernel_mode"])
def test_sketch_step_with_a_sketch_never_built(label, spec, kernel_mode):
    """An all-zero sketch names no page: every block is a candidate (units of up
    to 1024 blocks are scored exactly from LDS, longer ones by the full scan),
    with the same results."""
    bt = _batch(label, spec)
    _say(f"[sketch-step] never built: {label}")
    d = bt.to(DEV)
    prob = btk.make_problem(d.q, d.k_cache, d.block_table)
    k = bt.top_k
    first = (d.seq_lens - 1).to(torch.int32)
    _, stale = _stale_centroids(bt)
    sketch = btk.new_sketch(prob, DEV)
    counts = torch.zeros((bt.batch, bt.num_kv_heads), dtype=torch.int32, device=DEV)
    a, b = _run_both(d, prob, k, stale.to(DEV), stale.to(DEV), sketch, first, counts=counts)
    _assert_same(a, b)
    nb = torch.tensor(n_blocks(bt.seq_lens))[:, None].expand(-1, bt.num_kv_heads)
    assert torch.equal(counts.cpu(), torch.where(nb <= k, torch.zeros_like(nb), nb).to(torch.int32))


@pytest.mark.parametrize("kernel_mode", ["auto", "unit"], indirect=True)
def test_sketch_step_flags_invalid_lengths_and_pages_like_the_step(kernel_mode):
    bt = synth.make_batch(name="sketch-guards", batch=5, num_q_heads=8, num_kv_heads=2,
                          head_dim=128, seq_lens=[700, 40, 2500, 300, 900], top_k=8, seed=41)
    _say("[sketch-step] invalid lengths and pages")
    d = bt.to(DEV)
    prob = btk.make_problem(d.q, d.k_cache, d.block_table)
    cent = torch.zeros((bt.num_pages, 2, 128), device=DEV)
    ws = btk.new_workspace(prob, bt.top_k, DEV)
    btk.btk_centroid_update(d.k_cache, d.block_table, d.seq_lens, cent, problem=prob)
    sketch = btk.new_sketch(prob, DEV)
    btk.btk_sketch_update(cent, d.block_table, d.seq_lens, sketch, ws, problem=prob)
    sl = d.seq_lens.clone()
    sl[1] = 0
    sl[3] = bt.max_blocks * 16 + 1
    table = d.block_table.clone()
    table[4, 5] = bt.num_pages + 7
    first = (sl - 1).clamp(min=0).to(torch.int32)
    dd = synth.Batch(**dict(d.__dict__))
    dd.seq_lens, dd.block_table = sl, table
    a, b = _run_both(dd, prob, bt.top_k, cent.clone(), cent.clone(), sketch, first)
    assert a["err"] == b["err"] == 1 | 2
    _assert_same(a, b, units=[0, 2, 4])
    assert (b["idx"][1] == -1).all() and (b["idx"][3] == -1).all()
    assert not (b["idx"][4] == 5).any()  # the bad page's block is never selected


@pytest.mark.parametrize("kernel_mode", ["auto", "unit"], indirect=True)
def test_sketch_step_three_decode_steps_on_one_sketch(kernel_mode):
    """Three decode steps in a row, each appending a token: the sketch is built
    once before the first and then kept current only by the sketched step; every
    step's results equal the full step's on the same caches."""
    # lengths whose next three tokens stay in the same block (no new page needed)
    lens = [1 + (i * 977) % 6000 for i in range(24)]
    lens = [L - ((L - 1) % 16) + (i % 13) for i, L in enumerate(lens)]
    bt = synth.make_batch(name="three-steps", batch=24, num_q_heads=16, num_kv_heads=4,
                          head_dim=128, seq_lens=lens, top_k=16, seed=52)
    d = bt.to(DEV)
    prob = btk.make_problem(d.q, d.k_cache, d.block_table)
    k = bt.top_k
    cent_a = torch.zeros((bt.num_pages, bt.num_kv_heads, bt.head_dim), device=DEV)
    ws = btk.new_workspace(prob, k, DEV)
    btk.btk_centroid_update(d.k_cache, d.block_table, d.seq_lens, cent_a, problem=prob)
    cent_b = cent_a.clone()
    sketch = btk.new_sketch(prob, DEV)
    btk.btk_sketch_update(cent_b, d.block_table, d.seq_lens, sketch, ws, problem=prob)
    ws_a, ws_b = btk.new_workspace(prob, k, DEV), btk.new_workspace(prob, k, DEV)
    sl = d.seq_lens.clone()
    B, H = bt.batch, bt.num_kv_heads
    heads = torch.arange(H, device=DEV)[None, :]
    for step in range(3):
        sl = sl + 1  # one more token per sequence, written into its slot
        k_new, v_new = synth.make_new_tokens(bt, seed=60 + step)
        L = sl.long()
        page = d.block_table[torch.arange(B, device=DEV), (L - 1) // 16].long()[:, None]
        slot = ((L - 1) % 16)[:, None]
        d.k_cache[page, heads, slot, :] = k_new.to(DEV)
        d.v_cache[page, heads, :, slot] = v_new.to(DEV)
        dd = synth.Batch(**dict(d.__dict__))
        dd.seq_lens = sl.to(torch.int32)
        first = (dd.seq_lens - 1).to(torch.int32)
        a, b = _run_both(dd, prob, k, cent_a, cent_b, sketch, first, ws_a=ws_a, ws_b=ws_b)
        assert a["err"] == 0
        _assert_same(a, b)
        _say(f"[sketch-step] decode step {step}: equal")
    # the last step against the oracle
    host = synth.Batch(**dict(bt.__dict__))
    host.k_cache, host.v_cache, host.seq_lens = d.k_cache.cpu(), d.v_cache.cpu(), sl.cpu().to(torch.int32)
    ora = oracle.sparse_step(host.q, host.k_cache, host.v_cache, host.block_table, host.seq_lens, k)
    st = check_indices(b["idx"], ora["indices"], ora["scores"], host.seq_lens, k,
                       sum_units=sum_factor(bt.group, bt.head_dim))
    check_outputs(b["out"], ora["out"], bt.dtype, st["equal_mask"], bt.group)
