"""btk_select_sketch against btk_select (bit for bit) and the oracle, on the GPU.

The sketch may only change which fp32 centroid rows are read, never the
selection, so every case compares the two calls' index rows exactly, on the same
inputs and centroids, and the sketch path against the oracle under the margin
rule.  Covered: the five workloads (the 32B sweep 8K-64K), ragged and edge
shapes (single token, k >= n_b, D=64, fp32, group sizes 1 and 16, 8192 blocks),
runs of exactly tied scores, a sketch never built (all zeros), a sketch whose
rows name other pages (the table relabelled after it was built), and a decode
step (new token written, the touched pages' centroids and sketch rows updated).
"""
import pytest
import torch

import block_top_sparse_btk_amd as btk
import oracle
import synth
from parity import check_indices, sum_factor

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)


def _both(bt, top_k=None, sketch=None, build=True, cent=None):
    """(btk_select indices, btk_select_sketch indices, device state) on one batch."""
    top_k = top_k or bt.top_k
    d = bt.to(DEV)
    prob = btk.make_problem(d.q, d.k_cache, d.block_table)
    ws = btk.new_workspace(prob, top_k, DEV)
    if cent is None:
        cent = torch.zeros((bt.num_pages, bt.num_kv_heads, bt.head_dim), dtype=torch.float32,
                           device=DEV)
        btk.btk_centroid_update(d.k_cache, d.block_table, d.seq_lens, cent, problem=prob)
    if sketch is None:
        sketch = btk.new_sketch(prob, DEV)
    if build:
        btk.btk_sketch_update(cent, d.block_table, d.seq_lens, sketch, ws, problem=prob)
    i1 = btk.btk_select(d.q, cent, d.block_table, d.seq_lens, top_k, ws, problem=prob)
    i2 = btk.btk_select_sketch(d.q, cent, sketch, d.block_table, d.seq_lens, top_k, ws,
                               problem=prob)
    torch.cuda.synchronize()
    assert btk.workspace_error_bits(ws) == 0
    return i1.cpu(), i2.cpu(), (d, prob, ws, cent, sketch)


def _oracle_rule(bt, idx, top_k=None):
    top_k = top_k or bt.top_k
    ora = oracle.sparse_step(bt.q, bt.k_cache, bt.v_cache, bt.block_table, bt.seq_lens, top_k)
    return check_indices(idx, ora["indices"], ora["scores"], bt.seq_lens, top_k,
                         sum_units=sum_factor(bt.group, bt.head_dim))


WORKLOADS = [(1, None), (2, None), (3, None), (4, None), (5, 8192), (5, 16384), (5, 32768),
             (5, 65536)]


@pytest.mark.parametrize("cfg,ctx", WORKLOADS, ids=[f"config{c}" + (f"-{x}" if x else "")
                                                     for c, x in WORKLOADS])
def test_sketch_selection_equals_select_on_workloads(cfg, ctx):
    bt = synth.make_config(cfg, context=ctx)
    _say(f"[sketch] config {cfg} ctx={ctx}")
    i1, i2, _ = _both(bt)
    assert torch.equal(i1, i2)
    if cfg != 5 or ctx == 8192:  # the oracle on the smaller ones (the sweep's rows are alike)
        st = _oracle_rule(bt, i2)
        _say(f"[sketch]   oracle: {st['units']} units, {st['strict']} strict, {st['differ']} differ")


EDGE = [
    ("single-token", dict(batch=3, num_q_heads=4, num_kv_heads=2, head_dim=128, seq_lens=[1, 1, 1],
                          top_k=4)),
    ("k-exceeds-blocks", dict(batch=3, num_q_heads=8, num_kv_heads=4, head_dim=128,
                              seq_lens=[40, 200, 16], top_k=20)),
    ("ragged-tail", dict(batch=5, num_q_heads=8, num_kv_heads=1, head_dim=128,
                         seq_lens=[4097, 9000, 12345, 70, 2049], top_k=33)),
    ("group-1", dict(batch=4, num_q_heads=4, num_kv_heads=4, head_dim=128,
                     seq_lens=[500, 777, 1024, 3], top_k=7)),
    ("group-16", dict(batch=2, num_q_heads=32, num_kv_heads=2, head_dim=128, seq_lens=[1500, 999],
                      top_k=12)),
    ("d64-bf16", dict(batch=4, num_q_heads=8, num_kv_heads=2, head_dim=64,
                      seq_lens=[300, 1, 1025, 64], top_k=5)),
    ("d128-fp32", dict(batch=3, num_q_heads=6, num_kv_heads=2, head_dim=128,
                       seq_lens=[333, 48, 1000], top_k=6, dtype=torch.float32)),
    ("d64-fp32-heavy", dict(batch=3, num_q_heads=4, num_kv_heads=1, head_dim=64,
                            seq_lens=[2000, 100, 513], top_k=9, dtype=torch.float32,
                            heavy_frac=0.1)),
    ("shared-prefix", dict(batch=4, num_q_heads=8, num_kv_heads=1, head_dim=128,
                           seq_lens=[300, 290, 512, 257], top_k=10, table="shared",
                           shared_prefix=256)),
    ("long-8k-blocks", dict(batch=1, num_q_heads=2, num_kv_heads=1, head_dim=128,
                            seq_lens=[131072], top_k=64, spare_pages=3, max_blocks=8192)),
]


@pytest.mark.parametrize("label,kw", EDGE, ids=[e[0] for e in EDGE])
def test_sketch_selection_equals_select_on_edge_shapes(label, kw):
    bt = synth.make_batch(name=label, seed=77, **kw)
    _say(f"[sketch] {label}")
    i1, i2, _ = _both(bt)
    assert torch.equal(i1, i2)
    _oracle_rule(bt, i2)


@pytest.mark.parametrize("top_k", [32, 64, 100])
def test_sketch_selection_keeps_exact_ties(top_k):
    """Runs of blocks whose scores tie exactly: the sketch must keep every tied
    block as a candidate, and the lowest indices win as in btk_select."""
    lens = [700, 2000, 4096, 333, 1500, 8000]
    bt = synth.make_tie_batch(seq_lens=lens, top_k=top_k, seed=41)
    i1, i2, _ = _both(bt)
    assert torch.equal(i1, i2)


def test_sketch_never_built_and_rows_of_other_pages():
    """An all-zero sketch names no page: every block is a candidate.  A sketch
    built for another table (pages relabelled afterwards) names other pages:
    those rows are ignored.  Both give btk_select's indices."""
    bt = synth.make_config(3)
    i1, i2, _ = _both(bt, build=False)
    assert torch.equal(i1, i2)
    # build on the original table, then relabel pages: same contents, new ids
    d = bt.to(DEV)
    prob = btk.make_problem(d.q, d.k_cache, d.block_table)
    ws = btk.new_workspace(prob, bt.top_k, DEV)
    cent = torch.zeros((bt.num_pages, bt.num_kv_heads, bt.head_dim), device=DEV)
    btk.btk_centroid_update(d.k_cache, d.block_table, d.seq_lens, cent, problem=prob)
    sketch = btk.new_sketch(prob, DEV)
    btk.btk_sketch_update(cent, d.block_table, d.seq_lens, sketch, ws, problem=prob)
    g = torch.Generator().manual_seed(5)
    perm = torch.randperm(bt.num_pages, generator=g)  # new id of every page
    inv = torch.argsort(perm)
    moved = synth.Batch(**dict(bt.__dict__))
    moved.k_cache = bt.k_cache[inv]
    moved.v_cache = bt.v_cache[inv]
    moved.block_table = perm[bt.block_table.long()].to(torch.int32)
    cent_moved = cent[inv.to(DEV)]
    j1, j2, _ = _both(moved, sketch=sketch, build=False, cent=cent_moved)
    assert torch.equal(j1, j2)
    assert torch.equal(j1, i1)  # relabelling pages changes nothing


def test_sketch_decode_update_of_touched_pages():
    """A decode step: the newest token of every sequence is written, the touched
    pages' centroids and sketch rows are updated (first_pos), and the sketch
    selection equals btk_select on the updated centroids."""
    bt = synth.make_config(3)
    d = bt.to(DEV)
    prob = btk.make_problem(d.q, d.k_cache, d.block_table)
    ws = btk.new_workspace(prob, bt.top_k, DEV)
    cent = torch.zeros((bt.num_pages, bt.num_kv_heads, bt.head_dim), device=DEV)
    btk.btk_centroid_update(d.k_cache, d.block_table, d.seq_lens, cent, problem=prob)
    sketch = btk.new_sketch(prob, DEV)
    btk.btk_sketch_update(cent, d.block_table, d.seq_lens, sketch, ws, problem=prob)
    # a new token (scaled up so that the touched blocks' scores move a lot)
    k_new, v_new = synth.make_new_tokens(bt, seed=91, scale=4.0)
    bt2 = synth.write_tokens(bt, k_new, v_new)
    d2 = bt2.to(DEV)
    first = (d2.seq_lens - 1).to(torch.int32)
    btk.btk_centroid_update(d2.k_cache, d2.block_table, d2.seq_lens, cent, first_pos=first,
                            problem=prob)
    btk.btk_sketch_update(cent, d2.block_table, d2.seq_lens, sketch, ws, first_pos=first,
                          problem=prob)
    i1 = btk.btk_select(d2.q, cent, d2.block_table, d2.seq_lens, bt.top_k, ws, problem=prob)
    i2 = btk.btk_select_sketch(d2.q, cent, sketch, d2.block_table, d2.seq_lens, bt.top_k, ws,
                               problem=prob)
    torch.cuda.synchronize()
    assert btk.workspace_error_bits(ws) == 0
    assert torch.equal(i1.cpu(), i2.cpu())
    _oracle_rule(bt2, i2.cpu())
