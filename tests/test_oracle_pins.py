"""Pins for the CPU oracle: every check here fixes the oracle to something other
than itself -- a hand-worked example, closed forms, brute force over subsets,
library routines (numpy mean, torch.mv, scaled_dot_product_attention,
logsumexp, lexsort, bf16 casting) and invariants of the method.

Method: Pith review of "Kinetics: Rethinking Test-Time Scaling Laws", section
"What carries the argument" (averaged-key block summaries, per-query-group
scoring, top-k blocks, attention over the kept blocks).
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _closed(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, {"exp": math.exp, "log": math.log}))


def _handworked():
    with open(os.path.join(GOLDEN, "handworked_tiny.json")) as f:
        fx = json.load(f)
    P, D = fx["page_size"], 2
    k = torch.tensor(fx["k_tokens"], dtype=torch.float32).reshape(3, 1, P, D)
    v = torch.tensor(fx["v_tokens"], dtype=torch.float32).reshape(3, 1, P, D)
    v = v.permute(0, 1, 3, 2).contiguous()  # dim-major pages
    q = torch.tensor(fx["q"], dtype=torch.float32).reshape(1, 2, D)
    bt = torch.tensor([[0, 1, 2]], dtype=torch.int32)
    sl = torch.tensor([fx["seq_len"]], dtype=torch.int32)
    return fx, q, k, v, bt, sl


# ---------------------------------------------------------------- golden example

def test_handworked_example():
    fx, q, k, v, bt, sl = _handworked()
    ex = fx["expected"]
    cents = oracle.centroids(k, bt, sl)
    assert cents[:, 0, :].tolist() == ex["centroids"]
    sc = oracle.scores(q, cents, bt, sl, page_size=2, sm_scale=fx["sm_scale"])
    assert sc[0, 0, :3].tolist() == ex["scores"]
    idx = oracle.select(sc, sl, fx["top_k"], page_size=2)
    assert idx[0, 0].tolist() == ex["indices"]
    out, lse, w = oracle.attend(q, k, v, bt, sl, idx, sm_scale=fx["sm_scale"], want_weights=True)
    want = torch.tensor([[_closed(e) for e in row] for row in ex["sparse_out"]])
    assert torch.allclose(out[0].double(), want.double(), atol=1e-6, rtol=0)
    want_lse = torch.tensor([_closed(e) for e in ex["sparse_lse"]])
    assert torch.allclose(lse[0].double(), want_lse.double(), atol=1e-6, rtol=0)
    assert float(w[0, 0, 4:].abs().sum()) == 0.0  # block 2 not attended
    dout, dlse, _ = oracle.attend(q, k, v, bt, sl, None, sm_scale=fx["sm_scale"])
    want = torch.tensor([[_closed(e) for e in row] for row in ex["dense_out"]])
    assert torch.allclose(dout[0].double(), want.double(), atol=1e-6, rtol=0)
    want_lse = torch.tensor([_closed(e) for e in ex["dense_lse"]])
    assert torch.allclose(dlse[0].double(), want_lse.double(), atol=1e-6, rtol=0)


# ---------------------------------------------------------------- centroids

def _small(dtype=torch.float32, **kw):
    args = dict(batch=3, num_q_heads=4, num_kv_heads=2, head_dim=8, seq_lens=[37, 16, 5],
                top_k=2, dtype=dtype, seed=7, table="shuffled")
    args.update(kw)
    return synth.make_batch(**args)


def _keys_of(b, seq, g):
    """Valid keys of a sequence in logical order, float64 [L, D]."""
    P, L = b.page_size, int(b.seq_lens[seq])
    rows = []
    for j in range((L + P - 1) // P):
        page = int(b.block_table[seq, j])
        v = min(P, L - j * P)
        rows.append(b.k_cache[page, g, :v, :].double())
    return torch.cat(rows)


def _values_of(b, seq, g):
    P, L = b.page_size, int(b.seq_lens[seq])
    rows = []
    for j in range((L + P - 1) // P):
        page = int(b.block_table[seq, j])
        v = min(P, L - j * P)
        rows.append(b.v_cache[page, g, :, :v].double().T)
    return torch.cat(rows)


def test_centroid_of_identical_keys_is_that_key():
    b = _small()
    page = int(b.block_table[0, 0])
    b.k_cache[page, 1] = b.k_cache[page, 1, 3]  # all 16 keys equal one key
    c = oracle.centroids(b.k_cache, b.block_table, b.seq_lens)
    assert torch.equal(c[page, 1], b.k_cache[page, 1, 3])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_centroid_equals_numpy_mean_and_sum_identity(dtype):
    b = _small(dtype=dtype, seq_lens=[37, 33, 1], head_dim=16)
    c = oracle.centroids(b.k_cache, b.block_table, b.seq_lens)
    P = b.page_size
    for s in range(b.batch):
        L = int(b.seq_lens[s])
        for g in range(b.num_kv_heads):
            total = np.zeros(b.head_dim)
            for j in range((L + P - 1) // P):
                page = int(b.block_table[s, j])
                v = min(P, L - j * P)
                keys = b.k_cache[page, g, :v].double().numpy()
                ref = np.mean(keys, axis=0).astype(np.float32)
                np.testing.assert_allclose(c[page, g].numpy(), ref, rtol=2e-7, atol=1e-7)
                total += v * c[page, g].double().numpy()
            # sum_j v_j c_j equals the sum of all keys (fp32 rounding of c only)
            allk = _keys_of(b, s, g).sum(0).numpy()
            np.testing.assert_allclose(total, allk, rtol=1e-6, atol=1e-5)


def test_centroid_ignores_unused_slots_and_unreferenced_pages():
    b = _small(seq_lens=[37, 16, 5])
    c1 = oracle.centroids(b.k_cache, b.block_table, b.seq_lens)
    k2 = b.k_cache.clone()
    last = int(b.block_table[0, 2])  # L=37 -> block 2 holds 5 valid tokens
    k2[last, :, 5:, :] = -1234.0
    c2 = oracle.centroids(k2, b.block_table, b.seq_lens)
    assert torch.equal(c1, c2)


def test_centroid_touched_pages_only():
    b = _small(seq_lens=[37, 16, 5])
    sentinel = torch.full((b.num_pages, b.num_kv_heads, b.head_dim), 7.0)
    first = torch.tensor([36, 15, 0], dtype=torch.int32)  # newest token of each sequence
    c = oracle.centroids(b.k_cache, b.block_table, b.seq_lens, first_pos=first, out=sentinel.clone())
    full = oracle.centroids(b.k_cache, b.block_table, b.seq_lens)
    touched = {int(b.block_table[0, 2]), int(b.block_table[1, 0]), int(b.block_table[2, 0])}
    for p in range(b.num_pages):
        if p in touched:
            assert torch.equal(c[p], full[p])
        else:
            assert torch.equal(c[p], sentinel[p])


def _relabel(b, seed=3):
    """Same logical batch with the physical pages renumbered."""
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(b.num_pages, generator=g)
    k2 = torch.empty_like(b.k_cache)
    v2 = torch.empty_like(b.v_cache)
    k2[perm] = b.k_cache
    v2[perm] = b.v_cache
    bt2 = perm[b.block_table.long()].to(torch.int32)
    return k2, v2, bt2, perm


def test_page_relabelling_changes_nothing_logical():
    b = _small(seq_lens=[37, 16, 5])
    c = oracle.centroids(b.k_cache, b.block_table, b.seq_lens)
    k2, v2, bt2, perm = _relabel(b)
    c2 = oracle.centroids(k2, bt2, b.seq_lens)
    assert torch.equal(c2[perm], c)
    s1 = oracle.scores(b.q, c, b.block_table, b.seq_lens)
    s2 = oracle.scores(b.q, c2, bt2, b.seq_lens)
    assert torch.equal(torch.nan_to_num(s1, nan=-9.0), torch.nan_to_num(s2, nan=-9.0))
    o1, l1, _ = oracle.attend(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens)
    o2, l2, _ = oracle.attend(b.q, k2, v2, bt2, b.seq_lens)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---------------------------------------------------------------- scores

def test_scores_with_one_head_per_group_are_a_gemv():
    b = _small(num_q_heads=2, num_kv_heads=2)
    c = oracle.centroids(b.k_cache, b.block_table, b.seq_lens)
    s = oracle.scores(b.q, c, b.block_table, b.seq_lens)
    scale = 1.0 / math.sqrt(b.head_dim)
    for seq in range(b.batch):
        nb = int(b.n_blocks()[seq])
        for g in range(2):
            pages = b.block_table[seq, :nb].long()
            ref = torch.mv(c[pages, g].double(), b.q[seq, g].double()) * scale
            assert torch.allclose(s[seq, g, :nb].double(), ref.float().double(), rtol=0, atol=1e-7)


def test_group_score_equals_mean_query_form():
    b = _small(num_q_heads=8, num_kv_heads=2, head_dim=16)
    c = oracle.centroids(b.k_cache, b.block_table, b.seq_lens)
    s = oracle.scores(b.q, c, b.block_table, b.seq_lens)
    r = b.group
    for seq in range(b.batch):
        nb = int(b.n_blocks()[seq])
        for g in range(2):
            qbar = b.q[seq, g * r:(g + 1) * r].double().mean(0)
            pages = b.block_table[seq, :nb].long()
            ref = (c[pages, g].double() @ qbar) / math.sqrt(b.head_dim)
            assert torch.allclose(s[seq, g, :nb].double(), ref, rtol=0, atol=1e-6)


def test_scores_explicit_scale_and_head_order():
    b = _small(num_q_heads=4, num_kv_heads=2)
    c = oracle.centroids(b.k_cache, b.block_table, b.seq_lens)
    s_def = oracle.scores(b.q, c, b.block_table, b.seq_lens)
    s_exp = oracle.scores(b.q, c, b.block_table, b.seq_lens, sm_scale=1.0 / math.sqrt(b.head_dim))
    assert torch.equal(torch.nan_to_num(s_def), torch.nan_to_num(s_exp))
    s_two = oracle.scores(b.q, c, b.block_table, b.seq_lens, sm_scale=2.0 / math.sqrt(b.head_dim))
    m = ~torch.isnan(s_def)
    assert torch.allclose(s_two[m].double(), 2 * s_def[m].double(), rtol=1e-6, atol=0)
    q2 = b.q[:, [1, 0, 3, 2]]  # swap heads inside each group of two
    s_sw = oracle.scores(q2, c, b.block_table, b.seq_lens)
    assert torch.allclose(s_sw[m], s_def[m], rtol=0, atol=1e-7)
    q3 = b.q[:, [2, 3, 0, 1]]  # swap whole groups -> groups swap
    s_g = oracle.scores(q3, c, b.block_table, b.seq_lens)
    assert not torch.allclose(s_g[m], s_def[m])


# ---------------------------------------------------------------- selection

def _brute_topk(s, k):
    """Best subset by exact total score; ties -> lexicographically smallest tuple."""
    n = len(s)
    kb = min(k, n)
    best, best_sum = None, None
    for sub in itertools.combinations(range(n), kb):
        tot = sum(Fraction(float(s[j])) for j in sub)
        if best is None or tot > best_sum or (tot == best_sum and sub < best):
            best, best_sum = sub, tot
    return list(best) + [-1] * (k - kb)


def test_selection_equals_exhaustive_enumeration():
    g = torch.Generator().manual_seed(11)
    P = 16
    for trial in range(300):
        n = int(torch.randint(1, 13, (1,), generator=g))
        k = int(torch.randint(1, 5, (1,), generator=g))
        # few distinct values so ties are common
        vals = torch.tensor([-1.5, -0.25, 0.0, 0.125, 0.5, 2.0])
        s = vals[torch.randint(0, len(vals), (n,), generator=g)]
        if trial % 3 == 0:
            s = torch.randn(n, generator=g)
        score = torch.full((1, 1, 16), float("nan"))
        score[0, 0, :n] = s
        sl = torch.tensor([n * P - int(torch.randint(0, P, (1,), generator=g))], dtype=torch.int32)
        idx = oracle.select(score, sl, k)
        assert idx[0, 0].tolist() == _brute_topk(s.tolist(), k), (s.tolist(), k)


def test_selection_matches_lexsort_on_large_inputs():
    g = torch.Generator().manual_seed(12)
    B, H, MB = 4, 3, 700
    score = torch.randn((B, H, MB), generator=g)
    score = torch.round(score * 64) / 64  # many exact ties
    sl = torch.tensor([700 * 16, 5000, 17, 1], dtype=torch.int32)
    for k in (1, 7, 64):
        idx = oracle.select(score, sl, k)
        for b in range(B):
            nb = (int(sl[b]) + 15) // 16
            for h in range(H):
                s = score[b, h, :nb].numpy()
                order = np.lexsort((np.arange(nb), -s))  # key: -s, then index
                want = sorted(order[:min(k, nb)].tolist()) + [-1] * max(0, k - nb)
                assert idx[b, h].tolist() == want


def test_signed_zero_scores_tie_and_lower_index_wins():
    score = torch.tensor([[[0.0, -0.0, -1.0, -0.0, 0.0]]])
    sl = torch.tensor([5 * 16], dtype=torch.int32)
    assert oracle.select(score, sl, 2)[0, 0].tolist() == [0, 1]
    score = torch.tensor([[[-0.0, -1.0, 0.0, -0.0, 0.0]]])
    assert oracle.select(score, sl, 3)[0, 0].tolist() == [0, 2, 3]


def test_k_at_least_blocks_selects_all_and_pads():
    score = torch.randn((1, 2, 8))
    sl = torch.tensor([50], dtype=torch.int32)  # 4 blocks
    idx = oracle.select(score, sl, 6)
    assert idx[0, 0].tolist() == [0, 1, 2, 3, -1, -1]
    assert idx[0, 1].tolist() == [0, 1, 2, 3, -1, -1]


def test_block_aligned_with_the_group_query_is_selected():
    b = _small(num_q_heads=4, num_kv_heads=2, head_dim=16, seq_lens=[200, 150, 90])
    r = b.group
    for seq in range(b.batch):
        for g in range(2):
            qbar = b.q[seq, g * r:(g + 1) * r].float().mean(0)
            j = int(torch.randint(0, int(b.n_blocks()[seq]), (1,)))
            page = int(b.block_table[seq, j])
            b.k_cache[page, g] += 50.0 * qbar / qbar.norm()
            st = oracle.sparse_step(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, 1)
            assert st["indices"][seq, g, 0].item() == j


# ---------------------------------------------------------------- attention

def _sdpa_ref(b, seq, h, blocks=None):
    """scaled_dot_product_attention in float64 on the gathered tokens."""
    P, L = b.page_size, int(b.seq_lens[seq])
    g = h // b.group
    keys, vals = _keys_of(b, seq, g), _values_of(b, seq, g)
    if blocks is not None:
        pos = torch.cat([torch.arange(j * P, min(L, j * P + P)) for j in blocks])
        keys, vals = keys[pos], vals[pos]
    qh = b.q[seq, h].double().reshape(1, 1, 1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(
        qh, keys.reshape(1, 1, -1, b.head_dim), vals.reshape(1, 1, -1, b.head_dim))
    logits = (keys @ b.q[seq, h].double()) / math.sqrt(b.head_dim)
    return out.reshape(-1), torch.logsumexp(logits, 0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_dense_equals_sdpa_and_logsumexp(dtype):
    b = _small(dtype=dtype, seq_lens=[37, 16, 1], head_dim=16)
    out, lse, w = oracle.attend(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens,
                                want_weights=True)
    for seq in range(b.batch):
        for h in range(b.num_q_heads):
            ref, ref_lse = _sdpa_ref(b, seq, h)
            assert torch.allclose(out[seq, h].double(), ref, rtol=0, atol=2e-7)
            assert abs(float(lse[seq, h]) - float(ref_lse)) < 1e-5
            assert abs(float(w[seq, h].sum()) - 1.0) < 1e-12


def test_sparse_equals_sdpa_on_the_selected_blocks():
    b = _small(seq_lens=[120, 64, 33], head_dim=16, top_k=3)
    st = oracle.sparse_step(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, 3)
    _, _, w = oracle.attend(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens,
                            st["indices"], want_weights=True)
    for seq in range(b.batch):
        for h in range(b.num_q_heads):
            blocks = [j for j in st["indices"][seq, h // b.group].tolist() if j >= 0]
            ref, ref_lse = _sdpa_ref(b, seq, h, blocks)
            assert torch.allclose(st["out"][seq, h].double(), ref, rtol=0, atol=2e-7)
            assert abs(float(st["lse"][seq, h]) - float(ref_lse)) < 1e-5
            assert abs(float(w[seq, h].sum()) - 1.0) < 1e-12
            on = set(blocks)
            for j in range((int(b.seq_lens[seq]) + 15) // 16):
                mass = float(w[seq, h, j * 16:(j + 1) * 16].sum())
                assert (mass > 0) == (j in on)


def test_all_blocks_selected_equals_dense_exactly():
    b = _small(seq_lens=[37, 16, 5])
    st = oracle.sparse_step(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, 64)
    dout, dlse, _ = oracle.attend(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens)
    assert torch.equal(st["out"], dout) and torch.equal(st["lse"], dlse)


def test_constant_values_give_that_value():
    b = _small(seq_lens=[37, 16, 5])
    const = torch.randn(b.num_kv_heads, b.head_dim)
    b.v_cache[:] = const.reshape(1, b.num_kv_heads, b.head_dim, 1)
    st = oracle.sparse_step(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, 2)
    for h in range(b.num_q_heads):
        assert torch.allclose(st["out"][:, h], const[h // b.group].expand(b.batch, -1), atol=1e-6)


def test_single_token_context_returns_its_value():
    b = _small(seq_lens=[1, 1, 1])
    out, lse, _ = oracle.attend(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens)
    for seq in range(3):
        for h in range(b.num_q_heads):
            page = int(b.block_table[seq, 0])
            assert torch.equal(out[seq, h], b.v_cache[page, h // b.group, :, 0])
            logit = float(b.q[seq, h].double() @ b.k_cache[page, h // b.group, 0].double())
            assert abs(float(lse[seq, h]) - logit / math.sqrt(b.head_dim)) < 1e-6


def test_shared_prefix_with_identical_suffixes_gives_identical_outputs():
    b = synth.make_batch(batch=3, num_q_heads=4, num_kv_heads=2, head_dim=16,
                         seq_lens=[100, 100, 100], top_k=3, dtype=torch.float32, seed=5,
                         table="shared", shared_prefix=64)
    # make sequences 1 and 2 copy sequence 0's private pages and its queries
    for s in (1, 2):
        for j in range(4, 7):
            b.k_cache[int(b.block_table[s, j])] = b.k_cache[int(b.block_table[0, j])]
            b.v_cache[int(b.block_table[s, j])] = b.v_cache[int(b.block_table[0, j])]
        b.q[s] = b.q[0]
    st = oracle.sparse_step(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, 3)
    assert torch.equal(st["indices"][1], st["indices"][0])
    assert torch.equal(st["out"][1], st["out"][0]) and torch.equal(st["out"][2], st["out"][0])


def test_bad_indices_are_rejected():
    b = _small(seq_lens=[37, 16, 5])
    idx = torch.zeros((3, 2, 2), dtype=torch.int32)  # block 0 listed twice
    with pytest.raises(RuntimeError):
        oracle.attend(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, idx)
    idx = torch.tensor([[[0, 3]] * 2, [[0, -1]] * 2, [[0, -1]] * 2], dtype=torch.int32)
    with pytest.raises(RuntimeError):  # block 3 of a 37-token sequence does not exist
        oracle.attend(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, idx)


# ---------------------------------------------------------------- output rounding

def test_bf16_rounding_matches_torch_cast():
    g = torch.Generator().manual_seed(2)
    x = torch.randn(100000, generator=g) * 3
    # exact halfway cases between two bf16 values, both parities
    base = torch.randn(2000, generator=g).to(torch.bfloat16).float()
    half = (base.view(torch.int32) + 0x8000).view(torch.float32)
    x = torch.cat([x, half, torch.tensor([0.0, -0.0, 1e-40, 3.0e38, -3.0e38])])
    assert torch.equal(oracle.round_bf16(x).view(torch.int16), x.to(torch.bfloat16).view(torch.int16))


# ---------------------------------------------------------------- local-window baseline
# (scime summary of "Kinetics: Rethinking Test-Time Scaling Law", "Measured effects
# reported in the paper": local attention over the most recent KV replaces the top-k
# selection; the window is counted in whole blocks, like the top-k budget.)

@pytest.mark.parametrize("window", [1, 2, 3])
def test_local_window_is_the_most_recent_tokens_of_whole_blocks(window):
    b = _small(batch=4, seq_lens=[37, 16, 1, 50], head_dim=16)
    out, lse, w = oracle.local_attend(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens,
                                      window, want_weights=True)
    for seq in range(b.batch):
        L = int(b.seq_lens[seq])
        nb = (L + 15) // 16
        first = 16 * max(0, nb - window)  # the window starts on a block boundary
        for h in range(b.num_q_heads):
            g = h // b.group
            keys, vals = _keys_of(b, seq, g)[first:L], _values_of(b, seq, g)[first:L]
            qh = b.q[seq, h].double()
            ref = torch.nn.functional.scaled_dot_product_attention(
                qh.reshape(1, 1, 1, -1), keys.reshape(1, 1, -1, b.head_dim),
                vals.reshape(1, 1, -1, b.head_dim)).reshape(-1)
            ref_lse = torch.logsumexp((keys @ qh) / math.sqrt(b.head_dim), 0)
            assert torch.allclose(out[seq, h].double(), ref, rtol=0, atol=2e-7)
            assert abs(float(lse[seq, h]) - float(ref_lse)) < 1e-5
            mass = w[seq, h]
            assert float(mass[:first].abs().sum()) == 0.0
            assert abs(float(mass[first:L].sum()) - 1.0) < 1e-12


def test_local_window_covering_the_sequence_equals_dense_exactly():
    b = _small(seq_lens=[37, 16, 5])
    lout, llse, _ = oracle.local_attend(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, 3)
    dout, dlse, _ = oracle.attend(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens)
    assert torch.equal(lout, dout) and torch.equal(llse, dlse)


def test_local_indices_layout():
    idx = oracle.local_indices(torch.tensor([37, 16, 1, 200], dtype=torch.int32), 2, 4)
    assert idx.shape == (4, 2, 4)
    assert idx[0, 0].tolist() == [0, 1, 2, -1]
    assert idx[1, 1].tolist() == [0, -1, -1, -1]
    assert idx[2, 0].tolist() == [0, -1, -1, -1]
    assert idx[3, 0].tolist() == [9, 10, 11, 12]


# ---------------------------------------------------------------- token-level top-k
# (scime summary of "Kinetics: Rethinking Test-Time Scaling Law", "Experimental setup":
# oracle top-k attention is a baseline; "Limitations": the upper bound of the sparse results.)

def test_token_view_is_a_relabelling():
    b = _small(dtype=torch.bfloat16, seq_lens=[37, 16, 5], head_dim=16)
    k1, v1, tt = oracle.token_view(b.k_cache, b.v_cache, b.block_table)
    for seq in range(b.batch):
        L = int(b.seq_lens[seq])
        for g in range(b.num_kv_heads):
            rows = tt[seq, :L].long()
            assert torch.equal(k1[rows, g, 0, :].double(), _keys_of(b, seq, g))
            assert torch.equal(v1[rows, g, :, 0].double(), _values_of(b, seq, g))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_token_topk_scores_selection_and_attention(dtype):
    b = _small(dtype=dtype, batch=3, seq_lens=[70, 33, 9], head_dim=16)
    T = 12
    st = oracle.token_step(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, T)
    scale = 1.0 / math.sqrt(b.head_dim)
    for seq in range(b.batch):
        L = int(b.seq_lens[seq])
        for g in range(b.num_kv_heads):
            keys = _keys_of(b, seq, g)
            qs = b.q[seq, g * b.group:(g + 1) * b.group].double()
            want = (keys @ qs.T).mean(dim=1) * scale  # mean of the group's scaled logits
            got = st["scores"][seq, g, :L].double()
            assert torch.allclose(got, want, rtol=0, atol=1e-6)
            # selection: lexsort on (score desc, position asc) of the stored fp32 scores
            s32 = st["scores"][seq, g, :L].numpy()
            order = np.lexsort((np.arange(L), -s32.astype(np.float64)))[:min(T, L)]
            sel = sorted(order.tolist())
            idx = st["indices"][seq, g].tolist()
            assert idx[:len(sel)] == sel and all(x == -1 for x in idx[len(sel):])
            for h in range(g * b.group, (g + 1) * b.group):
                qh = b.q[seq, h].double()
                kk, vv = keys[sel], _values_of(b, seq, g)[sel]
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qh.reshape(1, 1, 1, -1), kk.reshape(1, 1, -1, b.head_dim),
                    vv.reshape(1, 1, -1, b.head_dim)).reshape(-1)
                assert torch.allclose(st["out"][seq, h].double(), ref, rtol=0, atol=2e-7)
                ref_lse = torch.logsumexp((kk @ qh) * scale, 0)
                assert abs(float(st["lse"][seq, h]) - float(ref_lse)) < 1e-5


def test_token_topk_covering_the_sequence_equals_dense():
    b = _small(seq_lens=[37, 16, 5])
    st = oracle.token_step(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, 64)
    dout, dlse, _ = oracle.attend(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens)
    assert torch.allclose(st["out"], dout, rtol=0, atol=1e-6)
    assert torch.allclose(st["lse"], dlse, rtol=0, atol=1e-6)


def test_token_topk_with_keys_constant_per_block_equals_block_topk():
    # every block's 16 keys equal: a block's tokens tie, so the top 16k tokens
    # are the tokens of the k best blocks, and the two baselines attend alike
    b = _small(batch=2, seq_lens=[160, 96], head_dim=16, top_k=3)
    b.k_cache[:] = b.k_cache[:, :, :1, :]
    k = 3
    blk = oracle.sparse_step(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, k)
    tok = oracle.token_step(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, 16 * k)
    for seq in range(b.batch):
        for g in range(b.num_kv_heads):
            blocks = blk["indices"][seq, g].tolist()
            want = [16 * j + t for j in blocks for t in range(16)]
            assert tok["indices"][seq, g].tolist() == want
    assert torch.allclose(tok["out"], blk["out"], rtol=0, atol=1e-6)
