"""GPU paths pinned directly to the CPU oracle (not only to another HIP path).

Covered here: the decode step with the KV append fused in (fresh tokens written
into the caches; caches, centroids, selection, outputs and lse against the
oracle run on CPU copies with the same tokens written in), the shared-prefix
(Best-of-N) selection against the oracle's scores and selection, and an explicit
softmax scale through every entry point that takes one.  Units whose selection
differs from the oracle's (near-ties under the margin rule) have their outputs
checked against the oracle's attention over the library's own indices.
"""
import pytest
import torch

import block_top_sparse_btk_amd as btk
import oracle
import synth
from parity import (CENTROID_TOL, SCORE_TOL, check_indices, check_lse, check_outputs, max_abs,
                    n_blocks, sum_factor)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)


def check_on_own_indices(bt, idx, out, lse, sm_scale=0.0):
    """Every unit's output and lse against the oracle's attention over the
    library's own selection (so units whose selection differs from the oracle's
    near a tie are checked too)."""
    o_ref, l_ref, _ = oracle.attend(bt.q, bt.k_cache, bt.v_cache, bt.block_table, bt.seq_lens,
                                    idx.cpu(), sm_scale=sm_scale)
    err = check_outputs(out.cpu(), o_ref, bt.dtype, what="out on own indices")
    check_lse(lse.cpu(), l_ref, bt.dtype)
    return err


# ------------------------------------------------------------------ fused KV append

APPEND_CASES = [
    ("config3", dict(cfg=3)),
    ("page-edges", dict(kw=dict(batch=6, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                seq_lens=[1, 16, 17, 33, 300, 5000], top_k=8, seed=141))),
    ("d64-fp32", dict(kw=dict(batch=3, num_q_heads=4, num_kv_heads=2, head_dim=64,
                              seq_lens=[100, 32, 999], top_k=5, seed=142, dtype=torch.float32))),
    ("group16", dict(kw=dict(batch=3, num_q_heads=32, num_kv_heads=2, head_dim=128,
                             seq_lens=[2049, 700, 48], top_k=12, seed=143))),
]


@pytest.mark.parametrize("label,spec", APPEND_CASES, ids=[c[0] for c in APPEND_CASES])
def test_decode_step_append_against_oracle(label, spec):
    """Fresh tokens (not the drawn ones) are appended by the fused step; the
    oracle runs the whole step on CPU caches with the same tokens written in."""
    bt = synth.make_config(spec["cfg"]) if "cfg" in spec else synth.make_batch(name=label,
                                                                               **spec["kw"])
    _say(f"[append-oracle] {label} B={bt.batch} lens[:4]={bt.seq_lens[:4].tolist()}")
    k_new, v_new = synth.make_new_tokens(bt, seed=bt.seed + 17)
    after = synth.write_tokens(bt, k_new, v_new)  # the caches the step must leave behind
    # centroids as the previous step left them: every page from the caches before
    # the append, the newest token's page stale
    cents = oracle.centroids(bt.k_cache, bt.block_table, bt.seq_lens)
    L = bt.seq_lens.long()
    touched = bt.block_table[torch.arange(bt.batch), (L - 1) // 16].long()
    stale = cents.clone()
    stale[touched] = float("nan")
    ora = oracle.sparse_step(after.q, after.k_cache, after.v_cache, after.block_table,
                             after.seq_lens, bt.top_k, cents=cents.clone(),
                             first_pos=(bt.seq_lens - 1).to(torch.int32))
    d = bt.to(DEV)
    prob = btk.make_problem(d.q, d.k_cache, d.block_table)
    ws = btk.new_workspace(prob, bt.top_k, DEV)
    kc, vc, c = d.k_cache.clone(), d.v_cache.clone(), stale.to(DEV)
    lse = torch.empty((bt.batch, bt.num_q_heads), device=DEV)
    out, idx = btk.btk_decode_step_append(d.q, k_new.to(DEV), v_new.to(DEV), kc, vc,
                                          d.block_table, d.seq_lens, c, bt.top_k, ws, lse=lse,
                                          problem=prob)
    torch.cuda.synchronize()
    assert btk.workspace_error_bits(ws) == 0
    assert torch.equal(kc.cpu(), after.k_cache) and torch.equal(vc.cpu(), after.v_cache)
    c_err = max_abs(c.cpu(), ora["centroids"])
    assert c_err <= CENTROID_TOL, c_err
    st = check_indices(idx.cpu(), ora["indices"], ora["scores"], bt.seq_lens, bt.top_k,
                       sum_units=sum_factor(bt.group, bt.head_dim))
    o_err = check_outputs(out.cpu(), ora["out"], bt.dtype, st["equal_mask"], bt.group)
    check_lse(lse.cpu(), ora["lse"], bt.dtype, st["equal_mask"], bt.group)
    check_on_own_indices(after, idx, out, lse)
    _say(f"[append-oracle]   ok centroid={c_err:.2e} out={o_err:.2e} near_tie={st['near_tie']} "
         f"differ={st['differ']}")


# ------------------------------------------------------------------ shared-prefix selection

SHARED_CASES = [
    ("config4", dict(cfg=4, groups=([0, 16], [128]))),
    ("custom-groups", dict(kw=dict(batch=7, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                   seq_lens=[700, 512, 1000, 530, 2200, 600, 900], top_k=9,
                                   seed=161, table="shared", shared_prefix=512),
                           groups=([0, 2, 3, 5, 6], [32, 32, 7, 0]))),
    ("two-groups-d64", dict(kw=dict(batch=6, num_q_heads=8, num_kv_heads=1, head_dim=64,
                                    seq_lens=[4100, 4200, 3000, 3500, 5000, 2600], top_k=20,
                                    seed=162, table="shared", shared_prefix=2048),
                            groups=([0, 3, 6], [128, 128]))),
]


@pytest.mark.parametrize("label,spec", SHARED_CASES, ids=[c[0] for c in SHARED_CASES])
def test_shared_prefix_selection_against_oracle(label, spec):
    bt = synth.make_config(spec["cfg"]) if "cfg" in spec else synth.make_batch(name=label,
                                                                               **spec["kw"])
    starts, blocks = spec["groups"]
    _say(f"[shared-oracle] {label} groups={starts} prefix={blocks}")
    cents = oracle.centroids(bt.k_cache, bt.block_table, bt.seq_lens)
    o_sc = oracle.scores(bt.q, cents, bt.block_table, bt.seq_lens)
    o_idx = oracle.select(o_sc, bt.seq_lens, bt.top_k)
    d = bt.to(DEV)
    prob = btk.make_problem(d.q, d.k_cache, d.block_table)
    ws = btk.new_workspace(prob, bt.top_k, DEV)
    sc = torch.full((bt.batch, bt.num_kv_heads, bt.max_blocks), float("nan"), device=DEV)
    idx = btk.btk_select_shared(d.q, cents.to(DEV), d.block_table, d.seq_lens, starts, blocks,
                                bt.top_k, ws, scores=sc, problem=prob)
    torch.cuda.synchronize()
    assert btk.workspace_error_bits(ws) == 0
    s_err = 0.0
    for b, nb in enumerate(n_blocks(bt.seq_lens)):
        s_err = max(s_err, max_abs(sc[b, :, :nb].cpu(), o_sc[b, :, :nb]))
    assert s_err <= SCORE_TOL, s_err
    st = check_indices(idx.cpu(), o_idx, o_sc, bt.seq_lens, bt.top_k,
                       sum_units=sum_factor(bt.group, bt.head_dim))
    _say(f"[shared-oracle]   ok score={s_err:.2e} near_tie={st['near_tie']} differ={st['differ']}")


# ------------------------------------------------------------------ explicit softmax scale

SCALE_CASES = [
    ("config3-b8", dict(cfg=3, batch=8, scale=0.07)),
    ("d64-fp32", dict(kw=dict(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64,
                              seq_lens=[2000, 17, 640], top_k=9, seed=171, dtype=torch.float32),
                      scale=0.3)),
    ("group1-d128", dict(kw=dict(batch=4, num_q_heads=4, num_kv_heads=4, head_dim=128,
                                 seq_lens=[500, 777, 1024, 3], top_k=7, seed=172), scale=0.02)),
]


@pytest.mark.parametrize("label,spec", SCALE_CASES, ids=[c[0] for c in SCALE_CASES])
def test_explicit_sm_scale_against_oracle(label, spec, monkeypatch):
    """sm_scale > 0 scales the block scores and the attention logits of select,
    sparse/dense/local attention and the single-launch steps (the step through
    the sketches in both of its kernels must equal the step bit for bit)."""
    s = spec["scale"]
    if "cfg" in spec:
        bt = synth.make_config(spec["cfg"], batch=spec.get("batch"))
    else:
        bt = synth.make_batch(name=label, **spec["kw"])
    k = bt.top_k
    _say(f"[scale] {label} sm_scale={s}")
    first = (bt.seq_lens - 1).to(torch.int32)
    cents = oracle.centroids(bt.k_cache, bt.block_table, bt.seq_lens)
    ora = oracle.sparse_step(bt.q, bt.k_cache, bt.v_cache, bt.block_table, bt.seq_lens, k,
                             cents=cents.clone(), first_pos=first, sm_scale=s)
    sf = bt.group / s  # margin factor to the plain sum of the heads' unscaled dot products
    d = bt.to(DEV)
    prob = btk.make_problem(d.q, d.k_cache, d.block_table, sm_scale=s)
    ws = btk.new_workspace(prob, k, DEV)
    cd = cents.to(DEV)
    # select (scores exported) and sparse attention, as separate calls
    sc = torch.full((bt.batch, bt.num_kv_heads, bt.max_blocks), float("nan"), device=DEV)
    idx = btk.btk_select(d.q, cd, d.block_table, d.seq_lens, k, ws, scores=sc, problem=prob)
    lse = torch.empty((bt.batch, bt.num_q_heads), device=DEV)
    out = btk.btk_sparse_attend(d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens, idx, ws,
                                lse=lse, problem=prob)
    # dense and local
    dlse = torch.empty_like(lse)
    dout = btk.btk_dense_attend(d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens, ws,
                                lse=dlse, problem=prob)
    llse = torch.empty_like(lse)
    lout = btk.btk_local_attend(d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens, k, ws,
                                lse=llse, problem=prob)
    # the single-launch step (the newest page stale) and the step with the append
    stale = cents.clone()
    L = bt.seq_lens.long()
    stale[bt.block_table[torch.arange(bt.batch), (L - 1) // 16].long()] = float("nan")
    ws2 = btk.new_workspace(prob, k, DEV)
    c2 = stale.to(DEV)
    slse = torch.empty_like(lse)
    sout, sidx = btk.btk_decode_step(d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens, c2, k,
                                     ws2, first_pos=first.to(DEV), lse=slse, problem=prob)
    kn = d.k_cache[bt.block_table[torch.arange(bt.batch), (L - 1) // 16].long()[:, None].to(DEV),
                   torch.arange(bt.num_kv_heads, device=DEV)[None, :],
                   ((L - 1) % 16)[:, None].to(DEV), :].contiguous()
    vn = d.v_cache[bt.block_table[torch.arange(bt.batch), (L - 1) // 16].long()[:, None].to(DEV),
                   torch.arange(bt.num_kv_heads, device=DEV)[None, :], :,
                   ((L - 1) % 16)[:, None].to(DEV)].contiguous()
    ws3 = btk.new_workspace(prob, k, DEV)
    c3 = stale.to(DEV)
    kc, vc = d.k_cache.clone(), d.v_cache.clone()
    alse = torch.empty_like(lse)
    aout, aidx = btk.btk_decode_step_append(d.q, kn, vn, kc, vc, d.block_table, d.seq_lens, c3, k,
                                            ws3, lse=alse, problem=prob)
    # the step through the block sketches, built from the stale centroids, in the
    # library's choice of kernel and in the one-workgroup-per-unit kernel
    sk_runs = []
    for flags in ("0", "2"):
        monkeypatch.setenv("BTK_STEP_TEST_FLAGS", flags)
        sk = btk.new_sketch(prob, DEV)
        wsk = btk.new_workspace(prob, k, DEV)
        c4 = stale.to(DEV)
        btk.btk_sketch_update(c4, d.block_table, d.seq_lens, sk, wsk, problem=prob)
        klse = torch.empty_like(lse)
        kout, kidx = btk.btk_decode_step_sketch(d.q, d.k_cache, d.v_cache, d.block_table,
                                                d.seq_lens, c4, sk, k, wsk,
                                                first_pos=first.to(DEV), lse=klse, problem=prob)
        torch.cuda.synchronize()
        sk_runs.append((wsk, c4, kidx, kout, klse))
    monkeypatch.delenv("BTK_STEP_TEST_FLAGS")
    torch.cuda.synchronize()
    for w in (ws, ws2, ws3):
        assert btk.workspace_error_bits(w) == 0
    for wsk, c4, kidx, kout, klse in sk_runs:
        assert btk.workspace_error_bits(wsk) == 0
        assert torch.equal(kidx, sidx) and torch.equal(kout, sout) and torch.equal(klse, slse)
        assert torch.equal(c4, c2)
    s_err = 0.0
    for b, nb in enumerate(n_blocks(bt.seq_lens)):
        s_err = max(s_err, max_abs(sc[b, :, :nb].cpu(), ora["scores"][b, :, :nb]))
    assert s_err <= SCORE_TOL, s_err
    for name, i_, o_, l_ in (("select+attend", idx, out, lse), ("step", sidx, sout, slse),
                             ("step+append", aidx, aout, alse)):
        st = check_indices(i_.cpu(), ora["indices"], ora["scores"], bt.seq_lens, k,
                           sum_units=sf)
        check_outputs(o_.cpu(), ora["out"], bt.dtype, st["equal_mask"], bt.group, what=name)
        check_lse(l_.cpu(), ora["lse"], bt.dtype, st["equal_mask"], bt.group)
        check_on_own_indices(bt, i_, o_, l_, sm_scale=s)
    assert max_abs(c2.cpu(), ora["centroids"]) <= CENTROID_TOL
    assert max_abs(c3.cpu(), ora["centroids"]) <= CENTROID_TOL
    assert torch.equal(kc, d.k_cache) and torch.equal(vc, d.v_cache)
    do, dl, _ = oracle.attend(bt.q, bt.k_cache, bt.v_cache, bt.block_table, bt.seq_lens,
                              sm_scale=s)
    check_outputs(dout.cpu(), do, bt.dtype, what="dense out")
    check_lse(dlse.cpu(), dl, bt.dtype)
    lo, ll, _ = oracle.local_attend(bt.q, bt.k_cache, bt.v_cache, bt.block_table, bt.seq_lens, k,
                                    sm_scale=s)
    check_outputs(lout.cpu(), lo, bt.dtype, what="local out")
    check_lse(llse.cpu(), ll, bt.dtype)
    _say(f"[scale]   ok score={s_err:.2e}")
