"""Parity rules between the HIP library and the CPU oracle (test helpers).

Selection (the margin rule): for a unit with n_b blocks and k_b = min(k, n_b),
margin = s_(k_b) - s_(k_b + 1) of the oracle's scores sorted in descending order.
If n_b <= k or margin > MARGIN, the library's index row must equal the
oracle's bit for bit.  Otherwise several sets are correct: every selected block
must score at least s_(k_b) - MARGIN, and the row must still be k_b distinct
in-range blocks in ascending order followed by -1.
The margin's unit depends on the reading of the group score: the mean of the
heads' scaled logits (the reading the library implements) or the plain sum of
the heads' unscaled dot products, which is larger by r * sqrt(D).  Given
``sum_factor`` = r * sqrt(D), exactness is also demanded wherever the margin
exceeds MARGIN in the sum's units, i.e. on almost every unit; both counts are
reported.
Outputs are compared with the oracle on units whose index rows are equal; the
attention step on its own is compared on the oracle's index rows.
"""
from __future__ import annotations

import math

import torch

MARGIN = 1e-3           # score units (scaled logits), as in the contract
OUT_TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-5}
LSE_TOL = {torch.bfloat16: 1e-3, torch.float32: 1e-5}
CENTROID_TOL = 1e-5
SCORE_TOL = 1e-4


def n_blocks(seq_lens, page=16):
    return [(int(L) + page - 1) // page for L in seq_lens.tolist()]


def sum_factor(group, head_dim):
    """Factor from the mean of the heads' scaled logits to the sum of their
    unscaled dot products (scale 1/sqrt(D))."""
    return group * math.sqrt(head_dim)


def check_indices(gpu_idx, ora_idx, ora_scores, seq_lens, top_k, margin=MARGIN, page=16,
                  sum_units=None):
    """Assert the margin rule on every unit; returns statistics.  page=1 applies
    the rule to token positions (the token-level baseline).  sum_units (see
    sum_factor) also applies the rule with the margin in the sum's units."""
    gpu_idx, ora_idx = gpu_idx.cpu(), ora_idx.cpu()
    B, H, K = ora_idx.shape
    assert K == top_k and tuple(gpu_idx.shape) == (B, H, K)
    nbs = n_blocks(seq_lens, page)
    stats = dict(units=0, strict=0, near_tie=0, differ=0, min_strict_margin=math.inf,
                 strict_sum=0)
    equal = torch.zeros((B, H), dtype=torch.bool)
    for b in range(B):
        nb = nbs[b]
        kb = min(top_k, nb)
        for g in range(H):
            stats["units"] += 1
            row, want = gpu_idx[b, g], ora_idx[b, g]
            sel = row[:kb]
            assert (row[kb:] == -1).all(), (b, g, row)
            assert (sel >= 0).all() and (sel < nb).all(), (b, g, row)
            assert (sel[1:] > sel[:-1]).all(), (b, g, row)  # strictly ascending, distinct
            same = torch.equal(row, want)
            equal[b, g] = same
            if nb <= top_k:
                assert same, (b, g)
                stats["strict"] += 1
                stats["strict_sum"] += 1
                continue
            s = ora_scores[b, g, :nb].double()
            srt = torch.sort(s, descending=True).values
            m = float(srt[kb - 1] - srt[kb])
            if sum_units is not None and m * sum_units > margin:
                stats["strict_sum"] += 1
                assert same, (b, g, m, "sum units", row, want)
            if m > margin:
                stats["strict"] += 1
                stats["min_strict_margin"] = min(stats["min_strict_margin"], m)
                assert same, (b, g, m, row, want)
            else:
                stats["near_tie"] += 1
                floor = float(srt[kb - 1]) - margin
                assert (s[sel.long()] >= floor).all(), (b, g, m)
            if not same:
                stats["differ"] += 1
    stats["equal_mask"] = equal
    return stats


def max_abs(a, b):
    return float((a.float().cpu() - b.float().cpu()).abs().max()) if a.numel() else 0.0


def check_outputs(gpu_out, ora_out, dtype, unit_mask=None, group=1, what="out"):
    """Max-abs check of [B, Hq, D] outputs; unit_mask [B, Hkv] restricts the units."""
    g = gpu_out.float().cpu()
    o = ora_out.float().cpu()
    if unit_mask is not None:
        head_mask = unit_mask.repeat_interleave(group, dim=1)
        g, o = g[head_mask], o[head_mask]
    err = max_abs(g, o)
    assert torch.isfinite(g).all(), f"{what}: non-finite values"
    assert err <= OUT_TOL[dtype], f"{what}: max abs {err} > {OUT_TOL[dtype]}"
    return err


def check_lse(gpu_lse, ora_lse, dtype, unit_mask=None, group=1):
    g, o = gpu_lse.float().cpu(), ora_lse.float().cpu()
    if unit_mask is not None:
        head_mask = unit_mask.repeat_interleave(group, dim=1)
        g, o = g[head_mask], o[head_mask]
    err = max_abs(g, o)
    assert err <= LSE_TOL[dtype], f"lse: max abs {err} > {LSE_TOL[dtype]}"
    return err
