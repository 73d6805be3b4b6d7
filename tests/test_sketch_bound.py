"""The block-sketch interval, checked on the CPU against fp32 scores (no GPU).

The sketched selection (btk_select_sketch, btk_decode_step_sketch) may drop a
block only when its score interval lies below k others, so its indices equal
the full scan's only if every fp32 score the scan can compute lies inside the
interval [sa - e, sa + e] that the 8-bit copy gives.  The row encoding is
stated in include/btk.h (code = rint(c / scale) + 128, scale = max|c| / 127)
and the bound there (e = 0.51 * scale * sum|qs|).  Here both are evaluated in
float32 with numpy, independently of the HIP code, on rows built to be hard:
every coordinate half a step from a code (the rounding error of each term at
its maximum, all of one sign against the query), cancelling queries, a single
large coordinate, tiny and zero rows; and the fp32 score is summed in several
orders (the bound must not depend on the order).  A bound with the quantisation
term alone (0.5) would fail here, which the last test shows.
"""
import numpy as np
import pytest

F = np.float32


def encode(c):
    """(codes as float32 in 1..255, scale) for one fp32 centroid row."""
    amax = F(np.max(np.abs(c)))
    scale = F(amax / F(127.0))
    if amax == 0:
        return np.full(c.shape, F(128.0)), scale
    q = np.rint((c / scale).astype(F)).astype(F)
    q = np.clip(q, F(-127.0), F(127.0))
    return (q + F(128.0)).astype(F), scale


def fma_chain(a, b, t=F(0.0)):
    """Sequential fused multiply-adds in float32 (product exact in float64)."""
    for x, y in zip(a, b):
        t = F(np.float64(x) * np.float64(y) + np.float64(t))
    return t


def sum_orders(terms):
    """float32 sums of the same terms in several orders."""
    terms = terms.astype(F)
    out = [F(np.sum(terms, dtype=F))]            # numpy's pairwise order
    s = F(0.0)
    for x in terms:
        s = F(s + x)
    out.append(s)                                 # left to right
    s = F(0.0)
    for x in terms[::-1]:
        s = F(s + x)
    out.append(s)                                 # right to left
    part = [F(np.sum(terms[i:i + 8], dtype=F)) for i in range(0, len(terms), 8)]
    s = F(0.0)
    for p in part:
        s = F(s + p)
    out.append(s)                                 # lanes of 8, then across lanes
    return out


def interval(qs, codes, scale, factor=0.51):
    """[lo, hi] as the sketch scan forms it: 16 codes per lane by fused
    multiply-adds, lane sums added, minus 128 * sum(qs), times the scale."""
    D = len(qs)
    lanes = [fma_chain(qs[i:i + 16], codes[i:i + 16]) for i in range(0, D, 16)]
    t = F(0.0)
    for x in lanes:
        t = F(t + x)
    q128 = F(F(128.0) * F(np.sum(qs, dtype=F)))
    qn1 = F(np.sum(np.abs(qs), dtype=F))
    sa = F(scale * F(t - q128))
    e = F(scale * F(F(factor) * qn1))
    return F(sa - e), F(sa + e)


def scores(qs, c):
    """fp32 scores of one row in several summation orders, including the scan's
    (16 lanes of 8 products each, lanes added)."""
    prods = (qs.astype(np.float64) * c.astype(np.float64)).astype(F)
    out = sum_orders(prods)
    lanes = [fma_chain(qs[i:i + 8], c[i:i + 8]) for i in range(0, len(qs), 8)]
    s = F(0.0)
    for x in lanes:
        s = F(s + x)
    out.append(s)
    return out


def hard_rows(rng, D):
    """Rows whose every coordinate sits exactly half a step between two codes,
    rounded (ties to even) against the query's sign, so that each term's
    quantisation error is exactly 0.5 * scale * |qs_d|, all of one sign.  The
    scale is a power of two, so c / scale is exact in float32."""
    rows = []
    for _ in range(60):
        qs = (rng.standard_normal(D) * rng.uniform(0.01, 2.0)).astype(F)
        scale = F(2.0 ** -int(rng.integers(0, 12)))
        k = rng.integers(-126, 126, size=D)
        # rint(k + 0.5) is k when k is even, k + 1 when odd: the code lands
        # below c where qs > 0 (k even) and above it where qs < 0 (k odd)
        k = np.where(qs > 0, k - (k % 2), k - (k % 2) + 1)
        x = ((k + 0.5) * scale).astype(F)
        pin = rng.integers(D)
        x[pin] = F(127.0) * scale   # pins max|c| and so the scale (no error there)
        qs[pin] = F(1e-30)          # so the error sum is 0.5 * scale * sum|qs|
        rows.append((qs, x))
    return rows


def other_rows(rng, D):
    rows = []
    for _ in range(60):  # the workloads' model: offset + mean of 16 noise keys
        qs = (rng.standard_normal(D) * 0.5 / np.sqrt(D)).astype(F)
        c = (rng.standard_normal(D) * 0.5 + rng.standard_normal(D) / 4).astype(F)
        rows.append((qs, c))
    for _ in range(20):  # cancelling query: sum(qs) ~ 0, sum|qs| large
        h = rng.standard_normal(D // 2).astype(F)
        qs = np.concatenate([h, -h]).astype(F)
        rows.append((qs, rng.standard_normal(D).astype(F)))
    for _ in range(20):  # one large coordinate, the rest tiny
        c = (rng.standard_normal(D) * 1e-4).astype(F)
        c[rng.integers(D)] = F(rng.choice([-1, 1]) * 50.0)
        rows.append((rng.standard_normal(D).astype(F), c))
    for _ in range(10):  # tiny rows
        rows.append((rng.standard_normal(D).astype(F),
                     (rng.standard_normal(D) * 1e-30).astype(F)))
    rows.append((rng.standard_normal(D).astype(F), np.zeros(D, dtype=F)))
    return rows


@pytest.mark.parametrize("D", [64, 128])
def test_every_fp32_score_lies_inside_the_sketch_interval(D):
    rng = np.random.default_rng(1234 + D)
    worst = 0.0
    for qs, c in hard_rows(rng, D) + other_rows(rng, D):
        codes, scale = encode(c)
        lo, hi = interval(qs, codes, scale)
        qn1 = float(np.sum(np.abs(qs.astype(np.float64))))
        for s in scores(qs, c):
            assert lo <= s <= hi, (float(lo), float(s), float(hi))
            if scale > 0 and qn1 > 0:
                mid = (float(lo) + float(hi)) / 2
                worst = max(worst, abs(float(s) - mid) / (float(scale) * qn1))
    # the hard rows reach the quantisation term itself
    assert 0.4999 < worst < 0.51


def test_the_quantisation_term_alone_is_not_a_bound():
    """With e = 0.5 * scale * sum|qs| some hard row's score falls outside: the
    extra 0.01 is what covers the rounding of the fp32 arithmetic."""
    rng = np.random.default_rng(99)
    D = 128
    outside = 0
    for qs, c in hard_rows(rng, D):
        codes, scale = encode(c)
        lo, hi = interval(qs, codes, scale, factor=0.5)
        outside += sum(not (lo <= s <= hi) for s in scores(qs, c))
    assert outside > 0


def test_codes_match_the_stated_layout():
    """code = rint(c / scale) + 128 (ties to even), scale = max|c| / 127: the
    largest magnitude maps to 1 or 255 and zero to 128."""
    c = np.array([0.0, 1.0, -2.54, 2.54, 0.01, -0.01], dtype=F)
    codes, scale = encode(c)
    assert scale == F(F(2.54) / F(127.0))
    assert codes[0] == 128 and codes[2] == 1 and codes[3] == 255
    assert codes[1] == 128 + np.rint(F(1.0) / scale)
    assert np.all((codes >= 1) & (codes <= 255))
