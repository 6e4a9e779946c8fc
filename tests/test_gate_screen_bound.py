"""The error bound behind the screened gate (CPU, no GPU).

Each fp32 gate weight is split, rounding to nearest, into two bf16 pieces and a
remainder, w = w1 + w2 + w3 exactly with |w3| <= 2^-16 |w|.  The screen adds the
exact fp32 products x * w1 and x * w2 in fp32, 256 of them (4 chunks of 32 K,
both pieces) per accumulator group, and the group sums into an fp32 total.  The
router assumes that for G groups the screened logit is within
    gamma_(256 + G + 2) |x|_2 (|w1|_2 + |w2|_2) + |x|_2 |w3|_2
of the exact dot product, whatever order the additions take; here that is
checked against exact rational dot products over several orders, and each of
the two terms on an input that brings the error close to it."""
import math
from fractions import Fraction

import numpy as np
import torch

U = 2.0 ** -24


def gamma(n):
    return n * U / (1 - n * U)


def bf16_rn(v: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even), returned as fp32."""
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def split2(w32: np.ndarray):
    w32 = np.asarray(w32, dtype=np.float32)
    w1 = bf16_rn(w32)
    r = (w32 - w1).astype(np.float32)
    w2 = bf16_rn(r)
    w3 = (r - w2).astype(np.float32)
    return w1, w2, w3


def bf16_exact(v: np.ndarray) -> bool:
    return bool(np.all((np.asarray(v, dtype=np.float32).view(np.uint32) & np.uint32(0xFFFF)) == 0))


def test_split_is_exact_and_the_remainder_small():
    rng = np.random.default_rng(0)
    w = np.concatenate([rng.standard_normal(100000) * 0.02, rng.standard_normal(1000) * 1e-20,
                        rng.standard_normal(1000) * 1e30,
                        [0.0, -0.0, 1.0, -3.0e38, 1.1754944e-38, 1e-45]]).astype(np.float32)
    w1, w2, w3 = split2(w)
    assert bf16_exact(w1) and bf16_exact(w2)
    # the remainder r = w - w1 and w3 = r - w2 are exact fp32 differences
    assert np.array_equal(w1.astype(np.float64) + w2.astype(np.float64) + w3.astype(np.float64),
                          w.astype(np.float64))
    normal = np.abs(w) >= 2.0 ** -126
    assert np.all(np.abs(w3[normal]).astype(np.float64) <= 2.0 ** -16 * np.abs(w[normal]).astype(np.float64))
    # products with a bf16 activation are exact in fp32 (8 x 8 significant bits)
    x = torch.randn(1000).to(torch.bfloat16).float().numpy()
    for p in (w1[:1000], w2[:1000]):
        prod32 = (x * p).astype(np.float32)
        assert np.array_equal(prod32.astype(np.float64), x.astype(np.float64) * p.astype(np.float64))


def _fp32_sum(terms, order):
    if order == "reverse":
        terms = terms[::-1]
    elif order == "sorted":
        terms = sorted(terms, key=abs)
    elif order == "largest_first":
        terms = sorted(terms, key=abs, reverse=True)
    if order == "pairwise":
        t = list(terms)
        while len(t) > 1:
            t = [np.float32(t[j] + t[j + 1]) if j + 1 < len(t) else t[j] for j in range(0, len(t), 2)]
        return t[0] if t else np.float32(0.0)
    acc = np.float32(0.0)
    for v in terms:
        acc = np.float32(acc + v)
    return acc


def _screen(x: np.ndarray, w: np.ndarray, order: str) -> float:
    """The screen's arithmetic with a chosen fp32 order inside each group."""
    w1, w2, _ = split2(w)
    tot = np.float32(0.0)
    for k0 in range(0, len(x), 128):
        xs = x[k0:k0 + 128].astype(np.float32)
        terms = list((xs * w2[k0:k0 + 128]).astype(np.float32)) + list((xs * w1[k0:k0 + 128]).astype(np.float32))
        tot = np.float32(tot + _fp32_sum(terms, order))
    return float(tot)


def _bound(x, w):
    w1, w2, w3 = split2(w)
    n2 = lambda v: math.sqrt(float(np.sum(np.asarray(v, dtype=np.float64) ** 2)))
    G = len(x) // 128
    return gamma(256 + G + 2) * n2(x) * (n2(w1) + n2(w2)), n2(x) * n2(w3)


ORDERS = ("forward", "reverse", "sorted", "largest_first", "pairwise")


def test_screened_logit_is_within_the_bound():
    rng = np.random.default_rng(1)
    H = 1024
    worst = 0.0
    for trial in range(12):
        x = torch.randn(H, generator=torch.Generator().manual_seed(trial)).to(torch.bfloat16).float().numpy()
        w = (rng.standard_normal(H) * (0.02 if trial % 3 else 3.0)).astype(np.float32)
        if trial % 4 == 1:                        # a few large terms among small ones
            w[rng.integers(0, H, 8)] *= 1e4
        exact = sum(Fraction(float(xi)) * Fraction(float(wi)) for xi, wi in zip(x, w))
        acc_part, rem_part = _bound(x, w)
        for order in ORDERS:
            err = abs(Fraction(_screen(x, w, order)) - exact)
            assert err <= Fraction(acc_part + rem_part), (trial, order, float(err), acc_part, rem_part)
            worst = max(worst, float(err) / (acc_part + rem_part))
    assert worst < 0.5            # the bound is not tight


def test_the_screen_misses_exactly_the_remainder():
    """Against the exact sum over the two pieces the screen is within the
    accumulation term alone; what it leaves out is the remainder's dot product,
    which the second term bounds and which, for x aligned with w3, comes close to it."""
    rng = np.random.default_rng(2)
    H = 1024
    w = (rng.standard_normal(H) * 0.02).astype(np.float32)
    w1, w2, w3 = split2(w)
    x = bf16_rn(np.sign(w3) * (1.0 + rng.random(H)))
    exact = sum(Fraction(float(xi)) * Fraction(float(wi)) for xi, wi in zip(x, w))
    pieces = sum(Fraction(float(xi)) * (Fraction(float(a)) + Fraction(float(b))) for xi, a, b in zip(x, w1, w2))
    rem = sum(Fraction(float(xi)) * Fraction(float(c)) for xi, c in zip(x, w3))
    assert exact == pieces + rem
    acc_part, rem_part = _bound(x, w)
    for order in ORDERS:
        assert abs(Fraction(_screen(x, w, order)) - pieces) <= Fraction(acc_part)
    assert 0.5 * rem_part < float(rem) <= rem_part


def test_the_accumulation_term_is_needed():
    """Terms of one sign whose partial sums keep losing their low bits: the
    accumulation error exceeds the remainder term, and stays within the bound."""
    H = 1024
    w = np.full(H, 1.0, dtype=np.float32)        # w1 = 1, w2 = w3 = 0
    x = np.empty(H, dtype=np.float32)
    x[0] = 2.0 ** 20
    x[1:] = bf16_rn(np.full(H - 1, 1.0 + 2.0 ** -7))
    exact = sum(Fraction(float(xi)) for xi in x)
    acc_part, rem_part = _bound(x, w)
    assert rem_part == 0.0
    err = abs(Fraction(_screen(x, w, "forward")) - exact)
    assert err > 0
    assert err <= Fraction(acc_part)


def _score64(z, sigmoid):
    z = np.asarray(z, dtype=np.float64)
    ez = np.exp(-np.abs(z))
    sig = np.where(z >= 0, 1 / (1 + ez), ez / (1 + ez))
    return sig if sigmoid else np.sqrt(np.maximum(z, 0) + np.log1p(ez))


def test_score_second_derivatives_are_below_a_tenth():
    """The router widens a score interval by 0.125 dl^2 for the change of slope: both
    score functions have |f''| < 0.1 (finite differences over [-60, 60])."""
    z = np.linspace(-60, 60, 1_200_001)
    h = 1e-3
    for sigmoid in (True, False):
        f2 = (_score64(z + h, sigmoid) - 2 * _score64(z, sigmoid) + _score64(z - h, sigmoid)) / h ** 2
        assert np.abs(f2).max() < 0.1
    # and f' <= 0.32 for sqrt(softplus), 0.25 for sigmoid
    f1 = (_score64(z + h, False) - _score64(z - h, False)) / (2 * h)
    assert f1.max() < 0.32 and f1.min() > 0


def test_one_evaluation_score_interval_holds_the_scores_around_it():
    """The key interval of one screened logit: f(l32) and its slope in fp32, widened by
    (slope (1 + 2^-10) + 0.125 dl) dl + 2^-16 f + ulp, contains the fp32 score of every
    logit within dl (sampled densely), for both score functions and dl from 1e-6 to 1."""
    rng = np.random.default_rng(5)
    for sigmoid in (True, False):
        for _ in range(400):
            l32 = np.float32(rng.normal() * rng.choice([0.5, 3.0, 12.0]))
            dl = float(10.0 ** rng.uniform(-6, 0))
            ez = np.float32(np.exp(np.float32(-abs(l32))))
            sig = np.float32(1) / (np.float32(1) + ez) if l32 >= 0 else ez / (np.float32(1) + ez)
            if sigmoid:
                sc, slope = np.float32(sig), np.float32(sig * (np.float32(1) - sig))
            else:
                sc = np.float32(np.sqrt(np.float32(max(l32, 0)) + np.float32(np.log1p(ez))))
                slope = np.float32(min(sig / (np.float32(2) * sc), 0.32)) if sc > 0 else np.float32(0.32)
            hw = np.float32((float(slope) * (1 + 2 ** -10) + 0.125 * dl) * dl) + sc * np.float32(2 ** -16) \
                + np.spacing(sc)
            u = np.spacing(np.float32(max(sc, hw)))
            lo, hi = np.float32(np.float32(sc - hw) - u), np.float32(np.float32(sc + hw) + u)
            zz = float(l32) + np.linspace(-dl, dl, 2001)
            s = _score64(zz, sigmoid).astype(np.float32)
            assert np.all(s >= lo) and np.all(s <= hi), (sigmoid, l32, dl)
