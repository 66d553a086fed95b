"""Pins for the oracle's outlier migration (SmoothQuant-style, exponent 1/2).

The scale is s[k] = sqrt(max|Xc[:,k]| / max|W[:,k]|) in fp32 with correctly
rounded division and square root; the pins recompute it by an independent
exact route (rational arithmetic and decimal square roots), check the
closed-form balance property, the invariance X' W'^T ~ X W^T within fp16
rounding, and the zero guards.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

import oracle

getcontext().prec = 60


def _round_f32(q: Fraction) -> np.float32:
    """Correctly rounded binary32 of a positive rational (ties to even)."""
    # bracket with nextafter on the float64 neighbourhood, then decide exactly
    f = np.float32(float(q))
    lo, hi = np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(np.inf))
    cands = [lo, f, hi]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - q),
                                     int(np.frombuffer(np.float32(c).tobytes(), np.uint32)[0]) & 1))
    return np.float32(best)


def _sqrt_f32(q: np.float32) -> np.float32:
    r = Decimal(float(q)).sqrt()
    return _round_f32(Fraction(r))


def test_scales_match_an_exact_route():
    rng = np.random.default_rng(0)
    K = 400
    xc = (rng.standard_normal((32, K)) * np.exp(rng.uniform(-6, 6, K))).astype(np.float16)
    w = (rng.standard_normal((48, K)) * np.exp(rng.uniform(-8, 2, K))).astype(np.float16)
    s = oracle.smooth_scales(xc, w)
    for k in range(K):
        ax = max(abs(Fraction(float(v))) for v in xc[:, k])
        aw = max(abs(Fraction(float(v))) for v in w[:, k])
        q = _round_f32(ax / aw)
        assert s[k].tobytes() == _sqrt_f32(q).tobytes(), k


def test_closed_form_and_zero_guards():
    xc = np.array([[4.0, -9.0, 0.0, 1.0], [-1.0, 3.0, 0.0, 0.5]], np.float16)
    w = np.array([[1.0, -0.25, 2.0, 0.0], [0.5, 1.0, -1.0, 0.0]], np.float16)
    s = oracle.smooth_scales(xc, w)
    assert s.tolist() == [2.0, 3.0, 1.0, 1.0]
    assert oracle.smooth_weights(w, s).astype(np.float32).tolist() == [[2.0, -0.75, 2.0, 0.0],
                                                                        [1.0, 3.0, -1.0, 0.0]]
    assert oracle.smooth_acts(xc, s).astype(np.float32).tolist() == [[2.0, -3.0, 0.0, 1.0],
                                                                      [-0.5, 1.0, 0.0, 0.5]]


def test_balance_and_product_invariance():
    rng = np.random.default_rng(1)
    K, N, T = 256, 64, 96
    xc = rng.standard_normal((T, K))
    xc[:, rng.choice(K, 4, replace=False)] *= 40
    xc = xc.astype(np.float16)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    s = oracle.smooth_scales(xc, w)
    x2, w2 = oracle.smooth_acts(xc, s), oracle.smooth_weights(w, s)
    # balance: both migrated column maxima equal sqrt(ax * aw) up to rounding
    ax = np.abs(xc.astype(np.float64)).max(0)
    aw = np.abs(w.astype(np.float64)).max(0)
    target = np.sqrt(ax * aw)
    for got in (np.abs(x2.astype(np.float64)).max(0), np.abs(w2.astype(np.float64)).max(0)):
        assert np.all(np.abs(got - target) <= 2.0 ** -9 * target)
    # invariance: each factor carries at most one fp16 rounding (2^-11 rel)
    y = xc.astype(np.float64) @ w.astype(np.float64).T
    y2 = x2.astype(np.float64) @ w2.astype(np.float64).T
    bound = 2 * 2.0 ** -10 * (np.abs(xc.astype(np.float64)) @ np.abs(w.astype(np.float64)).T)
    assert np.all(np.abs(y2 - y) <= bound)
