"""The bound that a later-chunk fork candidate's key puts on its vector's
maximum, checked on a model of the arithmetic that produces it.

A candidate vector at temperature > 0 is passed on with the key e + hi, where
e is the binary exponent of its sum of terms vs = sum_e 2^(x_e c - hi): each
term is exp2 of the fused x c - hi rounded once to fp32, the terms are added
pairwise in fp32, and e is such that vs lies in [2^(e-1), 2^e).  The ranking
treats the vector's maximum as lying in

    [(key - 1 - log2(VEC) - m) / c, (key + m) / c],   m = 1e-3 + 1e-5 |key|.

This module models that arithmetic in numpy (fp32 where the kernels use
fp32) and checks the window against the exact maximum on random vectors,
including the scales where it is tightest: small temperatures (large c),
logits of large magnitude, references far from the vector, ties and
vectors with padding (-inf) elements.  CPU only.
"""

import numpy as np
import pytest


def _terms_sum(x32, c32, hi32):
    """fp32 model: fused x c - hi rounded once, fp32 exp2, pairwise fp32 sum."""
    hi = np.asarray(hi32, dtype=np.float64)[..., None]
    arg = (x32.astype(np.float64) * np.float64(c32) - hi).astype(np.float32)
    t = np.exp2(arg).astype(np.float32)
    while t.shape[-1] > 1:
        h = t.shape[-1] // 2
        t = (t[..., :h] + t[..., h:]).astype(np.float32)
    return t[..., 0]


def _key(vs, hi32):
    """e + hi for vs in [2^(e-1), 2^e); +inf where vs is zero, subnormal or
    not finite."""
    vs = np.asarray(vs, dtype=np.float32)
    ok = (vs >= np.float32(1.17549435e-38)) & np.isfinite(vs)
    _, e = np.frexp(np.where(ok, vs, np.float32(1.0)))
    return np.where(ok, (e.astype(np.float32) + hi32).astype(np.float32), np.float32(np.inf))


def _window(key, c32, vec):
    low_bits = 1.0 + np.log2(vec)
    k64 = np.where(np.isfinite(key), key, 0.0).astype(np.float64)  # no bound: set below
    m = 1e-3 + 1e-5 * np.abs(k64)
    inv_c = 1.0 / np.float64(c32)
    lo = ((k64 - low_bits - m) * inv_c).astype(np.float32)
    hi = ((k64 + m) * inv_c).astype(np.float32)
    lo = np.where(np.isfinite(key), lo, np.float32(-np.inf))
    hi = np.where(np.isfinite(key), hi, np.float32(np.inf))
    return lo, hi


CASES = [  # (logit scale, offset, temperature, reference shift in logits)
    (1.0, 0.0, 0.7, 0.0), (1.0, 0.0, 0.7, 5.0), (40.0, 0.0, 0.02, 0.0), (40.0, 0.0, 0.05, 30.0),
    (1.0, 1000.0, 0.05, 0.0), (1.0, -1000.0, 0.3, 2.0), (1e-3, 0.0, 100.0, 0.0),
    (4.0, 500.0, 0.02, 1.0), (1.0, 0.0, 4.0, 60.0),
]


@pytest.mark.parametrize("vec", [8, 4])
@pytest.mark.parametrize("scale,offset,tau,shift", CASES)
def test_key_window_holds_the_maximum(vec, scale, offset, tau, shift):
    rng = np.random.default_rng(int(1000 * tau) + vec + int(scale))
    n = 20000
    x = (rng.standard_normal((n, vec)) * 3.0 * scale + offset).astype(np.float32)
    # ties, and padding / masked elements (-inf) in some vectors
    x[: n // 10, 1:] = x[: n // 10, :1]
    x[n // 10: n // 5, vec // 2:] = -np.inf
    c32 = np.float32(np.log2(np.e) / tau)
    # the lane reference: a maximum seen earlier in the lane, at or above
    # this vector's (shifted up by `shift` logits), rounded like the kernels
    ref = (x.max(axis=1) + np.float32(shift)).astype(np.float32)
    hi32 = (ref * c32).astype(np.float32)
    vs = _terms_sum(x, c32, hi32)
    key = _key(vs, hi32)
    lo, hi = _window(key, c32, vec)
    xmax = x.max(axis=1)
    bounded = np.isfinite(key)
    # a key is missing (no bound, the vector is re-read) only where the
    # vector's largest term underflows fp32
    top_arg = xmax.astype(np.float64) * np.float64(c32) - hi32.astype(np.float64)
    assert np.all(top_arg[~bounded] < -120), top_arg[~bounded].max()
    assert np.all(xmax[bounded] <= hi[bounded]), "upper end below the maximum"
    assert np.all(xmax[bounded] >= lo[bounded]), "lower end above the maximum"
    # the window is the width the derivation promises, plus the margins and
    # the fp32 rounding of its two ends
    width = (hi - lo)[bounded].astype(np.float64) * np.float64(c32)
    slack = (np.spacing(np.abs(hi[bounded])) + np.spacing(np.abs(lo[bounded]))).astype(
        np.float64) * np.float64(c32)
    assert np.all(width <= 1.0 + np.log2(vec) + 2 * (1e-3 + 1e-5 * np.abs(key[bounded]))
                  + slack + 1e-4)


def test_key_of_an_empty_or_underflowed_sum_bounds_nothing():
    hi32 = np.float32(10.0)
    key = _key(np.array([0.0, 1e-40, np.inf, np.nan], dtype=np.float32), hi32)
    assert np.all(np.isinf(key))
