"""Pins of the oracle's 4-bit error quantizer (first and third paragraphs of the
MicroAdam page): codes in range, extremes exact, per-element error below one
level, empirical unbiasedness, and Lemma 1's omega bound on every realization."""
import numpy as np
import pytest

import oracle as O


def _levels(lo, hi):
    return (np.float32(hi) - np.float32(lo)) / np.float32(15.0)


def test_codes_range_and_extremes():
    rng = np.random.default_rng(10)
    for t in range(1, 30):
        n = int(rng.integers(2, 20000))
        x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-8, 3)).astype(np.float32)
        lo, hi = O.group_minmax(x)
        assert lo == x.min() and hi == x.max()
        codes = O.quant_group(x, 42, t, 3, 0, lo, hi)
        assert codes.max() <= 15
        assert (codes[x == lo] == 0).all()
        assert (codes[x == hi] == 15).all()
        xh = O.dequant_group(codes, lo, hi)
        s = np.float64(_levels(lo, hi))
        err = np.abs(xh.astype(np.float64) - x.astype(np.float64))
        # stochastic rounding moves to one of the two neighbouring levels
        assert (err <= s * (1 + 1e-5) + 1e-38).all()
        assert abs(float(xh[x == lo][0]) - float(lo)) <= 1e-6 * abs(float(lo)) + 1e-38


def test_constant_group():
    x = np.full(1000, 0.25, np.float32)
    lo, hi = O.group_minmax(x)
    codes = O.quant_group(x, 1, 1, 0, 0, lo, hi)
    assert (codes == 0).all()
    assert (O.dequant_group(codes, lo, hi) == np.float32(0.25)).all()
    # the all-zero initial state dequantizes to exactly zero
    assert (O.dequant_group(np.zeros(10, np.uint8), 0.0, 0.0) == 0).all()


def test_signed_zero_statistics_are_canonical():
    lo, hi = O.group_minmax(np.array([-0.0, -0.0], np.float32))
    assert np.float32(lo).view(np.uint32) == 0 and np.float32(hi).view(np.uint32) == 0


def test_quantizer_is_unbiased():
    # fixed x, many independent draws (different steps): the mean of Q^{-1}Q(x)
    # approaches x.  Per coordinate |mean err| <= 6 sigma/sqrt(N).
    rng = np.random.default_rng(11)
    n, N = 4096, 3000
    x = rng.standard_normal(n).astype(np.float32)
    lo, hi = O.group_minmax(x)
    acc = np.zeros(n)
    acc2 = np.zeros(n)
    for t in range(1, N + 1):
        xh = O.dequant_group(O.quant_group(x, 42, t, 0, 0, lo, hi), lo, hi).astype(np.float64)
        e = xh - x
        acc += e
        acc2 += e * e
    mean = acc / N
    s = float(_levels(lo, hi))
    # stochastic rounding to the two neighbouring levels: err/s is Bernoulli(p)
    # shifted by -p with p = frac((x - lo)*15/(hi - lo)), computed here in double
    y = (x.astype(np.float64) - float(lo)) * 15.0 / (float(hi) - float(lo))
    p = y - np.floor(y)
    sd = s * np.sqrt(p * (1 - p))
    # floor: the 16-bit resolution of xi leaves a bias of at most s*2^-16
    z = np.abs(mean) / np.maximum(sd / np.sqrt(N), s * 2.0 ** -16)
    assert z.max() < 6.0, z.max()
    # the pooled bias is tiny against the level spacing (2^-16 resolution of xi)
    assert abs(mean.mean()) < 5 * s / np.sqrt(N * n) + s * 2 ** -16


def test_round_to_nearest_would_be_caught():
    # guard for the unbiasedness pin: the same statistic, applied to deterministic
    # rounding rules planted in a numpy copy of the quantizer (nearest level, and
    # always down), rejects them
    rng = np.random.default_rng(11)
    n, N = 4096, 3000
    x = rng.standard_normal(n).astype(np.float32)
    lo, hi = O.group_minmax(x)
    s = float(_levels(lo, hi))
    y = (x.astype(np.float64) - float(lo)) * 15.0 / (float(hi) - float(lo))
    p = y - np.floor(y)
    sd = s * np.sqrt(p * (1 - p))
    for planted in (np.rint(y), np.floor(y)):
        xh = float(lo) + np.clip(planted, 0, 15) * s
        mean = xh - x.astype(np.float64)          # every draw gives the same value
        z = np.abs(mean) / np.maximum(sd / np.sqrt(N), s * 2.0 ** -16)
        assert z.max() > 6.0


def _omega(n, lo, hi, b=4):
    lo, hi = float(lo), float(hi)
    return np.sqrt(n - 2) / (2 ** b - 1) * (hi - lo) / np.sqrt(hi * hi + lo * lo)


def test_lemma1_per_block_every_realization():
    rng = np.random.default_rng(12)
    for t in range(1, 200):
        n = int(rng.integers(3, 16385))
        x = (rng.standard_t(3, n) * 1e-3).astype(np.float32)
        x[rng.random(n) < 0.01] = 0.0      # zeroed Top-k entries are part of the residual
        lo, hi = O.group_minmax(x)
        xh = O.dequant_group(O.quant_group(x, 7, t, 0, 0, lo, hi), lo, hi)
        err = np.linalg.norm(xh.astype(np.float64) - x.astype(np.float64))
        bound = _omega(n, lo, hi) * np.linalg.norm(x.astype(np.float64))
        assert err <= bound * (1 + 1e-5)


def test_lemma1_global_over_blocks():
    # blockwise statistics satisfy the same bound with n = d and the global extremes
    rng = np.random.default_rng(13)
    d, B = 200_000, 16384
    x = (rng.standard_normal(d) * 1e-3).astype(np.float32)
    xh = np.empty_like(x)
    for j in range(-(-d // B)):
        sl = slice(j * B, min(d, (j + 1) * B))
        lo, hi = O.group_minmax(x[sl])
        xh[sl] = O.dequant_group(O.quant_group(x[sl], 7, 1, j, 0, lo, hi), lo, hi)
    err = np.linalg.norm(xh.astype(np.float64) - x.astype(np.float64))
    bound = _omega(d, x.min(), x.max()) * np.linalg.norm(x.astype(np.float64))
    assert err <= bound


def test_tiny_range_without_finite_scale_is_flat():
    # 15/(Delta - delta) overflows fp32 below ~4.4e-38: every code is 0
    x = np.array([0.0, 1e-45, 2e-45, 1e-39], np.float32)
    lo, hi = O.group_minmax(x)
    with np.errstate(over="ignore"):   # the overflow is the point
        assert not np.isfinite(np.float32(15.0) / (np.float32(hi) - np.float32(lo)))
    assert (O.quant_group(x, 1, 1, 0, 0, lo, hi) == 0).all()
    # just above the limit the scale is finite and the extremes map to 0 and 15
    x = np.array([0.0, 1e-36], np.float32)
    lo, hi = O.group_minmax(x)
    c = O.quant_group(x, 1, 1, 0, 0, lo, hi)
    assert c[0] == 0 and c[1] == 15
