"""Pins of the oracle's reading for non-finite values (the MicroAdam page,
first paragraph, ranks by |a_t| and assumes finite gradients).  The reading:

- the Top-k key is the 31-bit pattern of |a|: +-Inf above every finite value,
  NaN above that; every NaN stands for the canonical quiet NaN, so all NaNs
  tie and go by index, and a selected NaN is stored as bfloat16 0x7fc0;
- non-finite values left after the selection are dropped from the residual
  (set to +0) before its min / max;
- a residual range Delta - delta with no finite fp32 value resets the error
  feedback: delta = Delta = 0, every code 0;
- the parameters follow IEEE arithmetic: a non-finite window value makes its
  parameter NaN, as AdamW does with a non-finite gradient.

Each is checked against a plain Python statement of the rule (brute force on
small blocks), not against the oracle's own code."""
import math

import numpy as np
import pytest

import oracle as O

NAN_BITS = [0x7fc0, 0xffc0, 0x7f81, 0x7fff, 0xffa5]   # bf16 NaNs: canonical, negative, signalling, max payload
INF_BITS = [0x7f80, 0xff80]


def _rank(v):
    """The reading's order, stated without bit patterns: NaN first, then the
    infinities, then finite values by magnitude; equal ranks go by index."""
    if math.isnan(v):
        return (2, 0.0)
    if math.isinf(v):
        return (1, 0.0)
    return (0, abs(v))


def _block(rng, n, n_nan, n_inf, scale=1e-3):
    g = O.bf16_rne((rng.standard_normal(n) * scale).astype(np.float32))
    pos = rng.permutation(n)
    nan_pos, inf_pos = pos[:n_nan], pos[n_nan:n_nan + n_inf]
    g[nan_pos] = rng.choice(NAN_BITS, n_nan)
    g[inf_pos] = rng.choice(INF_BITS, n_inf)
    return g


def _one_block_step(g, kb, m=2, flags=0, state=None):
    n = g.size
    cfg = O.make_cfg(n, n, kb, m, flags=flags)
    st = state or O.FullState(cfg)
    theta = np.zeros(n, np.float32)
    st.step(theta, g)
    return cfg, st, theta


@pytest.mark.parametrize("n_nan,n_inf,kb", [(3, 4, 20), (30, 0, 20), (0, 30, 20), (25, 25, 20), (5, 5, 10),
                                            (400, 0, 64), (0, 0, 20)])
def test_selection_order_with_nonfinite_values(n_nan, n_inf, kb):
    # first step, no error feedback yet: a = g exactly
    rng = np.random.default_rng(100 + n_nan + n_inf + kb)
    n = 512
    g = _block(rng, n, n_nan, n_inf)
    _, st, _ = _one_block_step(g, kb)
    with np.errstate(invalid="ignore"):
        a = O.bf16_to_f32(g).astype(np.float64)
    want = sorted(range(n), key=lambda i: (tuple(-x for x in _rank(a[i])), i))[:kb]
    row = st.G.reshape(2, -1)[1]
    I = (row & 0xffff).astype(np.int64)
    np.testing.assert_array_equal(I, np.sort(want))
    Vb = (row >> 16).astype(np.uint16)
    for i, vb in zip(I, Vb):
        if math.isnan(a[i]):
            assert vb == 0x7fc0                      # the canonical NaN, whatever the input's payload and sign
        elif math.isinf(a[i]):
            assert vb == (0x7f80 if a[i] > 0 else 0xff80)
        else:
            assert vb == O.bf16_rne(np.float32(a[i]))[0]


@pytest.mark.parametrize("n_nan,n_inf,kb", [(3, 4, 20), (25, 25, 20), (400, 0, 64), (0, 300, 64)])
def test_leftover_nonfinite_values_are_dropped(n_nan, n_inf, kb):
    rng = np.random.default_rng(200 + n_nan + n_inf)
    n = 512
    g = _block(rng, n, n_nan, n_inf)
    cfg, st, _ = _one_block_step(g, kb)
    a = O.bf16_to_f32(g).astype(np.float32).copy()
    sel = (st.G.reshape(2, -1)[1] & 0xffff).astype(np.int64)
    a[sel] = 0.0
    a[~np.isfinite(a)] = 0.0                         # what is left non-finite is dropped
    lo, hi = st.stats
    assert lo == a.min() and hi == a.max()
    assert np.isfinite(st.stats).all()
    # the codes quantize that residual
    np.testing.assert_array_equal(O.unpack_nibbles(st.ef, n),
                                  O.quant_group(a, cfg.seed, 1, 0, 0, lo, hi))
    # the next step's feedback is finite
    xh = O.dequant_group(O.unpack_nibbles(st.ef, n), lo, hi)
    assert np.isfinite(xh).all()


def test_residual_range_overflow_resets_the_feedback():
    # finite values of both signs near the fp32 limit, more than the quota:
    # Delta - delta overflows, so delta = Delta = 0 and every code is 0
    rng = np.random.default_rng(7)
    n, kb = 1024, 16
    g = O.bf16_rne((rng.standard_normal(n) * 1e-3).astype(np.float32))
    big = O.bf16_rne(np.array([3.0e38], np.float32))[0]
    g[rng.permutation(n)[:200]] = big
    g[rng.permutation(n)[:200]] = big | 0x8000
    with np.errstate(over="ignore"):
        span = O.bf16_to_f32(np.array([big]))[0] - O.bf16_to_f32(np.array([big | 0x8000]))[0]
    assert span.dtype == np.float32 and np.isinf(span)       # 3e38 - (-3e38) is not a finite fp32
    cfg, st, _ = _one_block_step(g, kb)
    assert st.stats[0] == 0 and st.stats[1] == 0
    assert (O.unpack_nibbles(st.ef, n) == 0).all()
    # the reset feedback dequantizes to exactly 0: the next accumulator is g itself
    g2 = O.bf16_rne((rng.standard_normal(n) * 1e-3).astype(np.float32))
    st.step(np.zeros(n, np.float32), g2)
    sel = (st.G.reshape(2, -1)[0] & 0xffff).astype(np.int64)
    gf = O.bf16_to_f32(g2)
    np.testing.assert_array_equal(np.sort(sel), np.sort(O.topk(gf, kb)))


def test_global_pair_range_overflow_resets():
    rng = np.random.default_rng(8)
    d, B = 4096, 1024
    g = O.bf16_rne((rng.standard_normal(d) * 1e-3).astype(np.float32))
    big = O.bf16_rne(np.array([3.0e38], np.float32))[0]
    g[100:150] = big            # block 0: above its quota of 10
    g[3000:3050] = big | 0x8000  # block 2
    cfg = O.make_cfg(d, B, d // 100, 2, flags=O.FLAG_GLOBAL_QUANT)
    st = O.FullState(cfg)
    st.step(np.zeros(d, np.float32), g)
    assert st.stats[0] == 0 and st.stats[1] == 0
    assert (O.unpack_nibbles(st.ef, d) == 0).all()


def test_nonfinite_window_values_make_their_parameters_nan():
    # like AdamW on a non-finite gradient: m_hat / (sqrt(v_hat) + eps) is NaN
    # for a NaN or infinite window value; every other parameter stays finite
    rng = np.random.default_rng(9)
    n, kb = 2048, 40
    g = _block(rng, n, 6, 6)
    cfg = O.make_cfg(n, n, kb, 3)
    st = O.FullState(cfg)
    theta = (rng.standard_normal(n) * 0.02).astype(np.float32)
    st.step(theta, g)
    row = st.G.reshape(3, -1)[1]
    I = (row & 0xffff).astype(np.int64)
    V = O.bf16_to_f32((row >> 16).astype(np.uint16))
    bad = I[~np.isfinite(V)]
    assert bad.size == 12
    assert np.isnan(theta[bad]).all()
    ok = np.setdiff1d(np.arange(n), bad)
    assert np.isfinite(theta[ok]).all()


def test_no_error_feedback_nan_payloads_are_canonical():
    # without error feedback a = widened g, signalling NaN included; the key
    # and the window value are still the canonical NaN's
    g = np.array([0x3c00, 0x7f81, 0xffc0, 0x7fc0, 0x3c00, 0xbc00], np.uint16)
    cfg, st, _ = _one_block_step(g, 2, flags=O.FLAG_NO_EF)
    row = st.G.reshape(2, -1)[1]
    np.testing.assert_array_equal(row & 0xffff, [1, 2])          # the two lowest-index NaNs
    np.testing.assert_array_equal(row >> 16, [0x7fc0, 0x7fc0])


def test_quantizer_codes_are_defined_outside_the_range():
    # the step never quantizes outside [lo, hi] with a finite range; the piece
    # still gives every input a defined code (no float-to-int conversion of NaN)
    x = np.array([np.nan, -np.inf, -1.0, 0.0, 0.5, 1.0, 2.0, np.inf], np.float32)
    c = O.quant_group(x, 1, 1, 0, 0, np.float32(0.0), np.float32(1.0))
    np.testing.assert_array_equal(c[[0, 1, 2]], [0, 0, 0])
    np.testing.assert_array_equal(c[[5, 6, 7]], [15, 15, 15])
    assert c[3] == 0 and c[4] in (7, 8)
