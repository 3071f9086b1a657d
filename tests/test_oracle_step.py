"""Pins of the oracle's full step: the window ring, AdamStats against Adam's
textbook recurrence in double, the closed forms at m = 1 and t = 1, update
sparsity (last paragraph of the MicroAdam page) and the memory arithmetic of
its second paragraph."""
import json
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _grads(rng, d, scale=1e-3, outlier=0.01):
    g = (rng.standard_normal(d) * scale).astype(np.float32)
    g[rng.random(d) < outlier] *= 50
    return O.bf16_rne(g)


def _entries(row):
    return (row & 0xffff).astype(np.int64), O.bf16_to_f32((row >> 16).astype(np.uint16))


def _row_as_dense(cfg, G, i):
    """Scatter window row i of the full G into a dense length-d vector."""
    d = cfg.d
    out = np.zeros(d, np.float64)
    for j in range(O.num_blocks(cfg)):
        s, n = O.block_range(cfg, j)
        off, kb = O.block_quota(cfg, j)
        I, V = _entries(G[i * cfg.k + off: i * cfg.k + off + kb])
        out[s + I] = V
    return out


def test_first_step_accumulator_is_the_gradient():
    # zero initial state: a_1 = g_1 exactly, so the stored values are bf16(g) = g
    rng = np.random.default_rng(20)
    d, B = 50_000, 4096
    cfg = O.make_cfg(d, B, d // 100, 4)
    st = O.FullState(cfg)
    theta = (rng.standard_normal(d) * 0.02).astype(np.float32)
    g = _grads(rng, d)
    st.step(theta, g)
    gf = O.bf16_to_f32(g)
    for j in range(O.num_blocks(cfg)):
        s, n = O.block_range(cfg, j)
        off, kb = O.block_quota(cfg, j)
        I, V = _entries(st.G[1 * cfg.k + off: 1 * cfg.k + off + kb])
        np.testing.assert_array_equal(I, np.sort(O.topk(gf[s:s + n], kb)))
        np.testing.assert_array_equal(V, gf[s + I])


def test_ring_rotation():
    rng = np.random.default_rng(21)
    d, B, m = 20_000, 1000, 3
    cfg = O.make_cfg(d, B, d // 50, m)
    st = O.FullState(cfg)
    theta = (rng.standard_normal(d) * 0.02).astype(np.float32)
    history = []
    for t in range(1, 8):
        before = st.G.copy().reshape(m, -1)
        st.step(theta, _grads(rng, d))
        after = st.G.reshape(m, -1)
        row = t % m
        for i in range(m):
            if i != row:
                np.testing.assert_array_equal(after[i], before[i])
        history.append(after[row].copy())
        # the rows hold exactly the last min(t, m) selections
        held = {tuple(after[i]) for i in range(m) if t >= m or i in [(t - q) % m for q in range(t)]}
        assert held == {tuple(h) for h in history[-min(t, m):]}


def test_adamstats_m1_closed_form_no_ef():
    # m = 1 and no error feedback: m_hat = c1*V and v_hat = c2*V^2 on I_t, 0 elsewhere
    rng = np.random.default_rng(22)
    d, B = 30_000, 2048
    cfg = O.make_cfg(d, B, d // 100, 1, flags=O.FLAG_NO_EF)
    st = O.FullState(cfg)
    theta = (rng.standard_normal(d) * 0.02).astype(np.float32)
    for t in range(1, 6):
        g = _grads(rng, d)
        mh, vh = st.step(theta, g, moments=True)
        _, _, c1, c2, _ = O.step_constants(cfg, t)
        V = _row_as_dense(cfg, st.G, 0).astype(np.float32)
        np.testing.assert_array_equal(mh, c1 * V)
        np.testing.assert_array_equal(vh, c2 * (V * V))
        # no error feedback: the selection is T_k of g itself
        gf = O.bf16_to_f32(g)
        nz = np.flatnonzero(V)
        assert np.all(V[nz] == gf[nz])


@pytest.mark.parametrize("ef", [True, False])
def test_adamstats_matches_adam_recurrence(ef):
    """t <= m: m_hat equals Adam's bias-corrected first moment of the sparse
    gradient sequence s_tau = scatter(I_tau, V_tau); t > m: the window keeps the
    last m terms, i.e. (m_t - beta^m m_{t-m}) / (1 - beta^t).  Same for v_hat
    with beta2 and s^2.  Reference in double from the recurrence."""
    rng = np.random.default_rng(23 + ef)
    d, B, m = 40_000, 4096, 4
    cfg = O.make_cfg(d, B, d // 100, m, flags=0 if ef else O.FLAG_NO_EF)
    b1, b2 = float(np.float32(0.9)), float(np.float32(0.999))
    st = O.FullState(cfg)
    theta = (rng.standard_normal(d) * 0.02).astype(np.float32)
    M1 = [np.zeros(d)]
    M2 = [np.zeros(d)]
    for t in range(1, 11):
        mh, vh = st.step(theta, _grads(rng, d), moments=True)
        s = _row_as_dense(cfg, st.G, t % m)
        M1.append(b1 * M1[-1] + (1 - b1) * s)
        M2.append(b2 * M2[-1] + (1 - b2) * s * s)
        if t <= m:
            ref1, ref2 = M1[t] / (1 - b1 ** t), M2[t] / (1 - b2 ** t)
        else:
            ref1 = (M1[t] - b1 ** m * M1[t - m]) / (1 - b1 ** t)
            ref2 = (M2[t] - b2 ** m * M2[t - m]) / (1 - b2 ** t)
        # fp32 accumulation of at most m terms: error below (m + 4) ulps of the
        # sum of magnitudes
        mag1 = np.zeros(d)
        mag2 = np.zeros(d)
        for r in range(min(t, m)):
            sr = _row_as_dense(cfg, st.G, (t - r) % m)
            mag1 += b1 ** r * np.abs(sr)
            mag2 += b2 ** r * sr * sr
        c1 = (1 - b1) / (1 - b1 ** t)
        c2 = (1 - b2) / (1 - b2 ** t)
        # plus the double reference's own cancellation error when t > m
        dbl1 = 1e-14 * (np.abs(M1[t]) + np.abs(M1[max(t - m, 0)])) / (1 - b1 ** t)
        dbl2 = 1e-14 * (np.abs(M2[t]) + np.abs(M2[max(t - m, 0)])) / (1 - b2 ** t)
        tol1 = (m + 4) * 2.0 ** -24 * c1 * mag1 + dbl1 + 1e-37
        tol2 = (m + 4) * 2.0 ** -24 * c2 * mag2 + dbl2 + 1e-37
        assert np.all(np.abs(mh - ref1) <= tol1)
        assert np.all(np.abs(vh - ref2) <= tol2)


def test_first_update_is_signlike_and_sparse():
    # t = 1: m_hat = V, v_hat = V^2, so theta moves by lr*V/(|V| + eps) on I_1
    rng = np.random.default_rng(24)
    d, B = 60_000, 16384
    cfg = O.make_cfg(d, B, d // 100, 10, lr=1e-4)
    st = O.FullState(cfg)
    theta0 = (rng.standard_normal(d) * 0.02).astype(np.float32)
    theta = theta0.copy()
    g = _grads(rng, d)
    st.step(theta, g)
    V = _row_as_dense(cfg, st.G, 1)
    moved = theta.astype(np.float64) - theta0
    sel = V != 0
    expect = -1e-4 * V[sel] / (np.abs(V[sel]) + 1e-8)
    np.testing.assert_allclose(moved[sel], expect, rtol=0, atol=2e-9)
    assert np.all(np.sign(moved[sel]) == -np.sign(V[sel]))
    # untouched parameters are bitwise unchanged
    np.testing.assert_array_equal(theta[~sel].view(np.uint32), theta0[~sel].view(np.uint32))


def test_update_sparsity_bound():
    # at most m*k parameters change per step: sparsity >= 1 - mk/d (90% at m=10, k=d/100)
    rng = np.random.default_rng(25)
    d, B, m = 2**18, 16384, 10
    cfg = O.make_cfg(d, B, d // 100, m)
    st = O.FullState(cfg)
    theta = (rng.standard_normal(d) * 0.02).astype(np.float32)
    for t in range(1, 16):
        before = theta.copy()
        st.step(theta, _grads(rng, d))
        changed = np.count_nonzero(theta.view(np.uint32) != before.view(np.uint32))
        union = np.zeros(d, bool)
        for i in range(m):
            union |= _row_as_dense(cfg, st.G, i) != 0
        assert changed <= union.sum() <= m * cfg.k
        assert 1 - changed / d >= 1 - m * cfg.k / d >= 0.9 - 1e-3


def test_decoupled_weight_decay_is_dense():
    rng = np.random.default_rng(26)
    d, B = 10_000, 1000
    cfg = O.make_cfg(d, B, d // 100, 5, lr=1e-2, wd=0.1)
    st = O.FullState(cfg)
    theta0 = (rng.standard_normal(d) * 0.02).astype(np.float32)
    theta = theta0.copy()
    st.step(theta, _grads(rng, d))
    V = _row_as_dense(cfg, st.G, 1)
    untouched = V == 0
    decay = np.float32(1 - 1e-3)
    np.testing.assert_array_equal(theta[untouched], theta0[untouched] * decay)


def test_block_state_equals_full_state():
    # blocks are independent: a detached block evolves exactly like its slice
    rng = np.random.default_rng(27)
    d, B, m = 70_001, 4096, 3
    cfg = O.make_cfg(d, B, d // 100, m)
    full = O.FullState(cfg)
    theta = (rng.standard_normal(d) * 0.02).astype(np.float32)
    nb = O.num_blocks(cfg)
    blocks = {j: O.BlockState.zeros(cfg, j) for j in (0, 5, nb - 1)}
    btheta = {j: theta[slice(*(lambda s, n: (s, s + n))(*O.block_range(cfg, j)))].copy() for j in blocks}
    for t in range(1, 7):
        g = _grads(rng, d)
        full.step(theta, g)
        for j, bs in blocks.items():
            s, n = O.block_range(cfg, j)
            bs.step(btheta[j], g[s:s + n])
            np.testing.assert_array_equal(btheta[j], theta[s:s + n])
            off, kb = O.block_quota(cfg, j)
            for i in range(m):
                np.testing.assert_array_equal(bs.gseg[i], full.G[i * cfg.k + off: i * cfg.k + off + kb])
            np.testing.assert_array_equal(bs.codes(), O.unpack_nibbles(full.ef, n, s))
            np.testing.assert_array_equal(bs.stats, full.stats[2 * j: 2 * j + 2])


def test_threaded_full_step_equals_single_threaded():
    # the full-size GPU parity tests step the oracle with its blocks spread over
    # threads; that must be the single-threaded full step exactly, every array
    # bitwise, ragged last block included
    from oracle_threads import oracle_step_threaded
    rng = np.random.default_rng(31)
    d, B, m = 300_001 - 1, 4096, 4     # 74 blocks, the last of 1004 elements
    cfg = O.make_cfg(d, B, d // 100, m)
    full = O.FullState(cfg)
    theta = (rng.standard_normal(d) * 0.02).astype(np.float32)
    th2 = theta.copy()
    ef2 = np.zeros_like(full.ef)
    st2 = np.zeros_like(full.stats)
    G2 = np.zeros_like(full.G)
    for t in range(1, 7):
        g = _grads(rng, d)
        full.step(theta, g)
        oracle_step_threaded(cfg, t, th2, g, ef2, st2, G2, threads=5)
        np.testing.assert_array_equal(th2.view(np.uint32), theta.view(np.uint32))
        np.testing.assert_array_equal(ef2, full.ef)
        np.testing.assert_array_equal(st2.view(np.uint32), full.stats.view(np.uint32))
        np.testing.assert_array_equal(G2, full.G)


def test_odd_block_length_nibbles_straddle():
    # B odd: blocks share EF bytes; per-element nibble order must still hold
    rng = np.random.default_rng(28)
    d, B = 1001, 77
    cfg = O.make_cfg(d, B, 50, 2)
    full = O.FullState(cfg)
    theta = (rng.standard_normal(d) * 0.02).astype(np.float32)
    for _ in range(3):
        full.step(theta, _grads(rng, d))
    codes = O.unpack_nibbles(full.ef, d)
    assert codes.max() <= 15
    # every block's minimum residual maps to code 0 somewhere
    for j in range(O.num_blocks(cfg)):
        s, n = O.block_range(cfg, j)
        assert codes[s:s + n].min() == 0


def test_global_quantizer_lemma1():
    # the literal scalar (delta, Delta) over all of d: Lemma 1 with n = d
    rng = np.random.default_rng(29)
    d, B = 100_000, 8192
    cfg = O.make_cfg(d, B, d // 100, 2, flags=O.FLAG_GLOBAL_QUANT)
    st = O.FullState(cfg)
    assert st.stats.size == 2
    theta = (rng.standard_normal(d) * 0.02).astype(np.float32)
    g = _grads(rng, d)
    st.step(theta, g)
    # reconstruct the residual a_1 = g with the selected entries zeroed
    a = O.bf16_to_f32(g).astype(np.float32).copy()
    V = _row_as_dense(cfg, st.G, 1)
    a[V != 0] = 0
    lo, hi = st.stats
    assert lo == a.min() and hi == a.max()
    xh = O.dequant_group(O.unpack_nibbles(st.ef, d), lo, hi)
    err = np.linalg.norm(xh.astype(np.float64) - a)
    omega = np.sqrt(d - 2) / 15 * (hi - lo) / np.sqrt(float(hi) ** 2 + float(lo) ** 2)
    assert err <= omega * np.linalg.norm(a.astype(np.float64))


def test_global_quantizer_with_one_block_is_block_quantizer():
    # d <= B_d: the pair over all d is the block's pair, so both readings agree
    rng = np.random.default_rng(31)
    d = 5000
    runs = []
    for flags in (0, O.FLAG_GLOBAL_QUANT):
        cfg = O.make_cfg(d, 8192, d // 100, 3, flags=flags)
        st = O.FullState(cfg)
        theta = (np.random.default_rng(3).standard_normal(d) * 0.02).astype(np.float32)
        r = np.random.default_rng(4)
        for t in range(1, 5):
            st.step(theta, _grads(r, d))
        runs.append((theta, st.ef.copy(), st.stats.copy(), st.G.copy()))
    for a, b in zip(*runs):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


def test_state_bytes_and_memory_paragraph():
    with open(os.path.join(GOLDEN, "microadam_memory_paragraph.json")) as f:
        page = json.load(f)
    d = page["llama2_7b_d"]
    m = page["m"]
    k = d // 100
    cfg = O.make_cfg(d, 16384, k, m)
    sb = O.state_bytes(cfg)
    assert sb == (d + 1) // 2 + 4 * m * k
    gib = 2 ** 30
    assert round(sb / gib, 2) == page["microadam_state_GB"]
    assert round(2 * d / gib, 2) == page["adamw_8bit_state_GB"]
    assert round(8 * d / gib, 2) == page["adamw_fp32_state_GB"]
    assert abs(sb / d - page["state_over_d_at_m10"]) < 1e-3
    # break-even window: 0.5d + 4m d/100 < 2d  <=>  m < 37.5
    assert 0.5 + 4 * page["m_max"] / 100 == 2.0
    for mm, below in ((37, True), (38, False)):
        c = O.make_cfg(13015449600, 16384, 13015449600 // 100, mm)
        assert (O.state_bytes(c) < 2 * 13015449600) == below
    assert 1 - m * k / d >= page["min_update_sparsity_at_m10"] - 1e-9


# ---------------------------------------------------------------- error feedback carried across steps

def _compose_step(cfg, t, g, ef_prev, stats_prev, global_q, mistake=None, stats_new=None):
    """Step t's compressor outputs (window row, statistics, unpacked codes),
    composed from separately pinned pieces (the bf16 widening, dequantizer,
    Top-k, bf16 rounding, min / max and quantizer) in the order of the first
    paragraph: a_t = g_t + Q^-1(e_t, delta_t, Delta_t); (I_t, V_t) = T_k(|a_t|);
    zero those entries; e_{t+1} = Q(a_t, delta_{t+1}, Delta_{t+1}).  `mistake`
    plants one plausible error, for the guard test below."""
    d = cfg.d
    nb = O.num_blocks(cfg)
    gf = O.bf16_to_f32(g)
    a = np.empty(d, np.float32)
    row = np.zeros(cfg.k, np.uint32)
    for j in range(nb):
        s, n = O.block_range(cfg, j)
        codes = O.unpack_nibbles(ef_prev, n, s)
        jj = (j + 1) % nb if mistake == "neighbour stats" else j
        src = stats_new if mistake == "new stats" else stats_prev
        lo, hi = (src[0], src[1]) if global_q else (src[2 * jj], src[2 * jj + 1])
        xh = O.dequant_group(codes, lo, hi)
        if mistake == "dropped feedback":
            a[s:s + n] = gf[s:s + n]
        elif mistake == "sign":
            a[s:s + n] = gf[s:s + n] - xh
        else:
            a[s:s + n] = gf[s:s + n] + xh
        off, kb = O.block_quota(cfg, j)
        sel = O.topk(a[s:s + n], kb)
        vb = O.bf16_rne(a[s + sel]).astype(np.uint32)
        row[off:off + kb] = sel.astype(np.uint32) | (vb << 16)
    resid = a.copy()
    for j in range(nb):
        s, n = O.block_range(cfg, j)
        off, kb = O.block_quota(cfg, j)
        sel = (row[off:off + kb] & 0xffff).astype(np.int64)
        if mistake != "quantize before zeroing":
            resid[s + sel] = 0.0
    tq = t - 1 if mistake == "stale step in the generator" else t
    codes_new = np.empty(d, np.uint8)
    if global_q:
        lo, hi = O.group_minmax(resid)
        stats = np.array([lo, hi], np.float32)
    else:
        stats = np.empty(2 * nb, np.float32)
    for j in range(nb):
        s, n = O.block_range(cfg, j)
        if not global_q:
            lo, hi = O.group_minmax(resid[s:s + n])
            stats[2 * j], stats[2 * j + 1] = lo, hi
        codes_new[s:s + n] = O.quant_group(resid[s:s + n], cfg.seed, tq, j, 0, lo, hi)
    return row, stats, codes_new


def _carry_over_run(global_q):
    rng = np.random.default_rng(41 + global_q)
    d, B, m = 50_001, 4096, 3            # 13 blocks, the last of 841 elements
    cfg = O.make_cfg(d, B, d // 100, m, flags=O.FLAG_GLOBAL_QUANT if global_q else 0)
    st = O.FullState(cfg)
    theta = (rng.standard_normal(d) * 0.02).astype(np.float32)
    out = []
    for t in range(1, 5):
        g = _grads(rng, d)
        ef_prev, stats_prev = st.ef.copy(), st.stats.copy()
        st.step(theta, g)
        out.append((t, g, ef_prev, stats_prev, st.G.reshape(m, -1)[t % m].copy(), st.stats.copy(),
                    O.unpack_nibbles(st.ef, d)))
    return cfg, out


@pytest.mark.parametrize("global_q", [False, True])
def test_error_feedback_carries_over_steps(global_q):
    """Steps 2-4 (where e_t != 0) from the previous step's codes and statistics:
    the window row, the new statistics and the new codes all equal the
    composition of the pinned pieces."""
    cfg, out = _carry_over_run(global_q)
    for t, g, ef_prev, stats_prev, row, stats, codes in out:
        if t >= 2:
            assert np.any(ef_prev != 0)         # the feedback is really there
        r, s, c = _compose_step(cfg, t, g, ef_prev, stats_prev, global_q)
        np.testing.assert_array_equal(row, r, err_msg=f"window row, t={t}")
        np.testing.assert_array_equal(stats.view(np.uint32), s.view(np.uint32), err_msg=f"statistics, t={t}")
        np.testing.assert_array_equal(codes, c, err_msg=f"codes, t={t}")


@pytest.mark.parametrize("global_q", [False, True])
@pytest.mark.parametrize("mistake", ["new stats", "sign", "dropped feedback", "neighbour stats",
                                     "quantize before zeroing", "stale step in the generator"])
def test_error_feedback_mistakes_would_be_caught(global_q, mistake):
    # guard for the pin above: each planted mistake changes at least one of the
    # compared outputs on the same inputs at some step t >= 2, so an oracle
    # making it would fail the pin
    if mistake == "neighbour stats" and global_q:
        pytest.skip("one pair over all d: there is no neighbouring block's pair")
    cfg, out = _carry_over_run(global_q)
    caught = False
    for t, g, ef_prev, stats_prev, row, stats, codes in out[1:]:
        r, s, c = _compose_step(cfg, t, g, ef_prev, stats_prev, global_q, mistake, stats_new=stats)
        if not (np.array_equal(row, r) and np.array_equal(stats.view(np.uint32), s.view(np.uint32))
                and np.array_equal(codes, c)):
            caught = True
    assert caught, mistake
