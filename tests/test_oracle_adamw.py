"""Pins of the oracle's fp32 AdamW baseline (the comparison optimizer of the
MicroAdam page's second paragraph): torch.optim.AdamW on the CPU (the same
algorithm, rounded in a different order) and the recurrence in double."""
import numpy as np
import torch

import oracle as O


def _run(d, steps, lr, wd, seed=0):
    rng = np.random.default_rng(seed)
    theta = (rng.standard_normal(d) * 0.02).astype(np.float32)
    gs = [O.bf16_rne((rng.standard_normal(d) * 10.0 ** rng.uniform(-4, -2)).astype(np.float32))
          for _ in range(steps)]
    return theta, gs


def test_adamw_matches_torch_adamw():
    d, lr, wd = 5000, 1e-3, 0.01
    theta, gs = _run(d, 12, lr, wd)
    th = theta.copy()
    m = np.zeros(d, np.float32)
    v = np.zeros(d, np.float32)
    p = torch.nn.Parameter(torch.from_numpy(theta.copy()))
    opt = torch.optim.AdamW([p], lr=lr, betas=(0.9, 0.999), eps=1e-8, weight_decay=wd, foreach=False)
    for t, g in enumerate(gs, start=1):
        prev = th.copy()
        O.adamw_step(t, th, g, m, v, lr=lr, wd=wd)
        p.grad = torch.from_numpy(O.bf16_to_f32(g).astype(np.float32))
        opt.step()
        ref = p.detach().numpy()
        # same algorithm, different rounding order: within a few ulps of the
        # operands of the last subtraction plus a few ulps (fp32) of the step;
        # the weight decay term alone (2e-7) is 50 ulps of a parameter
        step_ref = ref.astype(np.float64) - prev
        scale = np.maximum(np.abs(prev), np.abs(step_ref)).astype(np.float32)
        tol = 4 * np.spacing(scale).astype(np.float64) + 4e-6 * np.abs(step_ref)
        assert np.all(np.abs(th.astype(np.float64) - ref) <= tol), t
        # a planted sign error in the step would be far outside that bound
        assert np.abs(step_ref).max() > 100 * np.spacing(scale).max()
        p.data.copy_(torch.from_numpy(th))   # follow the oracle's trajectory


def test_adamw_matches_double_recurrence():
    d, lr, wd = 3000, 2e-3, 0.1
    theta, gs = _run(d, 8, lr, wd, seed=1)
    th = theta.copy()
    m = np.zeros(d, np.float32)
    v = np.zeros(d, np.float32)
    M = np.zeros(d)
    V = np.zeros(d)
    for t, g in enumerate(gs, start=1):
        x = th.astype(np.float64)
        O.adamw_step(t, th, g, m, v, lr=lr, wd=wd)
        gd = O.bf16_to_f32(g).astype(np.float64)
        # the hyperparameters are fp32 values; the recurrence in double
        b1, b2 = float(np.float32(0.9)), float(np.float32(0.999))
        lr_, wd_, eps_ = float(np.float32(lr)), float(np.float32(wd)), float(np.float32(1e-8))
        mag1 = b1 * np.abs(M) + (1 - b1) * np.abs(gd)
        M = b1 * M + (1 - b1) * gd
        V = b2 * V + (1 - b2) * gd * gd
        ref = x * (1 - lr_ * wd_) - lr_ * (M / (1 - b1 ** t)) / (np.sqrt(V / (1 - b2 ** t)) + eps_)
        assert np.all(np.abs(m - M) <= 1e-6 * mag1)
        assert np.all(np.abs(v - V) <= 1e-6 * V + 1e-38)
        step = np.abs(ref - x)
        scale = np.maximum(np.abs(x), step).astype(np.float32)
        assert np.all(np.abs(th - ref) <= 4e-6 * step + 4 * np.spacing(scale).astype(np.float64))
        M, V = m.astype(np.float64), v.astype(np.float64)   # follow the fp32 moments


def _deq(cm, cv, sm, sr):
    q = np.repeat(np.arange(sm.size), O.Q8_BLOCK)[:cm.size]
    qm = (sm / np.float32(127.0)).astype(np.float32)[q]
    qr = (sr / np.float32(255.0)).astype(np.float32)[q]
    ro = (cv.astype(np.float32) * qr).astype(np.float32)
    return (cm.astype(np.float32) * qm).astype(np.float32), (ro * ro).astype(np.float32), qm, qr


def test_adamw8_is_adamw_on_the_dequantized_moments():
    # the step equals the fp32 AdamW step (pinned above) applied to the
    # dequantized moments; the new moments are then within half a code step
    rng = np.random.default_rng(7)
    n = 3 * O.Q8_BLOCK + 77
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    nq = -(-n // O.Q8_BLOCK)
    cm = np.zeros(n, np.int8)
    cv = np.zeros(n, np.uint8)
    sm = np.zeros(nq, np.float32)
    sr = np.zeros(nq, np.float32)
    for t in range(1, 9):
        g = O.bf16_rne((rng.standard_normal(n) * 10.0 ** rng.uniform(-4, -2)).astype(np.float32))
        m0, v0, _, _ = _deq(cm, cv, sm, sr)
        th_ref, m_ref, v_ref = th.copy(), m0.copy(), v0.copy()
        O.adamw_step(t, th_ref, g, m_ref, v_ref, lr=1e-3, wd=0.01)
        O.adamw8_step(t, th, g, cm, cv, sm, sr, lr=1e-3, wd=0.01)
        assert np.array_equal(th.view(np.uint32), th_ref.view(np.uint32)), t
        # scales are the block maxima of the new moments
        for q in range(nq):
            sl = slice(q * O.Q8_BLOCK, min(n, (q + 1) * O.Q8_BLOCK))
            assert sm[q] == np.abs(m_ref[sl]).max()
            assert sr[q] == np.sqrt(v_ref[sl]).max()
            assert np.abs(cm[sl]).max() == 127 and cv[sl].max() == 255
        m1, v1, qm, qr = _deq(cm, cv, sm, sr)
        # half a code step, plus the rounding of the fp32 scales (|code| * 2 ulp <= 3e-5 step)
        assert np.all(np.abs(m1.astype(np.float64) - m_ref) <= 0.5 * qm * (1 + 1e-4))
        r1 = (cv.astype(np.float32) * qr).astype(np.float64)   # the dequantized sqrt(v)
        assert np.all(np.abs(r1 - np.sqrt(v_ref)) <= 0.5 * qr * (1 + 1e-4) + 1e-30)


def test_adamw8_rounds_to_nearest_not_toward_zero():
    # a planted truncation would put codes up to a whole step off; nearest
    # rounding keeps the mean code error near zero
    rng = np.random.default_rng(9)
    n = 64 * O.Q8_BLOCK
    th = np.zeros(n, np.float32)
    cm, cv = np.zeros(n, np.int8), np.zeros(n, np.uint8)
    sm, sr = np.zeros(n // O.Q8_BLOCK, np.float32), np.zeros(n // O.Q8_BLOCK, np.float32)
    g = O.bf16_rne(rng.standard_normal(n).astype(np.float32))
    O.adamw8_step(1, th, g, cm, cv, sm, sr)
    m_true = (np.float32(1 - np.float32(0.9)) * O.bf16_to_f32(g)).astype(np.float32)
    m1, _, qm, _ = _deq(cm, cv, sm, sr)
    err = (m1 - m_true) / qm
    assert abs(err.mean()) < 0.02 and np.abs(err).max() <= 0.5 + 1e-4
