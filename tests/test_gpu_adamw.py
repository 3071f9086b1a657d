"""GPU parity of the fp32 AdamW baseline (ma_adamw_step) with the oracle's
orc_adamw_step, element by element: aligned runs of 8, ragged tails and
misaligned arrays."""
import numpy as np
import pytest
import torch

import oracle as O
from memory_compressed_adaptive_amd.baselines import adamw_step

from gpu_harness import assert_bits_equal, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _dev(a, misalign):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if not misalign:
        return t.cuda()
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
    buf[1:].copy_(t.cuda())
    return buf[1:]


@pytest.mark.parametrize("n,misalign,wd", [(1, False, 0.0), (7, False, 0.1), (8, False, 0.0),
                                           (1_000_003, False, 0.01), (100_001, True, 0.01),
                                           (3_000_000, False, 0.0)])
def test_adamw_matches_oracle(n, misalign, wd):
    rng = np.random.default_rng(n)
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    th_d, m_d, v_d = _dev(th, misalign), _dev(m, misalign), _dev(v, misalign)
    for t in range(1, 6):
        g = O.bf16_rne((rng.standard_normal(n) * 1e-3).astype(np.float32))
        say(f"[adamw] n={n} misalign={misalign} wd={wd} step {t}")
        adamw_step(th_d, _dev(g.view(np.int16), misalign), m_d, v_d, t, lr=1e-3, wd=wd)
        torch.cuda.synchronize()
        O.adamw_step(t, th, g, m, v, lr=1e-3, wd=wd)
        assert_bits_equal(f"adamw theta t={t}", th_d.cpu().numpy(), th)
        assert_bits_equal(f"adamw m t={t}", m_d.cpu().numpy(), m)
        assert_bits_equal(f"adamw v t={t}", v_d.cpu().numpy(), v)


@pytest.mark.parametrize("n,misalign,wd", [(1, False, 0.0), (255, False, 0.1), (256 * 5, False, 0.0),
                                           (1_000_003, False, 0.01), (100_001, True, 0.01)])
def test_adamw8_matches_oracle(n, misalign, wd):
    from memory_compressed_adaptive_amd.baselines import Q8_BLOCK, adamw8_step
    rng = np.random.default_rng(n + 1)
    nq = -(-n // Q8_BLOCK)
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    cm = np.zeros(n, np.int8)
    cv = np.zeros(n, np.uint8)
    sm = np.zeros(nq, np.float32)
    sr = np.zeros(nq, np.float32)
    d_th, d_cm, d_cv = _dev(th, misalign), _dev(cm, misalign), _dev(cv, misalign)
    d_sm, d_sr = _dev(sm, False), _dev(sr, False)
    for t in range(1, 6):
        g = O.bf16_rne((rng.standard_normal(n) * 10.0 ** rng.uniform(-4, -2)).astype(np.float32))
        say(f"[adamw8] n={n} misalign={misalign} wd={wd} step {t}")
        adamw8_step(d_th, _dev(g.view(np.int16), misalign), d_cm, d_cv, d_sm, d_sr, t, lr=1e-3, wd=wd)
        torch.cuda.synchronize()
        O.adamw8_step(t, th, g, cm, cv, sm, sr, lr=1e-3, wd=wd)
        assert_bits_equal(f"adamw8 theta t={t}", d_th.cpu().numpy(), th)
        assert_bits_equal(f"adamw8 cm t={t}", d_cm.cpu().numpy(), cm)
        assert_bits_equal(f"adamw8 cv t={t}", d_cv.cpu().numpy(), cv)
        assert_bits_equal(f"adamw8 sm t={t}", d_sm.cpu().numpy(), sm)
        assert_bits_equal(f"adamw8 sr t={t}", d_sr.cpu().numpy(), sr)
