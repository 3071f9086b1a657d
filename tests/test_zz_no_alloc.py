"""ma_step_noalloc, the step for callers that cannot allocate (HIP graph
capture, serving loops, harnesses that forbid hipMalloc), against ma_step on
the same inputs through the C ABI: parameters, window, codes and statistics
bit for bit after every step.  Its scratch (the deferred-block list and its
counters, the global quantizer's per-block partials) lives in one static
device array shared by every call on the device, so the cases run back to
back, the second with a smaller input than the first, and include blocks the
fused kernel defers (their list is that scratch) and the global quantizer."""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle as O
from memory_compressed_adaptive_amd import MicroAdam
from memory_compressed_adaptive_amd import _lib as L

from gpu_harness import assert_bits_equal, gauss_grads, say, to_gpu_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _noalloc_fn():
    return L.lib().ma_step_noalloc


def _tied(rng, d, t):
    # blocks 1 and 2 hold one constant value: the fused kernel defers them
    g = gauss_grads(rng, d, t)
    g[16384:3 * 16384] = O.bf16_rne(np.full(2 * 16384, 1e-3, np.float32))
    return g


def _run(label, d, B, k, m, steps, flags=0, wd=0.0, grad_fn=gauss_grads, seed=0):
    say(f"[noalloc {label}] d={d} B={B} k={k} m={m} flags={flags} wd={wd}")
    fn = _noalloc_fn()
    rng = np.random.default_rng(seed)
    theta0 = (rng.standard_normal(d) * 0.02).astype(np.float32)
    lr = 1e-2 if wd else 1e-4
    ref = MicroAdam(d, B, k, m, lr=lr, wd=wd)
    na = MicroAdam(d, B, k, m, lr=lr, wd=wd)
    ref.set_flags(flags)
    na.set_flags(flags)
    th_ref = torch.from_numpy(theta0.copy()).cuda()
    th_na = torch.from_numpy(theta0.copy()).cuda()
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    for t in range(1, steps + 1):
        g = to_gpu_bf16(grad_fn(rng, d, t))
        say(f"[noalloc {label}] step {t}")
        ref.step(th_ref, g)
        rc = fn(na.handle, C.c_void_p(th_na.data_ptr()), C.c_void_p(g.data_ptr()), stream)
        assert rc == L.MA_OK, L.last_error()
        torch.cuda.synchronize()
        assert na.t == ref.t == t
        assert_bits_equal(f"noalloc {label} t={t} theta", th_na.cpu().numpy().view(np.uint32),
                          th_ref.cpu().numpy().view(np.uint32))
        assert_bits_equal(f"noalloc {label} t={t} window", na.window(), ref.window())
        assert_bits_equal(f"noalloc {label} t={t} codes", na.codes_bytes(), ref.codes_bytes())
        assert_bits_equal(f"noalloc {label} t={t} stats", na.stats().view(np.uint32), ref.stats().view(np.uint32))
    ref.close()
    na.close()


def test_noalloc_step_equals_step_fused_then_smaller():
    # fused kernel with deferred blocks and a ragged last block, then a
    # smaller set: the second call starts from the scratch the first left
    _run("fused", 6 * 16384 + 1234, 16384, (6 * 16384 + 1234) // 100, 4, 5, grad_fn=_tied)
    _run("fused, smaller", 3 * 16384 + 77, 16384, (3 * 16384 + 77) // 100, 4, 5, grad_fn=_tied, seed=1)


def test_noalloc_step_equals_step_whole_line_write_back():
    # m = 10: the fused column-sorted kernel writes every parameter line whole
    # (with deferred blocks), then with decay on a smaller set
    _run("whole lines", 6 * 16384 + 1234, 16384, (6 * 16384 + 1234) // 100, 10, 12, grad_fn=_tied)
    _run("whole lines, decay, smaller", 3 * 16384 + 77, 16384, (3 * 16384 + 77) // 100, 10, 11, wd=0.1, seed=3)


def test_noalloc_step_equals_step_two_kernels_and_global():
    # a long window (two kernels, one block range) with decay, then the global
    # quantizer (per-block partials in the scratch) on a smaller set, fused
    # and as separate kernels
    _run("two kernels", 5 * 16384 + 999, 16384, (5 * 16384 + 999) // 100, 37, 4, wd=0.1)
    _run("global", 4 * 16384 + 5, 16384, (4 * 16384 + 5) // 100, 4, 4, flags=L.MA_FLAG_GLOBAL_QUANT,
         grad_fn=_tied)
    _run("global, unfused", 2 * 16384 + 3, 16384, (2 * 16384 + 3) // 100, 3, 4,
         flags=L.MA_FLAG_GLOBAL_QUANT | L.MA_FLAG_UNFUSED, seed=2)


def test_noalloc_step_rejects_more_blocks_than_its_scratch():
    # 2^20 + 1 blocks of 64: beyond the static scratch; rejected before any
    # launch, t unchanged
    d = ((1 << 20) + 1) * 64
    opt = MicroAdam(d, 64, d // 100, 1)
    th = torch.zeros(d, dtype=torch.float32, device="cuda")
    g = torch.zeros(d, dtype=torch.int16, device="cuda")
    rc = _noalloc_fn()(opt.handle, C.c_void_p(th.data_ptr()), C.c_void_p(g.data_ptr()),
                       C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == L.MA_EUNSUPPORTED
    code, msg = L.last_error()
    assert code == L.MA_EUNSUPPORTED and "scratch" in msg
    assert opt.t == 0
    opt.close()
