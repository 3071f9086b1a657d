"""GPU parity: the HIP path against the CPU oracle, element by element, on the
same seeded inputs.  Covers the tiny workload in full, ragged and degenerate
shapes, every kernel variant (chunk counts, aligned and unaligned, sparse and
dense update, the general selection path, multi-pass slot allocation), and
full-size workloads on deterministic block samples."""
import numpy as np
import pytest
import torch

import oracle as O
from memory_compressed_adaptive_amd import MicroAdam
from memory_compressed_adaptive_amd import _lib as L
from memory_compressed_adaptive_amd import synth

from gpu_harness import (assert_bits_equal, assert_close_f32, check_theta, full_parity, full_state_parity,
                         gauss_grads, sampled_parity, say, to_gpu_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_tiny_workload_full_state_20_steps():
    w = synth.WORKLOADS["tiny"]
    full_parity("tiny", w.d, w.block, w.k, w.m, w.steps)


@pytest.mark.parametrize("d,B,k,m,steps", [
    (100_003, 16384, 1000, 3, 6),     # ragged last block (1699 elements)
    (20_011, 1003, 500, 4, 5),        # B odd: code bytes straddle blocks, unaligned path
    (1000, 64, 100, 2, 5),            # tiny blocks
    (1, 1, 1, 1, 3),                  # a single parameter
    (7, 3, 2, 2, 4),                  # every block partial
    (50_000, 4096, 500, 5, 4),        # one chunk per thread
    (50_000, 8192, 500, 5, 4),        # two chunks per thread
    (100_000, 32766, 1000, 3, 4),     # eight chunks per thread, largest B_d
])
def test_ragged_and_small_shapes(d, B, k, m, steps):
    full_parity(f"shape d={d} B={B}", d, B, k, m, steps)


def test_k_zero_only_error_feedback():
    full_parity("k=0", 40_000, 4096, 0, 3, 4)


def test_k_equals_d_selects_everything():
    full_parity("k=d", 5_000, 1024, 5_000, 2, 3)


def test_general_selection_path_large_quota():
    # k_b ~ 1638 > 512: the workgroup-wide bit search
    full_parity("k=d/10", 100_000, 16384, 10_000, 3, 4)


def test_ties_constant_and_few_values():
    def const(rng, d, t):
        return O.bf16_rne(np.full(d, 1e-3 * t, np.float32))

    def few(rng, d, t):
        vals = np.array([0.0, 1e-3, -1e-3, 2e-3, -2e-3], np.float32)
        return O.bf16_rne(vals[rng.integers(0, vals.size, d)])

    full_parity("const grads", 60_000, 16384, 600, 3, 4, grad_fn=const)
    full_parity("few values", 60_000, 16384, 600, 3, 4, grad_fn=few)


def test_all_zero_gradients():
    full_parity("zero grads", 30_000, 8192, 300, 3, 3, grad_fn=lambda r, d, t: np.zeros(d, np.uint16))


def test_m1_no_error_feedback_closed_form():
    d, B, k = 50_000, 16384, 500
    opt, theta_gpu, theta_cpu, _ = full_parity("m=1 no-EF", d, B, k, 1, 4, flags=L.MA_FLAG_NO_EF)
    # the closed form on the GPU's own window: m_hat = c1 V, v_hat = c2 V^2
    cfg = O.make_cfg(d, B, k, 1)
    _, _, c1, c2, _ = O.step_constants(cfg, opt.t)
    G = opt.window()
    mh, vh = opt.moments(np.arange(opt.num_blocks))
    mh, vh = mh.cpu().numpy(), vh.cpu().numpy()
    for j in range(opt.num_blocks):
        off, kb = O.block_quota(cfg, j)
        e = G[off:off + kb]
        I = (e & 0xffff).astype(np.int64)
        V = O.bf16_to_f32((e >> 16).astype(np.uint16))
        np.testing.assert_array_equal(mh[j, I], c1 * V)
        np.testing.assert_array_equal(vh[j, I], c2 * (V * V))


def test_weight_decay_dense_update():
    full_parity("wd dense", 70_000, 16384, 700, 4, 5, lr=1e-2, wd=0.1)


def test_forced_dense_equals_sparse():
    full_parity("force dense", 70_000, 16384, 700, 4, 5, gpu_only_flags=L.MA_FLAG_FORCE_DENSE)


def test_misaligned_gradient_pointer():
    full_parity("misaligned grads", 70_000, 16384, 700, 3, 4, misalign=True)


@pytest.mark.parametrize("chunks,wd,misalign", [
    (5, 0.0, False),      # update of range i overlaps compression of range i+1
    (5, 0.1, False),      # dense update under the overlap
    (3, 0.0, True),       # unaligned gradients: general compressor per range
    (64, 0.0, False),     # more ranges than blocks: one block per range
])
def test_pipelined_step(chunks, wd, misalign):
    # two-kernel path (the fused per-block kernel switched off)
    full_parity(f"pipeline {chunks}", 200_003, 16384, 2000, 4, 5, lr=1e-2 if wd else 1e-4, wd=wd,
                misalign=misalign, chunks=chunks, gpu_only_flags=L.MA_FLAG_UNFUSED)


@pytest.mark.parametrize("B", [4096, 8192, 16384])
def test_fused_step_one_two_four_chunks(B):
    # full blocks through the fused kernel, the ragged last block through the
    # two kernels after it
    d = 31 * B + 1234
    full_parity(f"fused B={B}", d, B, d // 100, 10, 12)


def test_fused_step_with_deferred_blocks():
    # blocks of constant gradients tie massively: the fused kernel defers them
    # (compress and update) to the general compressor and the list update
    def mixed(rng, d, t):
        g = gauss_grads(rng, d, t)
        g[16384:3 * 16384] = O.bf16_rne(np.full(2 * 16384, 1e-3, np.float32))
        return g
    full_parity("fused deferred", 6 * 16384, 16384, 6 * 164, 5, 6, grad_fn=mixed)


@pytest.mark.parametrize("B", [4096, 8192, 16384])
def test_fused_step_with_decay(B):
    # decoupled decay: the fused kernel streams every parameter of its block
    # (dense update), the ragged last block runs the two kernels after it
    d = 31 * B + 1234
    full_parity(f"fused decay B={B}", d, B, d // 100, 10, 12, lr=1e-2, wd=0.1)


@pytest.mark.parametrize("B,wd,flags", [
    (16384, 0.0, 0),                          # parameters through LDS in two chunks
    (16384, 0.0, L.MA_FLAG_FORCE_SPARSE),     # the touched parameters gathered by slot instead
    (16384, 0.1, L.MA_FLAG_FORCE_DENSE),      # every parameter streamed through registers instead
    (8192, 0.1, 0),                           # one chunk, decay on the untouched positions
    (4096, 0.0, 0),
])
def test_fused_parameter_write_back_forms(B, wd, flags):
    # the fused kernel's three forms of the parameter update at m = 10 (fp32,
    # 16-byte aligned) give the oracle's bits
    d = 9 * B + 321
    full_parity(f"fused write-back B={B} wd={wd} flags={flags}", d, B, d // 100, 10, 12, lr=1e-2 if wd else 1e-4,
                wd=wd, gpu_only_flags=flags)


def test_fused_parameters_through_lds_with_nothing_touched():
    # k = 0: no window entries, so no slot; with decay every parameter of the
    # LDS chunks is scaled, without it each is written back unchanged
    full_parity("k=0 decay m=10", 4 * 16384, 16384, 0, 10, 3, lr=1e-2, wd=0.1)
    full_parity("k=0 m=10", 4 * 16384, 16384, 0, 10, 3)


def test_fused_decay_without_error_feedback():
    # the fused kernel's dense update with the error feedback switched off
    full_parity("fused decay no EF", 5 * 16384 + 77, 16384, 900, 6, 8, lr=1e-2, wd=0.1, flags=O.FLAG_NO_EF)


def test_fused_decay_with_deferred_blocks():
    # tie-heavy blocks deferred by the fused kernel get the dense update from the list kernel
    def mixed(rng, d, t):
        g = gauss_grads(rng, d, t)
        g[16384:3 * 16384] = O.bf16_rne(np.full(2 * 16384, 1e-3, np.float32))
        return g
    full_parity("fused decay deferred", 6 * 16384, 16384, 6 * 164, 5, 6, lr=1e-2, wd=0.1, grad_fn=mixed)


@pytest.mark.parametrize("d,B,k,m,misalign,unfused", [
    (100_003, 16384, 1000, 4, False, False),   # full blocks (first pass fused with the update), ragged last block
    (100_003, 16384, 1000, 4, False, True),    # the same, first pass and update as separate kernels
    (3 * 8192, 8192, 600, 2, False, False),    # fused, two chunks per thread, no partial block
    (50_001, 8192, 2000, 3, True, False),      # unaligned gradients, odd d
    (7, 3, 2, 2, False, False),                # every block partial
])
def test_global_quantizer(d, B, k, m, misalign, unfused):
    # one (delta, Delta) over all d: pass 1, global min / max, pass 2
    full_parity(f"global Q d={d} B={B} unfused={unfused}", d, B, k, m, 6, misalign=misalign, global_quant=True,
                gpu_only_flags=L.MA_FLAG_UNFUSED if unfused else 0)


@pytest.mark.parametrize("unfused,misalign", [(False, False), (True, False), (False, True)])
def test_global_quantizer_with_decay(unfused, misalign):
    # decoupled decay: the dense update after (or fused with) the first pass
    full_parity(f"global Q decay unfused={unfused} misalign={misalign}", 100_003, 16384, 1000, 4, 5, lr=1e-2, wd=0.1,
                misalign=misalign, global_quant=True, gpu_only_flags=L.MA_FLAG_UNFUSED if unfused else 0)


@pytest.mark.parametrize("unfused", [False, True])
def test_global_quantizer_with_deferred_blocks(unfused):
    # tie-heavy blocks leave the staged first pass for the general selection
    def mixed(rng, d, t):
        g = gauss_grads(rng, d, t)
        g[16384:3 * 16384] = O.bf16_rne(np.full(2 * 16384, 1e-3, np.float32))
        return g
    full_parity(f"global Q deferred unfused={unfused}", 6 * 16384, 16384, 6 * 164, 4, 5, grad_fn=mixed,
                global_quant=True, gpu_only_flags=L.MA_FLAG_UNFUSED if unfused else 0)


def test_global_quantizer_single_block_equals_block_mode():
    # with one block the global pair is the block's pair: both modes give the same bits
    d, B, k, m = 12_000, 16384, 120, 3
    outs = []
    for gq in (False, True):
        rng = np.random.default_rng(5)
        theta = torch.from_numpy((rng.standard_normal(d) * 0.02).astype(np.float32)).cuda()
        opt = MicroAdam(d, B, k, m)
        if gq:
            opt.set_flags(L.MA_FLAG_GLOBAL_QUANT)
        for t in range(1, 5):
            opt.step(theta, to_gpu_bf16(gauss_grads(rng, d, t)))
        torch.cuda.synchronize()
        outs.append((theta.cpu().numpy(), opt.codes_bytes(), opt.stats(), opt.window()))
    for a, b in zip(*outs):
        assert_bits_equal("block vs global, one block", a, b)


@pytest.mark.parametrize("d,B,k,m,wd,flags,misalign", [
    (100_003, 16384, 1000, 4, 0.0, 0, False),                  # fused kernel + ragged block
    (100_003, 16384, 1000, 4, 0.0, L.MA_FLAG_UNFUSED, False),  # sparse two-kernel update
    (70_000, 16384, 700, 4, 0.1, 0, False),                    # decay: dense update, 16-byte rows
    (70_000, 16384, 700, 4, 0.1, 0, True),                     # decay, parameters 2 bytes off
    (20_011, 1003, 500, 3, 0.0, 0, False),                     # odd B_d
    (100_003, 16384, 1000, 4, 0.0, L.MA_FLAG_GLOBAL_QUANT, False),  # one (delta, Delta) over all d
    (100_003, 16384, 1000, 4, 0.1, L.MA_FLAG_GLOBAL_QUANT, False),  # the same with decay (dense, fused)
    (60_000, 16384, 6000, 37, 0.0, 0, False),                  # window too large for LDS: rows from HBM
    (5 * 16384 + 9, 16384, (5 * 16384 + 9) // 100, 20, 0.0, 0, False),   # fused column-sorted update
    (5 * 16384 + 9, 16384, (5 * 16384 + 9) // 100, 20, 0.1, 0, False),   # the same with decay
])
def test_bf16_parameters(d, B, k, m, wd, flags, misalign):
    # ma_step_bf16: widen, fp32 step, round to nearest even once
    rng = np.random.default_rng(8)
    lr = 1e-2 if wd else 1e-3
    th16 = O.bf16_rne((rng.standard_normal(d) * 0.02).astype(np.float32))
    opt = MicroAdam(d, B, k, m, lr=lr, wd=wd)
    opt.set_flags(flags)
    orc = O.FullState(O.make_cfg(d, B, k, m, 4, 0.9, 0.999, 1e-8, lr, wd, 42,
                                 O.FLAG_GLOBAL_QUANT if flags & L.MA_FLAG_GLOBAL_QUANT else 0))
    th_cpu = th16.copy()
    if misalign:
        buf = torch.empty(d + 1, dtype=torch.int16, device="cuda")
        th_gpu = buf[1:]
    else:
        th_gpu = torch.empty(d, dtype=torch.int16, device="cuda")
    th_gpu.copy_(torch.from_numpy(th16.view(np.int16)))
    changed = 0
    for t in range(1, max(6, m + 3)):
        g = gauss_grads(rng, d, t)
        say(f"[bf16 params] step {t}: d={d} B={B} m={m} wd={wd} flags={flags} misalign={misalign}")
        opt.step(th_gpu, to_gpu_bf16(g))
        torch.cuda.synchronize()
        before = th_cpu.copy()
        orc.step_bf16(th_cpu, g)
        changed += int((before != th_cpu).sum())
        assert_bits_equal(f"bf16 t={t} window", opt.window(), orc.G)
        assert_bits_equal(f"bf16 t={t} codes", opt.codes_bytes(), orc.ef)
        assert_bits_equal(f"bf16 t={t} theta", th_gpu.cpu().numpy().view(np.uint16), th_cpu)
    assert changed > 0


def test_long_window_multi_pass_slots():
    # m * k_b > LDS slots: the update kernel runs several slot passes
    full_parity("m=37 k=d/10", 40_000, 16384, 4_000, 37, 40, moments=True)


@pytest.mark.parametrize("m,steps", [(200, 206), (1024, 1030)])
def test_long_windows_up_to_the_limit(m, steps):
    # 2m decay factors staged in LDS by several waves; the window wraps
    full_parity(f"m={m}", 3_000, 1024, 30, m, steps, moments=False)


@pytest.mark.parametrize("d,k,m,beta1,beta2,eps,lr", [
    (6 * 16384 + 777, 6 * 164, 10, 0.5, 0.95, 1e-3, 1e-2),    # fused kernel
    (4 * 16384, 4 * 164, 37, 0.8, 0.9, 1e-6, 3e-3),            # update kernel, two slot passes
])
def test_other_hyperparameters(d, k, m, beta1, beta2, eps, lr):
    # the decay tables beta^r, the bias factors and eps at values other than
    # the defaults
    full_parity(f"hyper b1={beta1} b2={beta2} eps={eps}", d, 16384, k, m, m + 3,
                beta1=beta1, beta2=beta2, eps=eps, lr=lr)


@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_learning_rate_schedule(wd):
    # ma_set_lr between steps (a scheduler): the step factor and the decoupled
    # decay 1 - lr * wd follow the current lr on both sides
    d, B, k, m = 100_003, 16384, 1000, 4
    rng = np.random.default_rng(21)
    theta0 = (rng.standard_normal(d) * 0.02).astype(np.float32)
    opt = MicroAdam(d, B, k, m, lr=1e-3, wd=wd)
    orc = O.FullState(O.make_cfg(d, B, k, m, 4, 0.9, 0.999, 1e-8, 1e-3, wd, 42, 0))
    th_gpu = torch.from_numpy(theta0.copy()).cuda()
    th_cpu = theta0.copy()
    for t in range(1, 7):
        lr = 1e-3 * 0.6 ** (t - 1)
        opt.set_lr(lr)
        orc.cfg.lr = lr
        g = gauss_grads(rng, d, t)
        say(f"[lr schedule] step {t}: lr={lr:.3g} wd={wd}")
        prev_gpu, prev_cpu = th_gpu.cpu().numpy(), th_cpu.copy()
        opt.step(th_gpu, to_gpu_bf16(g))
        torch.cuda.synchronize()
        orc.step(th_cpu, g)
        assert_bits_equal(f"lr t={t} window", opt.window(), orc.G)
        assert_bits_equal(f"lr t={t} codes", opt.codes_bytes(), orc.ef)
        assert check_theta(f"lr t={t} theta", th_gpu.cpu().numpy(), th_cpu, prev_gpu, prev_cpu) == 0


@pytest.mark.parametrize("B,flags,gq", [
    (16384, 0, False),                  # per-block (delta, Delta), state from the fused kernel
    (1003, 0, False),                   # odd B_d: code bytes straddle blocks
    (16384, 0, True),                   # global quantizer: the one pair in every block's statistics
    (4096, L.MA_FLAG_NO_EF, False),     # no error feedback: a = f32(g)
])
def test_residual_stage_a1(B, flags, gq):
    # the first line of the step on its own: a_t = g_t + Q^-1(e_t, delta_t,
    # Delta_t) from the state after 3 steps, against the oracle's pieces
    d, m = 50_001, 4
    k = d // 100
    rng = np.random.default_rng(31)
    opt = MicroAdam(d, B, k, m)
    opt.set_flags(flags | (L.MA_FLAG_GLOBAL_QUANT if gq else 0))
    no_ef = bool(flags & L.MA_FLAG_NO_EF)
    cfg = O.make_cfg(d, B, k, m, 4, 0.9, 0.999, 1e-8, 1e-4, 0.0, 42,
                     (O.FLAG_NO_EF if no_ef else 0) | (O.FLAG_GLOBAL_QUANT if gq else 0))
    orc = O.FullState(cfg)
    theta0 = (rng.standard_normal(d) * 0.02).astype(np.float32)
    th_gpu = torch.from_numpy(theta0.copy()).cuda()
    th_cpu = theta0.copy()
    for t in range(1, 4):
        g = gauss_grads(rng, d, t)
        opt.step(th_gpu, to_gpu_bf16(g))
        orc.step(th_cpu, g)
    torch.cuda.synchronize()
    assert_bits_equal("a1 state codes", opt.codes_bytes(), orc.ef)
    g4 = gauss_grads(rng, d, 4)
    nb = opt.num_blocks
    blocks = sorted({0, nb // 2, nb - 1})
    say(f"[residual a1] B={B} flags={flags} global={gq} blocks={blocks}")
    got = opt.residual(to_gpu_bf16(g4), blocks).cpu().numpy()
    for q, j in enumerate(blocks):
        s, n = O.block_range(cfg, j)
        gf = O.bf16_to_f32(g4[s:s + n])
        if no_ef:
            want = gf
        else:
            lo, hi = (orc.stats[0], orc.stats[1]) if gq else (orc.stats[2 * j], orc.stats[2 * j + 1])
            want = gf + O.dequant_group(O.unpack_nibbles(orc.ef, n, s), lo, hi)
        assert want.dtype == np.float32
        assert_bits_equal(f"a1 block {j}", got[q, :n], want)
        assert (got[q, n:] == 0).all()
    # the state is unchanged: the next step still matches the oracle
    opt.step(th_gpu, to_gpu_bf16(g4))
    orc.step(th_cpu, g4)
    torch.cuda.synchronize()
    assert_bits_equal("a1 then step, window", opt.window(), orc.G)


def test_run_twice_is_bitwise_deterministic():
    runs = []
    for _ in range(2):
        opt, theta_gpu, _, _ = full_parity("determinism", 60_000, 16384, 600, 4, 6, rng_seed=3,
                                           moments=False)
        runs.append((theta_gpu.cpu().numpy(), opt.export_state()))
    np.testing.assert_array_equal(runs[0][0].view(np.uint32), runs[1][0].view(np.uint32))
    for key in ("codes", "stats", "window"):
        np.testing.assert_array_equal(np.asarray(runs[0][1][key]).view(np.uint8),
                                      np.asarray(runs[1][1][key]).view(np.uint8))


def test_export_import_resume():
    d, B, k, m = 60_000, 16384, 600, 4
    rng = np.random.default_rng(9)
    theta0 = (rng.standard_normal(d) * 0.02).astype(np.float32)
    grads = [gauss_grads(rng, d, t) for t in range(1, 9)]
    a = MicroAdam(d, B, k, m)
    ta = torch.from_numpy(theta0.copy()).cuda()
    for t in range(4):
        a.step(ta, to_gpu_bf16(grads[t]))
    torch.cuda.synchronize()
    st = a.export_state()
    # the one-call export (ma_export_state) equals the buffer-by-buffer reads
    assert st["t"] == 4
    np.testing.assert_array_equal(st["codes"], a.codes_bytes())
    np.testing.assert_array_equal(st["stats"].view(np.uint32), a.stats().view(np.uint32))
    np.testing.assert_array_equal(st["window"], a.window())
    tb = ta.clone()
    b = MicroAdam(d, B, k, m)
    b.import_state(st)
    assert b.t == 4
    say("[resume] continuing both runs for 4 steps")
    for t in range(4, 8):
        a.step(ta, to_gpu_bf16(grads[t]))
        b.step(tb, to_gpu_bf16(grads[t]))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ta.cpu().numpy().view(np.uint32), tb.cpu().numpy().view(np.uint32))
    sa, sb = a.export_state(), b.export_state()
    for key in ("codes", "stats", "window"):
        np.testing.assert_array_equal(np.asarray(sa[key]).view(np.uint8), np.asarray(sb[key]).view(np.uint8))


def test_update_sparsity_on_gpu():
    # at most |union of window rows| <= m*k parameters change per step
    w = synth.WORKLOADS["tiny"]
    opt = MicroAdam(w.d, w.block, w.k, w.m)
    opt.set_count_touched(True)
    theta = torch.empty(w.d, dtype=torch.float32, device="cuda")
    synth.fill_params(theta)
    g = torch.empty(w.d, dtype=torch.int16, device="cuda")
    src = synth.GradSource(w)
    total = 0
    for t in range(1, 16):
        src.fill(g, t)
        before = theta.clone()
        opt.step(theta, g)
        torch.cuda.synchronize()
        changed = int((theta.view(torch.int32) != before.view(torch.int32)).sum())
        touched = opt.touched_count() - total
        total += touched
        assert changed <= touched <= min(t, w.m) * w.k
        assert 1 - changed / w.d >= 1 - w.m * w.k / w.d >= 0.9 - 1e-3


def test_error_codes_on_gpu_handle():
    opt = MicroAdam(1000, 100, 10, 2)
    theta = torch.zeros(1000, dtype=torch.float32, device="cuda")
    g = torch.zeros(1000, dtype=torch.int16, device="cuda")
    lib = L.lib()
    import ctypes as C
    assert lib.ma_step(opt.handle, None, C.c_void_p(g.data_ptr()), None) == L.MA_EINVAL
    assert lib.ma_step(opt.handle, C.c_void_p(theta.data_ptr() + 2), C.c_void_p(g.data_ptr()), None) == L.MA_EINVAL
    assert opt.t == 0
    assert lib.ma_read_state(opt.handle, L.MA_STATE_CODES, 0, 10_000, C.c_void_p(1)) == L.MA_EINVAL
    buf = (C.c_uint8 * 8)()
    assert lib.ma_debug_moments(opt.handle, buf, 1, C.c_void_p(1), C.c_void_p(1), None) == L.MA_EINVAL
    # the binding rejects what the C ABI could not check (host memory, lengths,
    # element sizes) before any call
    for p_, g_ in ((theta.cpu(), g), (theta, g[:999]), (theta, g.float()), (theta.double(), g)):
        with pytest.raises(ValueError):
            opt.step(p_, g_)
    assert opt.t == 0
    opt.step(theta, g)
    torch.cuda.synchronize()
    assert opt.t == 1


def test_create_destroy_does_not_leak():
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(30):
        o = MicroAdam(5_000_000, 16384, 50_000, 10)
        o.close()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free0 - free1 < 64 << 20


# ---------------------------------------------------------------- full-size workloads, sampled blocks

def test_bert_base_sampled():
    sampled_parity("bert_base", synth.WORKLOADS["bert_base"], 10, 4, every=97)


def test_bert_base_full_state():
    # every block, past the window's first wrap (m = 10, 12 steps)
    full_state_parity("bert_base full", synth.WORKLOADS["bert_base"], 10, 12)


def test_opt_1_3b_full_state():
    # three steps from t = 1 (rows 1-3), then both sides jump to t = 10: steps
    # 11-13 wrap the row index and overwrite rows 1-3
    full_state_parity("opt_1_3b full", synth.WORKLOADS["opt_1_3b"], 10, 3, jump=(10, 3))


def test_opt_1_3b_sampled():
    sampled_parity("opt_1_3b", synth.WORKLOADS["opt_1_3b"], 10, 3, every=397, jump=(10, 3))


def test_llama2_7b_sampled():
    # the configured 10 steps, then past the wrap: rows 1 and 2 overwritten
    rows = sampled_parity("llama2_7b", synth.WORKLOADS["llama2_7b"], 10, 10, every=997, jump=(10, 2))
    assert rows == set(range(10))


@pytest.mark.parametrize("m,jump", [(1, (1000, 2)), (10, (7, 5)), (20, (17, 5)), (37, (34, 5))])
def test_llama2_13b_sampled_window_sweep(m, jump):
    # the configured 5 steps per m (rows 1-5), moments checked at every m;
    # then both sides jump to t0 = m - 3: rows m - 2, m - 1 (at element offsets
    # i*k above 2^31 for i >= 17), then the row index wraps onto rows 0-2, of
    # which 1 and 2 were written before
    rows = sampled_parity(f"llama2_13b m={m}", synth.WORKLOADS["llama2_13b"], m, 5, every=3989, jump=jump)
    if m > 1:
        assert max(rows) == m - 1 and 1 in rows
        w = synth.WORKLOADS["llama2_13b"]
        assert m < 17 or (m - 1) * w.k > 2 ** 31


# ---------------------------------------------------------------- non-finite gradients

NAN_BF16 = [0x7fc0, 0xffc0, 0x7f81, 0x7fff, 0xffa5]


def _nonfinite_grads(B):
    big = int(O.bf16_rne(np.array([3.0e38], np.float32))[0])

    def fn(rng, d, t):
        g = gauss_grads(rng, d, t)
        # scattered NaNs (payloads, signs, signalling) and infinities, far
        # fewer than any block's quota: all selected
        n_sp = max(1, d // 3000)
        pos = rng.choice(d, n_sp, replace=False)
        g[pos] = rng.choice(NAN_BF16 + [0x7f80, 0xff80], n_sp)
        nb = -(-d // B)
        blk = lambda j: slice(j * B, min((j + 1) * B, d))
        if nb > 6:
            # block 1: all NaN on odd steps, all +-Inf on even ones
            g[blk(1)] = rng.choice(NAN_BF16, g[blk(1)].size) if t % 2 else rng.choice([0x7f80, 0xff80], g[blk(1)].size)
            # block 2: 300 NaN and 300 infinities: more than the quota
            p = rng.permutation(g[blk(2)].size)
            b2 = g[blk(2)]
            b2[p[:300]] = rng.choice(NAN_BF16, 300)
            b2[p[300:600]] = rng.choice([0x7f80, 0xff80], 300)
            # block 3: +-3e38 on 400 entries each: the residual's range overflows
            p = rng.permutation(g[blk(3)].size)
            b3 = g[blk(3)]
            b3[p[:400]] = big
            b3[p[400:800]] = big | 0x8000
            # block 4: just above a quota of NaNs (the cut falls among NaN keys)
            b4 = g[blk(4)]
            b4[rng.permutation(b4.size)[:B // 96]] = 0x7fc0
            # block 5: NaNs and infinities around the quota (the cut among infinities)
            p = rng.permutation(g[blk(5)].size)
            b5 = g[blk(5)]
            b5[p[:B // 160]] = 0xffc0
            b5[p[B // 160:B // 80]] = 0x7f80
        return g
    return fn


@pytest.mark.parametrize("B,flags,gq,wd,m", [
    (16384, 0, False, 0.0, 4),                  # fused kernel (and the blocks it defers)
    (16384, 0, False, 0.0, 10),                 # fused, parameter lines written whole
    (16384, L.MA_FLAG_UNFUSED, False, 0.0, 4),  # two kernels
    (16384, 0, True, 0.0, 4),                   # one (delta, Delta) over all d
    (16384, 0, False, 0.1, 4),                  # dense update with decay
    (1003, 0, False, 0.0, 4),                   # odd B_d: the general compressor
    (4096, L.MA_FLAG_NO_EF, False, 0.0, 4),     # no error feedback: a = widened g, signalling NaNs kept
])
def test_nonfinite_gradients(B, flags, gq, wd, m):
    # the reading for non-finite values: NaN and +-Inf are selected first (NaN
    # canonical), what is left is dropped from the error feedback, a range with
    # no finite value resets it; window, codes and statistics bit-exact, the
    # parameters NaN where the oracle's are
    d = 7 * B + 777 if B >= 4096 else 60 * B + 17
    oflags = (O.FLAG_NO_EF if flags & L.MA_FLAG_NO_EF else 0)
    full_parity(f"non-finite B={B} flags={flags} global={gq} wd={wd} m={m}", d, B, d // 100, m, m + 1,
                lr=1e-2 if wd else 1e-4, wd=wd, flags=oflags, gpu_only_flags=flags & ~L.MA_FLAG_NO_EF,
                grad_fn=_nonfinite_grads(B), global_quant=gq)


def _tiny_grads(kind):
    # "mixed": a background of 1e-30 with 2 % of the entries at magnitudes
    # log-uniform in 1e-17 .. 1e-12, so the selected values' v_hat fall on
    # both sides of 2^-96 (the square root's two paths, often in one wave);
    # "subnormal": everything in 1e-38 .. 1e-20 (V^2 subnormal or zero)
    def fn(rng, d, t):
        if kind == "mixed":
            mag = np.full(d, 1e-30)
            big = rng.random(d) < 0.02
            mag[big] = 10.0 ** rng.uniform(-17, -12, int(big.sum()))
        else:
            mag = 10.0 ** rng.uniform(-38, -20, d)
        return O.bf16_rne((rng.standard_normal(d) * mag).astype(np.float32))
    return fn


@pytest.mark.parametrize("kind", ["mixed", "subnormal"])
@pytest.mark.parametrize("m,row_sums,wd", [(4, False, 0.0), (4, True, 0.0), (4, False, 0.1), (10, False, 0.0),
                                           (20, False, 0.0), (20, False, 0.1)])
def test_tiny_gradients_square_root_paths(kind, m, row_sums, wd):
    # the update's correctly rounded square root: its fast path where a wave's
    # v_hat are all in [2^-96, FLT_MAX], sqrtf otherwise; both equal the
    # oracle's bit for bit, as do the subnormal sums (row sums and column
    # sums, sparse and dense)
    d, B = 5 * 16384 + 321, 16384
    full_parity(f"tiny grads {kind} m={m} rows={row_sums} wd={wd}", d, B, d // 100, m, m + 2,
                wd=wd, grad_fn=_tiny_grads(kind), gpu_only_flags=L.MA_FLAG_ROW_SUMS if row_sums else 0)


# ---------------------------------------------------------------- the two update algorithms

@pytest.mark.parametrize("d,B,k,m,wd,flags", [
    (200_003, 16384, 2000, 4, 0.0, L.MA_FLAG_UNFUSED),        # sparse update, ragged block
    (200_003, 16384, 2000, 4, 0.1, L.MA_FLAG_UNFUSED),        # dense update (decay)
    (60_000, 16384, 6000, 37, 0.0, 0),                        # m * k_b beyond the column-sorted update's LDS
    (4 * 16384 + 99, 16384, (4 * 16384 + 99) // 100, 37, 0.0, 0),  # m = 37 at k = d/100: several slot passes
    (20_011, 1003, 500, 4, 0.0, L.MA_FLAG_UNFUSED),           # odd B_d
])
@pytest.mark.parametrize("row_sums", [False, True])
def test_update_algorithms(d, B, k, m, wd, flags, row_sums):
    # the column-sorted update (default) and the row-by-row sums
    # (MA_FLAG_ROW_SUMS) against the oracle, with the moments
    full_parity(f"update row_sums={row_sums} d={d} m={m} wd={wd}", d, B, k, m, m + 3, lr=1e-2 if wd else 1e-4,
                wd=wd, gpu_only_flags=flags | (L.MA_FLAG_ROW_SUMS if row_sums else 0))


@pytest.mark.parametrize("label,wd,flags,gq,grad_fn,misalign", [
    ("plain", 0.0, 0, False, None, False),
    ("decay", 0.1, 0, False, None, False),                 # dense update, 16-byte groups
    ("global", 0.0, 0, True, None, False),                 # first pass fused with the update
    ("global decay", 0.1, 0, True, None, False),
    ("no EF", 0.0, L.MA_FLAG_NO_EF, False, None, False),
    ("deferred", 0.0, 0, False, "tied", False),            # tie-heavy blocks: the column-sorted list kernel
])
def test_fused_column_sorted_update(label, wd, flags, gq, grad_fn, misalign):
    # m = 20 at k = d/100: the window does not fit step_full_kernel's LDS, so
    # full blocks run step_csu_kernel (compressor and column-sorted update in
    # one workgroup); the ragged last block runs the two kernels
    def tied(rng, d, t):
        g = gauss_grads(rng, d, t)
        g[16384:3 * 16384] = O.bf16_rne(np.full(2 * 16384, 1e-3, np.float32))
        return g
    d = 6 * 16384 + 777
    full_parity(f"fused csu {label}", d, 16384, d // 100, 20, 23, lr=1e-2 if wd else 1e-4, wd=wd,
                flags=flags & O.FLAG_NO_EF, global_quant=gq, grad_fn=tied if grad_fn == "tied" else None,
                misalign=misalign, moments=True)


def test_fused_column_sorted_update_unaligned_parameters():
    # parameters 4 bytes off a 16-byte boundary: the sparse update element by element
    d, m = 5 * 16384, 20
    k = d // 100
    rng = np.random.default_rng(13)
    theta0 = (rng.standard_normal(d) * 0.02).astype(np.float32)
    opt = MicroAdam(d, 16384, k, m)
    orc = O.FullState(O.make_cfg(d, 16384, k, m))
    buf = torch.empty(d + 1, dtype=torch.float32, device="cuda")
    th_gpu = buf[1:]
    th_gpu.copy_(torch.from_numpy(theta0))
    th_cpu = theta0.copy()
    for t in range(1, m + 4):
        g = gauss_grads(rng, d, t)
        say(f"[fused csu unaligned params] step {t}")
        prev_gpu, prev_cpu = th_gpu.cpu().numpy(), th_cpu.copy()
        opt.step(th_gpu, to_gpu_bf16(g))
        torch.cuda.synchronize()
        orc.step(th_cpu, g)
        assert_bits_equal(f"unaligned t={t} window", opt.window(), orc.G)
        assert_bits_equal(f"unaligned t={t} codes", opt.codes_bytes(), orc.ef)
        assert check_theta(f"unaligned t={t} theta", th_gpu.cpu().numpy(), th_cpu, prev_gpu, prev_cpu) == 0


# ---------------------------------------------------------------- limits

def test_k_zero_long_window_takes_the_two_kernel_path():
    # k = 0 puts nothing in the window rows, but the fused kernel's LDS holds
    # only 64 decay factors: m = 40 must not take it
    full_parity("k=0 m=40", 5 * 4096 + 100, 4096, 0, 40, 3)


def test_create_reports_out_of_memory_and_leaks_nothing():
    # a window far beyond the device's memory: ma_create returns NULL with
    # MA_ENOMEM, and what it allocated before the failing call is released
    torch.cuda.synchronize()
    free0, total = torch.cuda.mem_get_info()
    d = 1 << 37                       # codes 64 GiB (allocates), window 4*m*k = 1 TiB (cannot)
    m = 200
    assert 4 * m * (d // 100) > 2 * total
    say(f"[out of memory] d={d} m={m} device total={total}")
    with pytest.raises(L.MicroAdamError) as ei:
        MicroAdam(d, 16384, d // 100, m)
    assert ei.value.code == L.MA_ENOMEM
    assert L.last_error()[0] == L.MA_ENOMEM
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert abs(free0 - free1) < 64 << 20
    # the library is still usable
    full_parity("after out of memory", 20_000, 4096, 200, 3, 2)
