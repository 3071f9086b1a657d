"""Shared helpers for the GPU parity tests: run the HIP library and the CPU
oracle on the same seeded inputs and compare them element by element.

Bars (from the step's definition): Top-k indices, packed 4-bit codes, block
statistics and the window contents bit-exact; m_hat, v_hat and the updated
parameters within 1e-6 relative (|gpu - cpu| <= 1e-6 * max(|cpu|, 1e-30)),
and so is the applied step theta_t - theta_{t-1} relative to the oracle's
step.  Every path of the library computes these bitwise equal to the oracle
(same fp32 operations in the same order), and the runners below assert that
too.  A NaN is compared by class: both sides NaN passes, whatever the payload
(the hardware's NaN propagation is not part of the method)."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle as O
from oracle_threads import oracle_step_threaded
from memory_compressed_adaptive_amd import MicroAdam
from memory_compressed_adaptive_amd import _lib as L
from memory_compressed_adaptive_amd import synth

REL_TOL = 1e-6


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gauss_grads(rng, d, t, scale=1e-3, outlier=0.01):
    g = (rng.standard_normal(d) * scale).astype(np.float32)
    g[rng.random(d) < outlier] *= 50
    return O.bf16_rne(g)


def assert_bits_equal(name, got, ref):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} != {ref.shape}"
    bad = np.flatnonzero(got.view(np.uint8) != ref.view(np.uint8)) if got.dtype != ref.dtype else \
        np.flatnonzero(got != ref)
    if bad.size:
        i = int(bad[0])
        raise AssertionError(f"{name}: {bad.size} mismatches, first at {i}: gpu={got.ravel()[i]!r} "
                             f"cpu={ref.ravel()[i]!r}")


def assert_close_f32(name, got, ref):
    """Within 1e-6 relative; returns the number of elements that are not
    bitwise equal (two NaNs count as equal)."""
    got = np.asarray(got, np.float32).ravel()
    ref = np.asarray(ref, np.float32).ravel()
    assert got.shape == ref.shape, f"{name}: shape {got.shape} != {ref.shape}"
    # bitwise-equal elements pass; the tolerance is checked on the others only
    diff = np.flatnonzero(got.view(np.uint32) != ref.view(np.uint32))
    if diff.size == 0:
        return 0
    gn, rn = np.isnan(got[diff]), np.isnan(ref[diff])
    if (gn != rn).any():
        i = int(diff[np.flatnonzero(gn != rn)[0]])
        raise AssertionError(f"{name}: NaN on one side only at {i}: gpu={got[i]!r} cpu={ref[i]!r}")
    diff = diff[~gn]
    if diff.size == 0:
        return 0
    g64 = got[diff].astype(np.float64)
    r64 = ref[diff].astype(np.float64)
    ok = np.abs(g64 - r64) <= REL_TOL * np.maximum(np.abs(r64), 1e-30)
    if not ok.all():
        i = int(diff[np.flatnonzero(~ok)[0]])
        raise AssertionError(f"{name}: {int((~ok).sum())} outside 1e-6 rel, first at {i}: "
                             f"gpu={got[i]!r} cpu={ref[i]!r}")
    return int(diff.size)


def assert_step_close(name, got, ref, prev_got, prev_ref):
    """The applied step theta_t - theta_{t-1} of each side (in double, from the
    fp32 values) within 1e-6 of the oracle's step, relative to that step."""
    got = np.asarray(got, np.float32).ravel().astype(np.float64)
    ref = np.asarray(ref, np.float32).ravel().astype(np.float64)
    dg = got - np.asarray(prev_got, np.float32).ravel()
    dr = ref - np.asarray(prev_ref, np.float32).ravel()
    fin = np.isfinite(dg) & np.isfinite(dr)
    bad = fin & ~(np.abs(dg - dr) <= REL_TOL * np.maximum(np.abs(dr), 1e-30))
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{name}: {int(bad.sum())} applied steps outside 1e-6 rel, first at {i}: "
                             f"gpu step={dg[i]!r} cpu step={dr[i]!r}")


def check_theta(name, got, ref, prev_got, prev_ref):
    n = assert_close_f32(name, got, ref)
    assert_step_close(name + " step", got, ref, prev_got, prev_ref)
    return n


def to_gpu_bf16(g_bits: np.ndarray, misalign: bool = False):
    t = torch.from_numpy(np.ascontiguousarray(g_bits).view(np.int16))
    if not misalign:
        return t.cuda()
    buf = torch.empty(t.numel() + 1, dtype=torch.int16, device="cuda")
    buf[1:].copy_(t.cuda())
    return buf[1:]


def full_parity(label, d, B, k, m, steps, *, lr=1e-4, wd=0.0, beta1=0.9, beta2=0.999, eps=1e-8,
                seed=42, flags=0, grad_fn=None, rng_seed=0, moments=True, misalign=False,
                gpu_only_flags=0, chunks=None, global_quant=False):
    """Full-state comparison after every step.  Returns the optimizer's exported
    state and the final parameters for further checks."""
    rng = np.random.default_rng(rng_seed)
    grad_fn = grad_fn or gauss_grads
    theta0 = (rng.standard_normal(d) * 0.02).astype(np.float32)
    opt = MicroAdam(d, B, k, m, beta1=beta1, beta2=beta2, eps=eps, lr=lr, wd=wd, seed=seed)
    opt.set_flags(flags | gpu_only_flags | (L.MA_FLAG_GLOBAL_QUANT if global_quant else 0))
    if chunks is not None:
        opt.set_pipeline(chunks)
    cfg = O.make_cfg(d, B, k, m, 4, beta1, beta2, eps, lr, wd, seed,
                     (flags & O.FLAG_NO_EF) | (O.FLAG_GLOBAL_QUANT if global_quant else 0))
    orc = O.FullState(cfg)
    assert opt.state_bytes() == O.state_bytes(cfg)
    theta_gpu = torch.from_numpy(theta0.copy()).cuda()
    theta_cpu = theta0.copy()
    nb = opt.num_blocks
    mblocks = np.unique(np.array([0, nb // 2, nb - 1], np.int64))
    nonbitwise = 0
    for t in range(1, steps + 1):
        g = grad_fn(rng, d, t)
        g_gpu = to_gpu_bf16(g, misalign)
        say(f"[{label}] step {t}: d={d} B={B} k={k} m={m} wd={wd} flags={flags | gpu_only_flags} "
            f"misalign={misalign} chunks={chunks}")
        prev_gpu = theta_gpu.cpu().numpy()
        prev_cpu = theta_cpu.copy()
        opt.step(theta_gpu, g_gpu)
        torch.cuda.synchronize()
        mh, vh = orc.step(theta_cpu, g, moments=True)
        assert opt.t == orc.t == t
        assert_bits_equal(f"{label} t={t} window", opt.window(), orc.G)
        assert_bits_equal(f"{label} t={t} codes", opt.codes_bytes(), orc.ef)
        if global_quant:
            # the one pair is stored as every block's statistics
            gs = opt.stats().reshape(-1, 2).view(np.uint32)
            assert_bits_equal(f"{label} t={t} stats", gs, np.broadcast_to(orc.stats.view(np.uint32), gs.shape))
        else:
            assert_bits_equal(f"{label} t={t} stats", opt.stats().view(np.uint32), orc.stats.view(np.uint32))
        nonbitwise += check_theta(f"{label} t={t} theta", theta_gpu.cpu().numpy(), theta_cpu, prev_gpu, prev_cpu)
        if moments:
            gm, gv = opt.moments(mblocks)
            gm, gv = gm.cpu().numpy(), gv.cpu().numpy()
            for q, j in enumerate(mblocks):
                s, n = O.block_range(cfg, int(j))
                nonbitwise += assert_close_f32(f"{label} t={t} m_hat[{j}]", gm[q, :n], mh[s:s + n])
                nonbitwise += assert_close_f32(f"{label} t={t} v_hat[{j}]", gv[q, :n], vh[s:s + n])
    assert nonbitwise == 0, f"{label}: {nonbitwise} values within tolerance but not bitwise equal"
    return opt, theta_gpu, theta_cpu, nonbitwise


def sampled_parity(label, workload: synth.Workload, m, steps, every=397, check_moments=True, jump=None):
    """Full-size run on the GPU; the oracle follows a deterministic block
    sample (every `every`-th block plus the first and last) exactly, since the
    blocks are independent.  `steps` steps from t = 1; then, if jump =
    (t0, n), both sides are set to step t0 (ma_set_step, the oracle's t) and
    run n more, so that late window rows and the wrap of the row index t mod
    m are written and compared without running t0 steps."""
    w = workload
    d, B, k = w.d, w.block, w.k
    theta = torch.empty(d, dtype=torch.float32, device="cuda")
    synth.fill_params(theta)
    g = torch.empty(d, dtype=torch.int16, device="cuda")
    src = synth.GradSource(w)
    opt = MicroAdam(d, B, k, m)
    cfg = O.make_cfg(d, B, k, m)
    nb = opt.num_blocks
    blocks = synth.sample_blocks(nb, every)
    ranges = [O.block_range(cfg, int(j)) for j in blocks]
    idx = torch.from_numpy(np.concatenate([np.arange(s, s + n) for s, n in ranges])).cuda()
    torch.cuda.synchronize()
    th_all = theta.index_select(0, idx).cpu().numpy()
    states, thetas, pos = {}, {}, 0
    for j, (s, n) in zip(blocks, ranges):
        states[int(j)] = O.BlockState.zeros(cfg, int(j))
        thetas[int(j)] = th_all[pos:pos + n].copy()
        pos += n
    schedule = list(range(1, steps + 1))
    if jump is not None:
        t0, n_more = jump
        assert t0 >= steps
        schedule += list(range(t0 + 1, t0 + n_more + 1))
    nonbitwise = 0
    rows_written = set()
    for t in schedule:
        if t != opt.t + 1:
            say(f"[{label}] both sides jump to step {t - 1}")
            opt.set_step(t - 1)
            for bs in states.values():
                bs.t = t - 1
        rows_written.add(t % m)
        say(f"[{label}] step {t}: {w.name} d={d} m={m} row {t % m} sampled blocks={len(blocks)}")
        src.fill(g, t)
        torch.cuda.synchronize()
        g_all = g.index_select(0, idx).cpu().numpy().view(np.uint16)
        th_prev = theta.index_select(0, idx).cpu().numpy()
        opt.step(theta, g)
        torch.cuda.synchronize()
        th_gpu = theta.index_select(0, idx).cpu().numpy()
        stats = opt.stats()
        mh_gpu = vh_gpu = None
        if check_moments:
            mg, vg = opt.moments(blocks)
            mh_gpu, vh_gpu = mg.cpu().numpy(), vg.cpu().numpy()
        pos = 0
        for q, (j, (s, n)) in enumerate(zip(blocks, ranges)):
            j = int(j)
            bs = states[j]
            th_prev_cpu = thetas[j].copy()
            mh, vh = bs.step(thetas[j], g_all[pos:pos + n], moments=True)
            nonbitwise += check_theta(f"{label} t={t} theta[{j}]", th_gpu[pos:pos + n], thetas[j],
                                      th_prev[pos:pos + n], th_prev_cpu)
            pos += n
            off, kb = O.block_quota(cfg, j)
            for i in range(m):
                assert_bits_equal(f"{label} t={t} window row {i} block {j}",
                                  opt.window(i * k + off, kb), bs.gseg[i])
            nib0 = s & 1
            b0 = s >> 1
            nbytes = (nib0 + n + 1) // 2
            gcodes = O.unpack_nibbles(opt.codes_bytes(b0, nbytes), n, nib0)
            assert_bits_equal(f"{label} t={t} codes block {j}", gcodes, bs.codes())
            assert_bits_equal(f"{label} t={t} stats block {j}", stats[2 * j:2 * j + 2].view(np.uint32),
                              bs.stats.view(np.uint32))
            if check_moments:
                nonbitwise += assert_close_f32(f"{label} t={t} m_hat[{j}]", mh_gpu[q, :n], mh)
                nonbitwise += assert_close_f32(f"{label} t={t} v_hat[{j}]", vh_gpu[q, :n], vh)
    del opt
    assert nonbitwise == 0, f"{label}: {nonbitwise} values within tolerance but not bitwise equal"
    return rows_written


def full_state_parity(label, workload: synth.Workload, m, steps, threads=None, jump=None):
    """Full-size run on the GPU against the oracle's whole state: every block,
    the oracle's blocks stepped on several threads (oracle_threads).  After
    every step the window, the codes and the block statistics are compared
    bit for bit and every parameter (and its applied step) within 1e-6
    relative, bitwise in fact.  jump = (t0, n): as in sampled_parity."""
    w = workload
    d, B, k = w.d, w.block, w.k
    theta = torch.empty(d, dtype=torch.float32, device="cuda")
    synth.fill_params(theta)
    g = torch.empty(d, dtype=torch.int16, device="cuda")
    src = synth.GradSource(w)
    opt = MicroAdam(d, B, k, m)
    cfg = O.make_cfg(d, B, k, m)
    torch.cuda.synchronize()
    theta_cpu = theta.cpu().numpy().copy()
    orc = O.FullState(cfg)
    schedule = list(range(1, steps + 1))
    if jump is not None:
        t0, n_more = jump
        assert t0 >= steps
        schedule += list(range(t0 + 1, t0 + n_more + 1))
    nonbitwise = 0
    for t in schedule:
        if t != opt.t + 1:
            say(f"[{label}] both sides jump to step {t - 1}")
            opt.set_step(t - 1)
        say(f"[{label}] step {t}: {w.name} d={d} m={m} row {t % m}, all {opt.num_blocks} blocks")
        src.fill(g, t)
        torch.cuda.synchronize()
        g_cpu = g.cpu().numpy().view(np.uint16)
        prev_gpu = theta.cpu().numpy()
        prev_cpu = theta_cpu.copy()
        opt.step(theta, g)
        torch.cuda.synchronize()
        t0_ = time.perf_counter()
        oracle_step_threaded(cfg, t, theta_cpu, g_cpu, orc.ef, orc.stats, orc.G, threads)
        say(f"[{label}] step {t}: oracle {time.perf_counter() - t0_:.1f} s")
        assert_bits_equal(f"{label} t={t} window", opt.window(), orc.G)
        assert_bits_equal(f"{label} t={t} codes", opt.codes_bytes(), orc.ef)
        assert_bits_equal(f"{label} t={t} stats", opt.stats().view(np.uint32), orc.stats.view(np.uint32))
        nonbitwise += check_theta(f"{label} t={t} theta", theta.cpu().numpy(), theta_cpu, prev_gpu, prev_cpu)
    del opt
    assert nonbitwise == 0, f"{label}: {nonbitwise} values within tolerance but not bitwise equal"
    return nonbitwise
