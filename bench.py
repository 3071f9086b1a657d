"""Benchmark: MicroAdam optimizer steps/s on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama2_7b] [--m 10]

A step is one full MicroAdam step (accumulate the 4-bit error, block Top-k,
requantize, window write, AdamStats and the AdamW update) over the whole flat
parameter vector of the workload (default: the LLaMA-2-7B-shaped set, m = 10,
k = d/100, B_d = 16384), with parameters, gradients and optimizer state
resident in HBM before the timed region.  Gradients come from a pool of
pre-generated seeded synthetic steps, cycled.

Prints ONE JSON line with steps/s (value), the dominant kernel's roofline
(algorithmic bytes per launch / its average HIP-event duration, against
8 TB/s), the CPU oracle timed on a bounded block sample of the same workload
(cpu_baseline) and the oracle-vs-GPU check of those sampled blocks after the
run (parity_sampled).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "MicroAdam optimizer steps/s at LLaMA-2-7B shape (m=10,k=d/100); HBM GB/s vs peak"
# the sources a committed counter summary was measured on: the kernels and the
# host code that chooses and launches them
KERNEL_SRCS = [os.path.join(ROOT, "memory_compressed_adaptive_amd", "csrc", f)
               for f in ("microadam_kernels.hpp", "microadam.hip")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha():
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(workload: str, m: int, variant: bool, kernels):
    """Counter-measured HBM bytes per launch, if a committed summary exists for
    the current kernel source (null once the kernels have changed).  The
    summaries are of the default step (fp32 parameters, per-block quantizer,
    sparse update, no decay): a variant run, or one whose kernels are not the
    ones the summary measured, gets none."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}_m{m}.json")
    if variant or not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_source_sha() or set(t.get("kernels", {})) != set(kernels):
        return None
    return t


def oracle_follow(cfg, blocks, ranges, th0, grads, bf16=False):
    """The CPU oracle (single-threaded) on the sampled blocks through every
    step: th0 the blocks' initial parameters (concatenated), grads the list of
    each step's gradients of those blocks.  Returns the blocks' states, their
    parameters and the seconds it took."""
    import numpy as np
    import oracle as O
    states = {int(j): O.BlockState.zeros(cfg, int(j)) for j in blocks}
    ths, pos = [], 0
    for (s0, n) in ranges:
        ths.append(th0[pos:pos + n].copy())
        pos += n
    c0 = time.perf_counter()
    for gh in grads:
        pos = 0
        for q, (j, (s0, n)) in enumerate(zip(blocks, ranges)):
            if bf16:
                # widen, fp32 step, round to nearest even once
                th32 = O.bf16_to_f32(ths[q]).astype(np.float32)
                states[int(j)].step(th32, gh[pos:pos + n])
                ths[q] = O.bf16_rne(th32)
            else:
                states[int(j)].step(ths[q], gh[pos:pos + n])
            pos += n
    return states, ths, time.perf_counter() - c0


def sampled_parity_check(opt, cfg, blocks, ranges, th_gpu, states, ths, bf16=False):
    """The sampled blocks' parameters, codes, statistics and window rows of the
    GPU run against the oracle's after the same steps."""
    import numpy as np
    import oracle as O
    m, k = cfg.m, cfg.k
    stats_gpu = opt.stats()
    bad = {"theta": 0, "codes": 0, "stats": 0, "window": 0}
    nonbitwise = 0
    pos = 0
    for q, (j, (s0, n)) in enumerate(zip(blocks, ranges)):
        j = int(j)
        bs = states[j]
        got = th_gpu[pos:pos + n]
        ref = ths[q]
        pos += n
        if bf16:
            same = got == ref
            close = same
        else:
            same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
            close = np.abs(got.astype(np.float64) - ref) <= 1e-6 * np.maximum(np.abs(ref), 1e-30)
        bad["theta"] += int((~(same | close)).sum())
        nonbitwise += int((~same).sum())
        codes = O.unpack_nibbles(opt.codes_bytes(s0 >> 1, ((s0 & 1) + n + 1) // 2), n, s0 & 1)
        bad["codes"] += int((codes != bs.codes()).sum())
        bad["stats"] += int((stats_gpu[2 * j:2 * j + 2].view(np.uint32) != bs.stats.view(np.uint32)).sum())
        off, kb = O.block_quota(cfg, j)
        for i in range(m):
            bad["window"] += int((opt.window(i * k + off, kb) != bs.gseg[i]).sum())
    return {"blocks": len(blocks), "ok": not any(bad.values()) and nonbitwise == 0, "mismatches": bad,
            "theta_not_bitwise": nonbitwise}


def traffic_for(workload, m, kern_names):
    """Counter bytes per step from a committed summary that matches the current
    source and the kernels this run used, else None."""
    t = load_traffic(workload, m, False, kern_names)
    if t is None:
        return None
    return sum(v["fetch_bytes"] + v["write_bytes"] for v in t["kernels"].values())


# The five workloads of the step's configurations, at 1 GPU: each at its own
# window and step count (LLaMA-2-13B over the window sweep).  The headline
# line is LLaMA-2-7B; these are reported beside it in "configs".
CONFIG_RUNS = [("tiny", 10), ("bert_base", 10), ("opt_1_3b", 10), ("llama2_13b", 1), ("llama2_13b", 10),
               ("llama2_13b", 20), ("llama2_13b", 37)]


def run_config(name, m, dev, copy_gbps, oracle_block_steps=1200, cpu_leg=True):
    """One configuration: m steps fill the window, 2 warmup steps, then the
    configuration's step count K.  Every step takes fresh gradients from the
    generator, produced before the step and outside its timing: each timed
    step is bracketed by HIP events on the step's stream.  The oracle follows a
    block sample through every step (parity and its extrapolated rate)."""
    import numpy as np
    import torch

    import oracle as O
    from memory_compressed_adaptive_amd import MicroAdam
    from memory_compressed_adaptive_amd import synth

    w = synth.WORKLOADS[name]
    d, B, k = w.d, w.block, w.k
    K, W = w.steps, 2
    n_all = m + W + K
    theta = torch.empty(d, dtype=torch.float32, device=dev)
    synth.fill_params(theta)
    g = torch.empty(d, dtype=torch.int16, device=dev)
    gsrc = synth.GradSource(w)
    opt = MicroAdam(d, B, k, m)
    nb = opt.num_blocks
    cfg = O.make_cfg(d, B, k, m)
    every = max(1, nb // max(8, oracle_block_steps // n_all))
    blocks = synth.sample_blocks(nb, every)
    ranges = [(int(j) * B, min(B, d - int(j) * B)) for j in blocks]
    idx = torch.from_numpy(np.concatenate([np.arange(s, s + n) for s, n in ranges])).to(dev)
    th0 = theta.index_select(0, idx).cpu().numpy()
    grads = []
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for s in range(n_all):
        gsrc.fill(g, s + 1)
        if cpu_leg:
            grads.append(g.index_select(0, idx).cpu().numpy().view(np.uint16))
        i = s - (m + W)
        if i == 0:
            torch.cuda.synchronize()
            opt.set_timing(True)
            opt.set_count_touched(True)
        if i >= 0:
            evs[i][0].record()
        opt.step(theta, g)
        if i >= 0:
            evs[i][1].record()
    torch.cuda.synchronize()
    ms_steps = [a.elapsed_time(b) for a, b in evs]
    ms = sum(ms_steps) / K
    kt = opt.kernel_times()
    touched = opt.touched_count() / K
    opt.set_count_touched(False)
    opt.set_timing(False)
    fused = kt["step_fused"][1] > 0
    kern_names = [n for n in ("step_fused", "compress", "adamstats_apply") if kt[n][1] > 0]
    bytes_step = 2 * d + 2 * ((d + 1) // 2) + 4 * k + 16 * nb + 4 * m * k + 8 * touched
    sps = 1e3 / ms
    out = {"workload": name, "d": d, "m": m, "k": k, "steps": K, "ms_per_step": round(ms, 4),
           "steps_per_s": round(sps, 2), "params_per_s": round(d * sps, 1),
           "path": "fused" if fused else "two-kernel",
           "algorithmic_GB_per_step": round(bytes_step / 1e9, 4),
           "algorithmic_GBps": round(bytes_step * sps / 1e9, 1),
           "algorithmic_frac_of_peak": round(bytes_step * sps / 1e9 / HBM_PEAK_GBPS, 4),
           "touched_fraction": round(touched / d, 5),
           "kernels_ms_per_step": {n: round(kt[n][0] / K, 4) for n in kt if kt[n][1] > 0}}
    cb = traffic_for(name, m, kern_names)
    out["counter_GB_per_step"] = None if cb is None else round(cb / 1e9, 3)
    out["counter_GBps"] = None if cb is None else round(cb * sps / 1e9, 1)
    out["counter_frac_of_peak"] = None if cb is None else round(cb * sps / 1e9 / HBM_PEAK_GBPS, 4)
    out["counter_frac_of_copy"] = None if cb is None else round(cb * sps / 1e9 / copy_gbps, 4)
    if cpu_leg:
        th_gpu = theta.index_select(0, idx).cpu().numpy()
        states, ths, secs = oracle_follow(cfg, blocks, ranges, th0, grads)
        out["parity_sampled"] = dict(sampled_parity_check(opt, cfg, blocks, ranges, th_gpu, states, ths),
                                     steps=n_all)
        out["cpu_baseline"] = {"value": round(1.0 / (secs / (len(blocks) * n_all) * nb), 6), "unit": "steps/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{len(blocks)} of {nb} blocks x {n_all} steps, {secs:.1f} s, "
                                         f"extrapolated to all blocks"}
    opt.close()
    del theta, g, gsrc
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log(f"config {name} m={m}: {sps:.2f} steps/s ({ms:.3f} ms), {out['algorithmic_GBps']} GB/s algorithmic, "
        f"parity ok={out.get('parity_sampled', {}).get('ok')}")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama2_7b")
    ap.add_argument("--m", type=int, default=None)
    ap.add_argument("--pool", type=int, default=0,
                    help="distinct pre-generated gradient steps (default: one per step, as memory allows)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-blocks", type=int, default=0,
                    help="blocks in the oracle sample (default: about 10000 block-steps of oracle work)")
    ap.add_argument("--dense", action="store_true", help="stream all parameters in the update")
    ap.add_argument("--bf16-params", action="store_true",
                    help="bfloat16 parameters (ma_step_bf16): the one-40-GB-GPU regime")
    ap.add_argument("--wd", type=float, default=0.0, help="decoupled weight decay (dense update)")
    ap.add_argument("--optimizer", choices=("microadam", "adamw", "adamw8"), default="microadam",
                    help="adamw / adamw8: the page's fp32 and 8-bit AdamW comparison points, same harness")
    ap.add_argument("--global-quant", action="store_true",
                    help="one (delta, Delta) over all d (two compressor passes); no oracle leg")
    ap.add_argument("--chunks", type=int, default=0,
                    help="block ranges whose update overlaps the next range's compression (0: library default)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other configurations (the `configs` array of the default line)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the MicroAdam step needs no communication "
              "(every block is independent); several GPUs would each own a contiguous range of blocks, "
              "which is not implemented here.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from memory_compressed_adaptive_amd import MicroAdam
    from memory_compressed_adaptive_amd import _lib as L
    from memory_compressed_adaptive_amd import synth

    w = synth.WORKLOADS[args.workload]
    m = args.m or w.m
    K = args.steps or w.steps
    W = args.warmup
    d, B, k = w.d, w.block, w.k
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"workload={w.name} d={d} B_d={B} k={k} m={m} steps={K} warmup={W}")

    # ---------------- HBM copy ceiling (plain streaming copy, same process)
    n_copy = 1 << 30
    src = torch.empty(n_copy, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1.0)
    synth.copy_f32(dst, src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        synth.copy_f32(dst, src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * 4 * n_copy / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    log(f"copy kernel: {copy_gbps:.0f} GB/s")

    if args.optimizer in ("adamw", "adamw8"):
        bench_adamw(args, w, K, W, copy_gbps, dev)
        return

    # ---------------- inputs resident in HBM
    theta = torch.empty(d, dtype=torch.float32, device=dev)
    synth.fill_params(theta)
    if args.bf16_params:
        # bfloat16 parameters: the seeded fp32 values rounded to nearest even
        theta = theta.to(torch.bfloat16).view(torch.int16)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    gsrc = synth.GradSource(w)
    free, _ = torch.cuda.mem_get_info()
    state_est = (d + 1) // 2 + 4 * m * k + 64 * (d // B + 1)
    fit = int((free - state_est - (8 << 30)) // (2 * d))
    n_steps = m + W + K
    P = max(1, min(args.pool or n_steps, n_steps, fit))
    pool = []
    for p in range(P):
        g = torch.empty(d, dtype=torch.int16, device=dev)
        gsrc.fill(g, p + 1)
        pool.append(g)
    torch.cuda.synchronize()
    log(f"inputs ready: theta {4 * d / 2**30:.1f} GiB, {P} gradient steps {2 * d * P / 2**30:.1f} GiB")

    opt = MicroAdam(d, B, k, m, wd=args.wd)
    flags = (L.MA_FLAG_FORCE_DENSE if args.dense else 0) | (L.MA_FLAG_GLOBAL_QUANT if args.global_quant else 0)
    if flags:
        opt.set_flags(flags)
    if args.chunks:
        opt.set_pipeline(args.chunks)
    nb = opt.num_blocks

    # The window holds m rows; before the timed region the optimizer state is
    # brought to steady state (every row written) by m untimed steps, then the
    # W warmup steps run.
    F = m
    n_pre = F + W

    # oracle sample: initial parameters and every pooled gradient of the sampled blocks
    # (the block-sampled oracle cannot follow the global quantizer: its pair
    # depends on every block)
    cpu_leg = not args.no_cpu_baseline and not args.global_quant
    if cpu_leg:
        want = args.cpu_blocks or max(16, 10000 // (n_pre + K))
        every = max(1, nb // max(1, want))
        blocks = synth.sample_blocks(nb, every)
        ranges = [(int(j) * B, min(B, d - int(j) * B)) for j in blocks]
        idx = torch.from_numpy(np.concatenate([np.arange(s, s + n) for s, n in ranges])).to(dev)
        th0 = theta.index_select(0, idx).cpu().numpy()
        if args.bf16_params:
            th0 = th0.view(np.uint16)
        g_host = [g.index_select(0, idx).cpu().numpy().view(np.uint16) for g in pool]

    # ---------------- fill the window, warmup, then exactly K timed steps
    for s in range(n_pre):
        opt.step(theta, pool[s % P])
    torch.cuda.synchronize()
    opt.set_timing(True)
    opt.set_count_touched(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(n_pre, n_pre + K):
        opt.step(theta, pool[s % P])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    kt = opt.kernel_times()
    touched = opt.touched_count() / K
    opt.set_count_touched(False)
    opt.set_timing(False)
    steps_per_s = K / elapsed
    log(f"{K} steps in {elapsed * 1e3:.2f} ms: {steps_per_s:.2f} steps/s")

    # ---------------- roofline of the dominant kernel
    # Per-kernel times are HIP events recorded on the stream each kernel runs
    # on, around every launch of the timed region.  When the update of one
    # block range overlaps the compression of the next (two-kernel path), both
    # durations include the time the two kernels share the device.
    bytes_c = 2 * d + 2 * ((d + 1) // 2) + 4 * k + 16 * nb       # g, codes r+w, window row, stats r+w
    if args.global_quant:
        bytes_c += 2 * d + (d + 1) // 2 + 16 * nb                # second pass: g and codes again, cut
    # global quantizer: the first pass reads g and the codes and writes the
    # window row and each block's min / max and cut; the second reads g and
    # the codes again and writes the codes and statistics
    bytes_c1 = 2 * d + (d + 1) // 2 + 4 * k + 16 * nb
    bytes_c2 = bytes_c - bytes_c1
    pb = 2 if args.bf16_params else 4                            # bytes per parameter
    if args.wd:
        bytes_a = 4 * m * k + 2 * pb * d                        # window read, every parameter r+w
    else:
        bytes_a = 4 * m * k + 2 * pb * touched                  # window read, touched parameters r+w
    # Full blocks run as one fused kernel (compress + update per block) when
    # the library takes that path; the kernels then share the bytes by blocks.
    if kt["step_fused"][1] > 0 and args.global_quant:
        # the first pass fused with the update; the second pass alone
        n_full = d // B
        f = n_full / nb
        kern = {"step_fused": f * (bytes_c1 + bytes_a), "compress": bytes_c2 + (1 - f) * bytes_c1,
                "adamstats_apply": (1 - f) * bytes_a}
    elif kt["step_fused"][1] > 0:
        n_full = d // B
        f = n_full / nb
        kern = {"step_fused": f * (bytes_c + bytes_a), "compress": (1 - f) * bytes_c,
                "adamstats_apply": (1 - f) * bytes_a}
    else:
        kern = {"compress": bytes_c, "adamstats_apply": bytes_a}
    kern = {n: b for n, b in kern.items() if kt[n][1] > 0}
    launches = {n: kt[n][1] / K for n in kern}                  # launches per step
    ms_step = {n: kt[n][0] / K for n in kern}                   # summed launch time per step
    dom = max(kern, key=lambda n: ms_step[n])
    bytes_launch = kern[dom] / launches[dom]
    ms_launch = kt[dom][0] / kt[dom][1]
    achieved = bytes_launch / (ms_launch * 1e-3) / 1e9
    traffic = load_traffic(w.name, m, bool(args.dense or args.global_quant or args.bf16_params or args.wd), kern)
    traffic_bytes = None
    if traffic is not None and dom in traffic.get("kernels", {}):
        kt_ = traffic["kernels"][dom]
        traffic_bytes = (kt_["fetch_bytes"] + kt_["write_bytes"]) / launches[dom]
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": None if traffic_bytes is None else int(traffic_bytes),
                "bytes_per_launch": int(bytes_launch), "avg_launch_ms": round(ms_launch, 4),
                "launches_per_step": launches[dom]}
    step_bytes = bytes_c + bytes_a
    hbm = {"algorithmic_GB_per_step": round(step_bytes / 1e9, 3),
           "algorithmic_GBps": round(step_bytes * steps_per_s / 1e9, 1),
           "algorithmic_frac_of_peak": round(step_bytes * steps_per_s / 1e9 / HBM_PEAK_GBPS, 4),
           "copy_kernel_GBps": round(copy_gbps, 1),
           "touched_fraction": round(touched / d, 5),
           "kernels_ms_per_step": {n: round(ms_step[n], 4) for n in kern},
           "kernels_algorithmic_GBps": {n: round(kern[n] / (ms_step[n] * 1e-3) / 1e9, 1) for n in kern}}
    if traffic is not None:
        tot = sum(v["fetch_bytes"] + v["write_bytes"] for v in traffic["kernels"].values())
        hbm["counter_GB_per_step"] = round(tot / 1e9, 3)
        hbm["counter_GBps_at_step_rate"] = round(tot * steps_per_s / 1e9, 1)
        hbm["counter_frac_of_peak"] = round(tot * steps_per_s / 1e9 / HBM_PEAK_GBPS, 4)
        hbm["counter_frac_of_copy"] = round(tot * steps_per_s / 1e9 / copy_gbps, 4)
        hbm["counter_note"] = ("counted bytes exceed the algorithmic ones by access granularity: the touched "
                               "parameters (a tenth, spread uniformly) lie on nearly every 128-byte line, and "
                               "the fused kernel reads and writes those lines whole, which measured faster "
                               "than writing back their dirty 32-byte sectors")

    result = {
        "metric": METRIC, "value": round(steps_per_s, 3), "unit": "steps/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(elapsed * 1e3 / K, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "d": d, "B_d": B, "k": k, "m": m, "b": 4,
                   "grad_pool": P, "update": "dense" if args.dense else "sparse",
                   "quantizer": "global" if args.global_quant else "per block",
                   "params": "bf16" if args.bf16_params else "f32", "wd": args.wd,
                   "path": "fused" if "step_fused" in kern else "two-kernel",
                   # block ranges whose update overlaps the next range's compression: the
                   # two-kernel path only (the fused kernel has none)
                   "overlap_ranges": None if "step_fused" in kern else opt.pipeline,
                   "window_filled_before_warmup": F},
        "params_per_s": round(d * steps_per_s, 1),
        "state_bytes": opt.state_bytes(),
        "resident_bytes": {"params": pb * d, "grads_one_step": 2 * d, "state": opt.state_bytes(),
                           "aux": opt.aux_bytes()},
        "hbm": hbm,
        "roofline": roofline,
    }

    # ---------------- CPU baseline: the oracle on the sampled blocks, same inputs
    if cpu_leg:
        import oracle as O
        log(f"oracle on {len(blocks)} sampled blocks x {n_pre + K} steps ...")
        th_gpu = theta.index_select(0, idx).cpu().numpy()
        if args.bf16_params:
            th_gpu = th_gpu.view(np.uint16)
        cfg = O.make_cfg(d, B, k, m, wd=args.wd)
        states, ths, secs = oracle_follow(cfg, blocks, ranges, th0, [g_host[s % P] for s in range(n_pre + K)],
                                          bf16=args.bf16_params)
        per_block_step = secs / (len(blocks) * (n_pre + K))
        cpu_steps_per_s = 1.0 / (per_block_step * nb)
        result["cpu_baseline"] = {
            "value": round(cpu_steps_per_s, 6), "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(blocks)} of {nb} blocks (every {every}th, plus first and last) x {n_pre + K} steps "
                      f"of {w.name}; {secs:.1f} s single-threaded, extrapolated to all blocks",
            "host_cpus": os.cpu_count()}
        result["parity_sampled"] = dict(sampled_parity_check(opt, cfg, blocks, ranges, th_gpu, states, ths,
                                                             bf16=args.bf16_params), steps=n_pre + K)
        log(f"cpu baseline {cpu_steps_per_s:.5f} steps/s (extrapolated); parity ok={result['parity_sampled']['ok']}")

    # ---------------- the other configurations, one after another
    default_line = not (args.dense or args.global_quant or args.bf16_params or args.wd or args.chunks
                        or args.m or args.workload != "llama2_7b")
    if default_line and not args.no_configs:
        opt.close()
        del theta, pool
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        result["configs"] = [run_config(nm, mm, dev, copy_gbps, cpu_leg=cpu_leg) for nm, mm in CONFIG_RUNS]
    opt.close()
    print(json.dumps(result), flush=True)


def bench_adamw(args, w, K, W, copy_gbps, dev):
    """The fp32 AdamW baseline (ma_adamw_step) on the same parameters and
    gradients: 8 bytes of state per parameter, 26 bytes moved per parameter."""
    import numpy as np
    import torch

    from memory_compressed_adaptive_amd import synth
    from memory_compressed_adaptive_amd.baselines import Q8_BLOCK, adamw8_step, adamw_step

    d = w.d
    q8 = args.optimizer == "adamw8"
    theta = torch.empty(d, dtype=torch.float32, device=dev)
    synth.fill_params(theta)
    if q8:
        nq = -(-d // Q8_BLOCK)
        st = (torch.zeros(d, dtype=torch.int8, device=dev), torch.zeros(d, dtype=torch.uint8, device=dev),
              torch.zeros(nq, dtype=torch.float32, device=dev), torch.zeros(nq, dtype=torch.float32, device=dev))

        def one(g, t):
            adamw8_step(theta, g, *st, t, lr=1e-4, wd=args.wd)
    else:
        m = torch.zeros(d, dtype=torch.float32, device=dev)
        v = torch.zeros_like(m)

        def one(g, t):
            adamw_step(theta, g, m, v, t, lr=1e-4, wd=args.wd)
    gsrc = synth.GradSource(w)
    free, _ = torch.cuda.mem_get_info()
    P = max(1, min(K + W, int((free - (8 << 30)) // (2 * d))))
    pool = []
    for p in range(P):
        g = torch.empty(d, dtype=torch.int16, device=dev)
        gsrc.fill(g, p + 1)
        pool.append(g)
    # oracle sample: a contiguous run (AdamW is elementwise)
    n_s = min(d, 1 << 21) if not args.no_cpu_baseline else 0
    th_s = theta[:n_s].cpu().numpy().copy() if n_s else None
    g_s = [g[:n_s].cpu().numpy().view(np.uint16) for g in pool] if n_s else None
    torch.cuda.synchronize()
    for s in range(W):
        one(pool[s % P], s + 1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for s in range(W, W + K):
        one(pool[s % P], s + 1)
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_launch = e0.elapsed_time(e1) / K
    steps_per_s = K / elapsed
    # parameter r+w, gradient, moments r+w (fp32: 4 B each; 8-bit: 1 B each + scales)
    bytes_step = (8 + 2 + 4 + 16 * (-(-d // Q8_BLOCK)) / d) * d if q8 else 26 * d
    bytes_step = int(bytes_step)
    achieved = bytes_step / (ms_launch * 1e-3) / 1e9
    result = {
        "metric": METRIC + (" (comparison: 8-bit AdamW)" if q8 else " (comparison: fp32 AdamW)"), "value": round(steps_per_s, 3), "unit": "steps/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(elapsed * 1e3 / K, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "d": d, "optimizer": "adamw 8-bit" if q8 else "adamw fp32", "wd": args.wd,
                   "grad_pool": P},
        "params_per_s": round(d * steps_per_s, 1),
        "state_bytes": 2 * d + 8 * (-(-d // Q8_BLOCK)) if q8 else 8 * d,
        "roofline": {"bound": "hbm", "kernel": "adamw8" if q8 else "adamw", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "bytes_per_launch": bytes_step, "avg_launch_ms": round(ms_launch, 4), "launches_per_step": 1},
        "hbm": {"copy_kernel_GBps": round(copy_gbps, 1)},
    }
    if n_s:
        import oracle as O
        mo = np.zeros(n_s, np.float32)
        vo = np.zeros(n_s, np.float32)
        ns_q = -(-n_s // Q8_BLOCK)
        q8s = (np.zeros(n_s, np.int8), np.zeros(n_s, np.uint8), np.zeros(ns_q, np.float32),
               np.zeros(ns_q, np.float32))
        c0 = time.perf_counter()
        for s in range(W + K):
            if q8:
                O.adamw8_step(s + 1, th_s, g_s[s % P], *q8s, lr=1e-4, wd=args.wd)
            else:
                O.adamw_step(s + 1, th_s, g_s[s % P], mo, vo, lr=1e-4, wd=args.wd)
        c1 = time.perf_counter()
        got = theta[:n_s].cpu().numpy()
        result["cpu_baseline"] = {
            "value": round(1.0 / ((c1 - c0) / (W + K) * d / n_s), 6), "unit": "steps/s", "cores": 1,
            "kind": "oracle", "host_cpus": os.cpu_count(),
            "sample": f"the first {n_s} of {d} parameters x {W + K} steps, {c1 - c0:.1f} s single-threaded, "
                      f"extrapolated to all parameters"}
        result["parity_sampled"] = {"elements": n_s, "steps": W + K,
                                    "ok": bool(np.array_equal(got.view(np.uint32), th_s.view(np.uint32)))}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
