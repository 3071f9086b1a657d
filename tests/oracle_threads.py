"""The oracle's full step with its blocks spread over threads (test
infrastructure).

One oracle step over all d (`orc_step`) is, per block j in turn, the oracle's
per-block step `orc_block_step` on that block's parameters, gradients, codes,
statistics and window segment; blocks share no state under per-block
statistics, and the C function keeps none of its own (its scratch is
allocated per call).  Running the same per-block calls for disjoint block
ranges in several threads therefore gives the single-threaded step's result
exactly; ctypes releases the GIL while the C code runs.  With an even B_d no
code byte holds nibbles of two blocks, so the threads write disjoint bytes."""
from __future__ import annotations

import ctypes as C
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle as O


def default_threads() -> int:
    """Threads for the oracle: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_step_threaded(cfg, t: int, theta: np.ndarray, g: np.ndarray, ef: np.ndarray,
                         stats: np.ndarray, G: np.ndarray, threads: int | None = None) -> None:
    """Step t (1-based) of the oracle over all blocks, in place on theta (fp32
    [d]), ef (codes, ceil(d/2) bytes), stats (2 per block) and G (window,
    m*k); g holds the step's bf16 gradients [d]."""
    assert cfg.B % 2 == 0, "an odd B_d puts two blocks' nibbles in one byte"
    assert not (cfg.flags & O.FLAG_GLOBAL_QUANT), "the global quantizer couples the blocks"
    for a, dt, n in ((theta, np.float32, cfg.d), (g, np.uint16, cfg.d), (ef, np.uint8, (cfg.d + 1) // 2),
                     (stats, np.float32, 2 * O.num_blocks(cfg)), (G, np.uint32, cfg.m * cfg.k)):
        assert a.dtype == dt and a.size == n and a.flags["C_CONTIGUOUS"]
    nb = O.num_blocks(cfg)
    lib = O.lib()
    tb, gb, eb, sb, Gb = (a.ctypes.data for a in (theta, g, ef, stats, G))
    cfgp = C.byref(cfg)

    def run(rng):
        for j in range(*rng):
            s, _ = O.block_range(cfg, j)
            off, _ = O.block_quota(cfg, j)
            rc = lib.orc_block_step(cfgp, t, j, C.c_void_p(tb + 4 * s), C.c_void_p(gb + 2 * s), C.c_void_p(eb),
                                    s, C.c_void_p(sb + 8 * j), C.c_void_p(Gb + 4 * off), cfg.k, None, None)
            if rc != 0:
                raise ValueError(f"oracle rejected the configuration (rc={rc})")

    n = threads or default_threads()
    parts = min(nb, 8 * n)
    edges = [nb * p // parts for p in range(parts + 1)]
    with ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(run, [(edges[p], edges[p + 1]) for p in range(parts) if edges[p] < edges[p + 1]]))
