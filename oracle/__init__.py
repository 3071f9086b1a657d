"""MicroAdam CPU oracle -- TEST INFRASTRUCTURE ONLY.

Python (ctypes + numpy) front end of the plain C oracle in microadam_oracle.c.
Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import it.  The product path (the GPU library and its
binding) never does.

The oracle follows the page "MicroAdam (Sparse-Gradient Adaptive Optimization
with Quantized Error Feedback)", first paragraph (the step), second paragraph
(the state it keeps) and third paragraph (the unbiased 4-bit quantizer); the
readings it takes where that page is silent are written next to the C code.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass, field

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle_microadam.so")

FLAG_NO_EF = 1
FLAG_GLOBAL_QUANT = 2

_lib = None


class Cfg(C.Structure):
    _fields_ = [("d", C.c_int64), ("B", C.c_int32), ("m", C.c_int32), ("k", C.c_int64),
                ("b", C.c_int32), ("beta1", C.c_float), ("beta2", C.c_float),
                ("eps", C.c_float), ("lr", C.c_float), ("wd", C.c_float),
                ("seed", C.c_uint64), ("flags", C.c_uint32)]


def lib():
    """Loads the oracle library, building it only when no build exists."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _b
        _b.build()
    L = C.CDLL(LIB_PATH)
    p = C.c_void_p
    i64, u64, u32, f32 = C.c_int64, C.c_uint64, C.c_uint32, C.c_float
    cfgp = C.POINTER(Cfg)
    L.orc_bf16_rne.restype = C.c_uint16
    L.orc_bf16_rne.argtypes = [f32]
    L.orc_philox4x32_10.argtypes = [p, p, p]
    L.orc_pcg_hash.restype = u32
    L.orc_pcg_hash.argtypes = [u32]
    L.orc_block_key.restype = u32
    L.orc_block_key.argtypes = [u64, i64, i64]
    L.orc_xi16.restype = u32
    L.orc_xi16.argtypes = [u64, i64, i64, i64]
    L.orc_floor_mul_div.restype = i64
    L.orc_floor_mul_div.argtypes = [i64, i64, i64]
    L.orc_block_range.argtypes = [cfgp, i64, p, p]
    L.orc_block_quota.argtypes = [cfgp, i64, p, p]
    L.orc_num_blocks.restype = i64
    L.orc_num_blocks.argtypes = [cfgp]
    L.orc_step_constants.argtypes = [cfgp, i64, p, p, p, p, p]
    L.orc_topk.argtypes = [p, i64, i64, p]
    L.orc_quant_group.argtypes = [p, i64, u64, i64, i64, i64, f32, f32, p]
    L.orc_group_minmax.argtypes = [p, i64, p, p]
    L.orc_range_reset.argtypes = [p, p]
    L.orc_dequant_group.argtypes = [p, i64, f32, f32, p]
    L.orc_block_step.restype = C.c_int
    L.orc_block_step.argtypes = [cfgp, i64, i64, p, p, p, i64, p, p, i64, p, p]
    L.orc_adamw_step.restype = None
    L.orc_adamw_step.argtypes = [i64, i64, C.c_float, C.c_float, C.c_float, C.c_float, C.c_float, p, p, p, p]
    L.orc_adamw8_step.restype = None
    L.orc_adamw8_step.argtypes = [i64, i64, C.c_float, C.c_float, C.c_float, C.c_float, C.c_float,
                                  p, p, p, p, p, p]
    L.orc_step.restype = C.c_int
    L.orc_step.argtypes = [cfgp, i64, p, p, p, p, p, p, p]
    L.orc_state_bytes.restype = u64
    L.orc_state_bytes.argtypes = [cfgp]
    L.orc_bf16_rne_array.argtypes = [p, i64, p]
    L.orc_pcg_hash_array.argtypes = [p, i64, p]
    L.orc_xi16_array.argtypes = [u64, i64, i64, i64, i64, p]
    _lib = L
    return L


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)


def make_cfg(d, B, k, m, b=4, beta1=0.9, beta2=0.999, eps=1e-8, lr=1e-4, wd=0.0,
             seed=42, flags=0) -> Cfg:
    return Cfg(int(d), int(B), int(m), int(k), int(b), beta1, beta2, eps, lr, wd,
               int(seed), int(flags))


# ---------------------------------------------------------------- pieces

def bf16_rne(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    out = np.empty(x.size, np.uint16)
    lib().orc_bf16_rne_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def pcg_hash(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint32).ravel()
    out = np.empty(x.size, np.uint32)
    lib().orc_pcg_hash_array(_ptr(x), x.size, _ptr(out))
    return out


def xi16(seed, t, j, local0, n) -> np.ndarray:
    out = np.empty(int(n), np.uint32)
    lib().orc_xi16_array(int(seed), int(t), int(j), int(local0), int(n), _ptr(out))
    return out


def floor_mul_div(k, x, d) -> int:
    return int(lib().orc_floor_mul_div(int(k), int(x), int(d)))


def num_blocks(cfg: Cfg) -> int:
    return int(lib().orc_num_blocks(C.byref(cfg)))


def block_range(cfg: Cfg, j: int):
    s, n = C.c_int64(), C.c_int64()
    lib().orc_block_range(C.byref(cfg), int(j), C.byref(s), C.byref(n))
    return s.value, n.value


def block_quota(cfg: Cfg, j: int):
    off, kb = C.c_int64(), C.c_int64()
    lib().orc_block_quota(C.byref(cfg), int(j), C.byref(off), C.byref(kb))
    return off.value, kb.value


def step_constants(cfg: Cfg, t: int):
    fac1 = np.empty(cfg.m, np.float32)
    fac2 = np.empty(cfg.m, np.float32)
    c1, c2, decay = C.c_float(), C.c_float(), C.c_float()
    lib().orc_step_constants(C.byref(cfg), int(t), _ptr(fac1), _ptr(fac2),
                             C.byref(c1), C.byref(c2), C.byref(decay))
    return fac1, fac2, np.float32(c1.value), np.float32(c2.value), np.float32(decay.value)


def topk(a, kb) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(max(int(kb), 0), np.int32)
    lib().orc_topk(_ptr(a), a.size, int(kb), _ptr(out))
    return out


def group_minmax(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    lo, hi = C.c_float(), C.c_float()
    lib().orc_group_minmax(_ptr(x), x.size, C.byref(lo), C.byref(hi))
    return np.float32(lo.value), np.float32(hi.value)


def quant_group(x, seed, t, j, local0, lo, hi) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.size, np.uint8)
    lib().orc_quant_group(_ptr(x), x.size, int(seed), int(t), int(j), int(local0),
                          float(lo), float(hi), _ptr(out))
    return out


def dequant_group(codes, lo, hi) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.size, np.float32)
    lib().orc_dequant_group(_ptr(codes), codes.size, float(lo), float(hi), _ptr(out))
    return out


def state_bytes(cfg: Cfg) -> int:
    return int(lib().orc_state_bytes(C.byref(cfg)))


def unpack_nibbles(ef: np.ndarray, n: int, nib0: int = 0) -> np.ndarray:
    """Codes of elements 0..n-1 stored from nibble nib0 of ef (low nibble first)."""
    idx = np.arange(n, dtype=np.int64) + nib0
    b = ef[idx >> 1]
    return np.where(idx & 1, b >> 4, b & 15).astype(np.uint8)


# ---------------------------------------------------------------- state

@dataclass
class FullState:
    """The whole optimizer state of the oracle for one (d, B, k, m) config."""
    cfg: Cfg
    ef: np.ndarray = field(default=None)
    stats: np.ndarray = field(default=None)
    G: np.ndarray = field(default=None)
    t: int = 0

    def __post_init__(self):
        c = self.cfg
        nb = num_blocks(c)
        if self.ef is None:
            self.ef = np.zeros((c.d + 1) // 2, np.uint8)
        if self.stats is None:
            n_stats = 2 if (c.flags & FLAG_GLOBAL_QUANT) else 2 * nb
            self.stats = np.zeros(n_stats, np.float32)
        if self.G is None:
            self.G = np.zeros(c.m * c.k, np.uint32)

    def step(self, theta: np.ndarray, g_bf16: np.ndarray, moments: bool = False):
        """One oracle step; theta (fp32) is updated in place.  Returns
        (mhat, vhat) when moments is True."""
        c = self.cfg
        assert theta.dtype == np.float32 and theta.size == c.d and theta.flags["C_CONTIGUOUS"]
        g = np.ascontiguousarray(g_bf16, dtype=np.uint16)
        assert g.size == c.d
        mh = np.empty(c.d, np.float32) if moments else None
        vh = np.empty(c.d, np.float32) if moments else None
        rc = lib().orc_step(C.byref(c), self.t + 1, _ptr(theta), _ptr(g), _ptr(self.ef),
                            _ptr(self.stats), _ptr(self.G), _ptr(mh), _ptr(vh))
        if rc != 0:
            raise ValueError(f"oracle rejected the configuration (rc={rc})")
        self.t += 1
        return (mh, vh) if moments else None

    def step_bf16(self, theta16: np.ndarray, g_bf16: np.ndarray, moments: bool = False):
        """One step for bfloat16 parameters (raw bits, updated in place).  Reading
        (the page's fourth paragraph fine-tunes LLaMA-2 7B on one 40 GB GPU but
        fixes no parameter precision or rounding): widen each parameter exactly
        to fp32, take the fp32 step above, round the result to nearest even
        once."""
        assert theta16.dtype == np.uint16
        th = bf16_to_f32(theta16).astype(np.float32)
        out = self.step(th, g_bf16, moments)
        theta16[:] = bf16_rne(th)
        return out


@dataclass
class BlockState:
    """The oracle's state for ONE block j, detached from the full arrays: its
    codes (as a byte run starting at nibble nib0), its statistics and its
    segment of every window row.  Blocks are independent under per-block
    statistics, so a sample of blocks evolves exactly like the full run."""
    cfg: Cfg
    j: int
    ef: np.ndarray
    nib0: int
    stats: np.ndarray
    gseg: np.ndarray   # [m, kb] uint32
    t: int

    @classmethod
    def zeros(cls, cfg: Cfg, j: int) -> "BlockState":
        s, n = block_range(cfg, j)
        _, kb = block_quota(cfg, j)
        nib0 = s & 1
        return cls(cfg, j, np.zeros((nib0 + n + 1) // 2, np.uint8), nib0,
                   np.zeros(2, np.float32), np.zeros((cfg.m, kb), np.uint32), 0)

    def codes(self) -> np.ndarray:
        _, n = block_range(self.cfg, self.j)
        return unpack_nibbles(self.ef, n, self.nib0)

    def step(self, theta_blk: np.ndarray, g_blk: np.ndarray, moments: bool = False):
        c = self.cfg
        _, n = block_range(c, self.j)
        assert theta_blk.dtype == np.float32 and theta_blk.size == n
        g = np.ascontiguousarray(g_blk, dtype=np.uint16)
        mh = np.empty(n, np.float32) if moments else None
        vh = np.empty(n, np.float32) if moments else None
        gseg = self.gseg
        rc = lib().orc_block_step(C.byref(c), self.t + 1, self.j, _ptr(theta_blk), _ptr(g),
                                  _ptr(self.ef), self.nib0, _ptr(self.stats), _ptr(gseg),
                                  gseg.shape[1], _ptr(mh), _ptr(vh))
        if rc != 0:
            raise ValueError(f"oracle rejected the configuration (rc={rc})")
        self.t += 1
        return (mh, vh) if moments else None


def adamw_step(t, theta, g_bf16, m, v, beta1=0.9, beta2=0.999, eps=1e-8, lr=1e-4, wd=0.0):
    """The fp32 AdamW baseline (orc_adamw_step), in place on theta, m, v."""
    g = np.ascontiguousarray(g_bf16, dtype=np.uint16)
    for a in (theta, m, v):
        assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"] and a.size == g.size
    lib().orc_adamw_step(g.size, int(t), beta1, beta2, eps, lr, wd, _ptr(theta), _ptr(g), _ptr(m), _ptr(v))

Q8_BLOCK = 256


def adamw8_step(t, theta, g_bf16, cm, cv, sm, sr, beta1=0.9, beta2=0.999, eps=1e-8, lr=1e-4, wd=0.0):
    """The 8-bit block-quantized AdamW baseline (orc_adamw8_step), in place:
    theta fp32, cm int8, cv uint8 (n each), sm, sr fp32 (ceil(n/256) each)."""
    g = np.ascontiguousarray(g_bf16, dtype=np.uint16)
    n = g.size
    assert theta.dtype == np.float32 and theta.size == n
    assert cm.dtype == np.int8 and cv.dtype == np.uint8 and cm.size == n and cv.size == n
    assert sm.dtype == np.float32 and sr.dtype == np.float32 and sm.size == sr.size == -(-n // Q8_BLOCK)
    lib().orc_adamw8_step(n, int(t), beta1, beta2, eps, lr, wd, _ptr(theta), _ptr(g), _ptr(cm), _ptr(cv),
                          _ptr(sm), _ptr(sr))
