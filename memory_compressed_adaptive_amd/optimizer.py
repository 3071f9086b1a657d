"""Python handle over libmicroadam: one MicroAdam optimizer for a flat fp32
parameter vector on the GPU.  PyTorch supplies device memory and the stream;
the step itself runs in the library's HIP kernels."""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import _lib as _L


def _stream_handle(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


class MicroAdam:
    """MicroAdam (page "MicroAdam (Sparse-Gradient Adaptive Optimization with
    Quantized Error Feedback)") over a flat parameter vector of length d.

    step(params, grads): params is a contiguous fp32 CUDA tensor of d elements,
    updated in place; grads a contiguous bfloat16 (or int16/uint16 bit
    pattern) CUDA tensor of d elements.
    """

    def __init__(self, d: int, block: int = 16384, k: int | None = None, m: int = 10, b: int = 4,
                 beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8, lr: float = 1e-4,
                 wd: float = 0.0, seed: int = 42):
        self.d = int(d)
        self.block = int(block)
        self.k = int(d // 100 if k is None else k)
        self.m = int(m)
        self.b = int(b)
        self.beta1, self.beta2, self.eps, self.lr, self.wd = beta1, beta2, eps, lr, wd
        self.seed = int(seed)
        L = _L.lib()
        h = L.ma_create(self.d, self.block, self.k, self.m, self.b, beta1, beta2, eps, lr, wd, self.seed)
        if not h:
            code, msg = _L.last_error()
            raise _L.MicroAdamError(code, msg)
        self._h = C.c_void_p(h)

    # ------------------------------------------------------------ lifecycle
    def close(self):
        if getattr(self, "_h", None):
            _L.lib().ma_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    # ------------------------------------------------------------ the step
    def step(self, params, grads, stream=None):
        """params: fp32 (4-byte elements) or bfloat16 (2-byte elements, updated
        through ma_step_bf16)."""
        _L.require(params.is_cuda and grads.is_cuda, "params and grads must be CUDA tensors")
        _L.require(params.numel() == self.d and grads.numel() == self.d,
                   f"params and grads must have d = {self.d} elements")
        _L.require(params.is_contiguous() and grads.is_contiguous(), "params and grads must be contiguous")
        _L.require(params.element_size() in (2, 4) and grads.element_size() == 2,
                   "params must be fp32 or bf16 and grads bf16 (or int16 bits)")
        fn = _L.lib().ma_step if params.element_size() == 4 else _L.lib().ma_step_bf16
        _L.check(fn(self._h, C.c_void_p(params.data_ptr()), C.c_void_p(grads.data_ptr()),
                    C.c_void_p(_stream_handle(stream))))

    # ------------------------------------------------------------ accessors
    @property
    def t(self) -> int:
        return int(_L.lib().ma_get_step(self._h))

    @property
    def num_blocks(self) -> int:
        return int(_L.lib().ma_num_blocks(self._h))

    def state_bytes(self) -> int:
        return int(_L.lib().ma_state_bytes(self._h))

    def aux_bytes(self) -> int:
        return int(_L.lib().ma_aux_bytes(self._h))

    def set_flags(self, flags: int):
        _L.check(_L.lib().ma_set_flags(self._h, int(flags)))

    def set_lr(self, lr: float):
        _L.check(_L.lib().ma_set_lr(self._h, float(lr)))
        self.lr = lr

    def set_step(self, t: int):
        _L.check(_L.lib().ma_set_step(self._h, int(t)))

    def read_state(self, which: int, offset: int, nbytes: int) -> np.ndarray:
        out = np.empty(int(nbytes), np.uint8)
        _L.check(_L.lib().ma_read_state(self._h, int(which), int(offset), int(nbytes),
                                        out.ctypes.data_as(C.c_void_p)))
        return out

    def write_state(self, which: int, offset: int, data: np.ndarray):
        data = np.ascontiguousarray(data).view(np.uint8)
        _L.check(_L.lib().ma_write_state(self._h, int(which), int(offset), data.size,
                                         data.ctypes.data_as(C.c_void_p)))

    def codes_bytes(self, offset: int = 0, nbytes: int | None = None) -> np.ndarray:
        n = (self.d + 1) // 2 - offset if nbytes is None else nbytes
        return self.read_state(_L.MA_STATE_CODES, offset, n)

    def stats(self, first_block: int = 0, nblocks: int | None = None) -> np.ndarray:
        nb = self.num_blocks - first_block if nblocks is None else nblocks
        return self.read_state(_L.MA_STATE_STATS, 8 * first_block, 8 * nb).view(np.float32)

    def window(self, offset: int = 0, n: int | None = None) -> np.ndarray:
        n = self.m * self.k - offset if n is None else n
        return self.read_state(_L.MA_STATE_WINDOW, 4 * offset, 4 * n).view(np.uint32)

    def export_state(self) -> dict:
        """The whole state (ma_export_state): codes, block statistics, window, t."""
        codes = np.empty((self.d + 1) // 2, np.uint8)
        stats = np.empty(2 * self.num_blocks, np.float32)
        window = np.empty(self.m * self.k, np.uint32)
        t = C.c_int64(0)
        _L.check(_L.lib().ma_export_state(self._h, codes.ctypes.data_as(C.c_void_p),
                                          stats.ctypes.data_as(C.c_void_p),
                                          window.ctypes.data_as(C.c_void_p) if window.size else None,
                                          C.byref(t)))
        return {"codes": codes, "stats": stats, "window": window, "t": int(t.value)}

    def import_state(self, st: dict):
        """Restores a state from export_state (ma_import_state)."""
        codes = np.ascontiguousarray(st["codes"], np.uint8)
        stats = np.ascontiguousarray(st["stats"], np.float32)
        window = np.ascontiguousarray(st["window"], np.uint32)
        _L.require(codes.size == (self.d + 1) // 2 and stats.size == 2 * self.num_blocks
                   and window.size == self.m * self.k, "state buffers of the wrong size")
        _L.check(_L.lib().ma_import_state(self._h, codes.ctypes.data_as(C.c_void_p),
                                          stats.ctypes.data_as(C.c_void_p),
                                          window.ctypes.data_as(C.c_void_p) if window.size else None,
                                          int(st["t"])))

    def moments(self, blocks, stream=None):
        """(m_hat, v_hat) of the last step for the given blocks, as CUDA
        tensors of shape [len(blocks), block]."""
        import torch
        blocks = np.ascontiguousarray(blocks, dtype=np.int64)
        mh = torch.empty((blocks.size, self.block), dtype=torch.float32, device="cuda")
        vh = torch.empty_like(mh)
        _L.check(_L.lib().ma_debug_moments(self._h, blocks.ctypes.data_as(C.c_void_p), blocks.size,
                                           C.c_void_p(mh.data_ptr()), C.c_void_p(vh.data_ptr()),
                                           C.c_void_p(_stream_handle(stream))))
        return mh, vh

    def residual(self, grads, blocks, stream=None):
        """The accumulator a_t = g_t + Q^-1(e_t) the next step would start
        from, for the given blocks and gradients (bf16 or int16 bits, CUDA),
        as a CUDA tensor of shape [len(blocks), block]; the state is not
        changed."""
        import torch
        _L.require(grads.is_cuda and grads.is_contiguous() and grads.numel() == self.d and grads.element_size() == 2,
                   f"grads must be a contiguous bf16 CUDA tensor of d = {self.d} elements")
        blocks = np.ascontiguousarray(blocks, dtype=np.int64)
        out = torch.empty((blocks.size, self.block), dtype=torch.float32, device="cuda")
        _L.check(_L.lib().ma_debug_residual(self._h, C.c_void_p(grads.data_ptr()), blocks.ctypes.data_as(C.c_void_p),
                                            blocks.size, C.c_void_p(out.data_ptr()),
                                            C.c_void_p(_stream_handle(stream))))
        return out

    def set_timing(self, on: bool):
        _L.check(_L.lib().ma_set_timing(self._h, 1 if on else 0))

    def kernel_times(self):
        """{'compress': (ms_total, launches), 'adamstats_apply': (...), 'step_fused': (...)}"""
        ms = (C.c_double * 3)()
        n = (C.c_int64 * 3)()
        _L.check(_L.lib().ma_kernel_times(self._h, ms, n, 3))
        return {"compress": (ms[0], n[0]), "adamstats_apply": (ms[1], n[1]), "step_fused": (ms[2], n[2])}

    def set_pipeline(self, chunks: int):
        """Number of block ranges whose update overlaps the next range's
        compression (1 = no overlap)."""
        _L.check(_L.lib().ma_set_pipeline(self._h, int(chunks)))

    @property
    def pipeline(self) -> int:
        """Block ranges the step uses (1: no overlap)."""
        return int(_L.lib().ma_get_pipeline(self._h))

    def set_count_touched(self, on: bool):
        _L.check(_L.lib().ma_set_count_touched(self._h, 1 if on else 0))

    def touched_count(self) -> int:
        """Touched parameters summed over the steps since set_count_touched(True)."""
        return int(_L.lib().ma_touched_count(self._h))
