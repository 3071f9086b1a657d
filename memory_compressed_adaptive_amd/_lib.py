"""ctypes binding of libmicroadam (C ABI in include/microadam.h).

Argument marshalling only: every stage of the step runs in the HIP kernels of
the library.  If the library is missing the import fails loudly; there is no
CPU fallback.
"""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmicroadam.so")

MA_OK = 0
MA_EINVAL = -1
MA_EUNSUPPORTED = -2
MA_ENOMEM = -3
MA_EHIP = -4

MA_FLAG_NO_EF = 1
MA_FLAG_FORCE_DENSE = 4
MA_FLAG_FORCE_SPARSE = 8
MA_FLAG_UNFUSED = 16
MA_FLAG_ROW_SUMS = 64
MA_FLAG_GLOBAL_QUANT = 32

MA_STATE_CODES = 0
MA_STATE_STATS = 1
MA_STATE_WINDOW = 2

# every symbol include/microadam.h declares
EXPORTS = (
    "ma_create", "ma_step", "ma_step_bf16", "ma_step_noalloc", "ma_adamw_step", "ma_adamw8_step", "ma_state_bytes", "ma_aux_bytes", "ma_destroy", "ma_last_error",
    "ma_last_error_message", "ma_get_step", "ma_num_blocks", "ma_set_step", "ma_set_flags",
    "ma_set_lr", "ma_read_state", "ma_write_state", "ma_export_state", "ma_import_state", "ma_debug_moments", "ma_debug_residual", "ma_set_timing",
    "ma_kernel_times", "ma_set_pipeline", "ma_get_pipeline", "ma_set_count_touched", "ma_touched_count",
)

_lib = None


class MicroAdamError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libmicroadam error {code}: {msg}")
        self.code = code


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m memory_compressed_adaptive_amd.build` "
                          "(or __graft_entry__.build())")
    L = C.CDLL(LIB_PATH)
    p, i32, i64, u32, u64, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32, C.c_uint64, C.c_float
    L.ma_create.restype = p
    L.ma_create.argtypes = [i64, i32, i64, i32, i32, f32, f32, f32, f32, f32, u64]
    L.ma_step.restype = C.c_int
    L.ma_step.argtypes = [p, p, p, p]
    L.ma_adamw_step.restype = C.c_int
    L.ma_adamw_step.argtypes = [i64, i64, f32, f32, f32, f32, f32, p, p, p, p, p]
    L.ma_adamw8_step.restype = C.c_int
    L.ma_adamw8_step.argtypes = [i64, i64, f32, f32, f32, f32, f32, p, p, p, p, p, p, p]
    L.ma_step_bf16.restype = C.c_int
    L.ma_step_bf16.argtypes = [p, p, p, p]
    L.ma_step_noalloc.restype = C.c_int
    L.ma_step_noalloc.argtypes = [p, p, p, p]
    L.ma_state_bytes.restype = C.c_size_t
    L.ma_state_bytes.argtypes = [p]
    L.ma_aux_bytes.restype = C.c_size_t
    L.ma_aux_bytes.argtypes = [p]
    L.ma_destroy.restype = None
    L.ma_destroy.argtypes = [p]
    L.ma_last_error.restype = C.c_int
    L.ma_last_error.argtypes = []
    L.ma_last_error_message.restype = C.c_char_p
    L.ma_last_error_message.argtypes = []
    L.ma_get_step.restype = i64
    L.ma_get_step.argtypes = [p]
    L.ma_num_blocks.restype = i64
    L.ma_num_blocks.argtypes = [p]
    L.ma_set_step.restype = C.c_int
    L.ma_set_step.argtypes = [p, i64]
    L.ma_set_flags.restype = C.c_int
    L.ma_set_flags.argtypes = [p, u32]
    L.ma_set_lr.restype = C.c_int
    L.ma_set_lr.argtypes = [p, f32]
    L.ma_read_state.restype = C.c_int
    L.ma_read_state.argtypes = [p, C.c_int, u64, u64, p]
    L.ma_write_state.restype = C.c_int
    L.ma_write_state.argtypes = [p, C.c_int, u64, u64, p]
    L.ma_export_state.restype = C.c_int
    L.ma_export_state.argtypes = [p, p, p, p, C.POINTER(i64)]
    L.ma_import_state.restype = C.c_int
    L.ma_import_state.argtypes = [p, p, p, p, i64]
    L.ma_debug_moments.restype = C.c_int
    L.ma_debug_moments.argtypes = [p, p, i64, p, p, p]
    L.ma_debug_residual.restype = C.c_int
    L.ma_debug_residual.argtypes = [p, p, p, i64, p, p]
    L.ma_set_timing.restype = C.c_int
    L.ma_set_timing.argtypes = [p, C.c_int]
    L.ma_kernel_times.restype = C.c_int
    L.ma_kernel_times.argtypes = [p, p, p, C.c_int]
    L.ma_set_pipeline.restype = C.c_int
    L.ma_set_pipeline.argtypes = [p, C.c_int]
    L.ma_get_pipeline.restype = C.c_int
    L.ma_get_pipeline.argtypes = [p]
    L.ma_set_count_touched.restype = C.c_int
    L.ma_set_count_touched.argtypes = [p, C.c_int]
    L.ma_touched_count.restype = i64
    L.ma_touched_count.argtypes = [p]
    _lib = L
    return L


def last_error():
    L = lib()
    return int(L.ma_last_error()), (L.ma_last_error_message() or b"").decode()


def check(rc: int):
    if rc != MA_OK:
        code, msg = last_error()
        raise MicroAdamError(rc, msg)
    return rc


def require(ok: bool, what: str) -> None:
    """An argument check of the binding, raised as ValueError (unlike an
    assert it also holds under python -O)."""
    if not ok:
        raise ValueError(what)
