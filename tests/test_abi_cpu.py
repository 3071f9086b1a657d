"""CPU-side checks of the C ABI: the built library loads, exports every symbol
include/microadam.h declares, and rejects invalid arguments with the
documented codes before touching any device.  No compute calls."""
import ctypes as C
import os
import re

import pytest

from memory_compressed_adaptive_amd import _lib as L
from memory_compressed_adaptive_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared(header):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ma[a-z]*_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared("microadam.h")
    assert len(names) >= 15
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTS)


def test_synth_library_loads():
    lib = synth.lib()
    for n in ("masyn_normal_f32", "masyn_grads_bf16", "masyn_copy_f32"):
        assert hasattr(lib, n)


@pytest.mark.parametrize("args,code", [
    ((0, 16384, 0, 10, 4, 0.9, 0.999, 1e-8, 1e-4, 0.0, 42), L.MA_EINVAL),        # d < 1
    ((100, 0, 1, 10, 4, 0.9, 0.999, 1e-8, 1e-4, 0.0, 42), L.MA_EINVAL),          # B_d < 1
    ((100, 32767, 1, 10, 4, 0.9, 0.999, 1e-8, 1e-4, 0.0, 42), L.MA_EINVAL),      # B_d >= 2^15 - 1
    ((100, 64, 101, 10, 4, 0.9, 0.999, 1e-8, 1e-4, 0.0, 42), L.MA_EINVAL),       # k > d
    ((100, 64, -1, 10, 4, 0.9, 0.999, 1e-8, 1e-4, 0.0, 42), L.MA_EINVAL),        # k < 0
    ((100, 64, 1, 0, 4, 0.9, 0.999, 1e-8, 1e-4, 0.0, 42), L.MA_EINVAL),          # m < 1
    ((100, 64, 1, 10, 4, 1.0, 0.999, 1e-8, 1e-4, 0.0, 42), L.MA_EINVAL),         # beta1 = 1
    ((100, 64, 1, 10, 4, 0.9, -0.1, 1e-8, 1e-4, 0.0, 42), L.MA_EINVAL),          # beta2 < 0
    ((100, 64, 1, 10, 4, 0.9, 0.999, 0.0, 1e-4, 0.0, 42), L.MA_EINVAL),          # eps = 0
    ((100, 64, 1, 10, 4, 0.9, 0.999, 1e-8, float("nan"), 0.0, 42), L.MA_EINVAL),  # lr NaN
    ((100, 64, 1, 10, 4, 0.9, 0.999, 1e-8, 1e-4, -1.0, 42), L.MA_EINVAL),        # wd < 0
    ((100, 64, 1, 10, 8, 0.9, 0.999, 1e-8, 1e-4, 0.0, 42), L.MA_EUNSUPPORTED),   # b = 8
    ((100, 64, 1, 10, 2, 0.9, 0.999, 1e-8, 1e-4, 0.0, 42), L.MA_EUNSUPPORTED),   # b = 2
    ((100, 64, 1, 1025, 4, 0.9, 0.999, 1e-8, 1e-4, 0.0, 42), L.MA_EUNSUPPORTED),  # m > 1024
])
def test_create_rejects_invalid_arguments(args, code):
    lib = L.lib()
    h = lib.ma_create(*args)
    assert not h
    got, msg = L.last_error()
    assert got == code and msg


def test_null_handles_are_safe():
    lib = L.lib()
    assert lib.ma_state_bytes(None) == 0
    assert lib.ma_aux_bytes(None) == 0
    lib.ma_destroy(None)
    assert lib.ma_get_step(None) == -1
    assert lib.ma_step(None, None, None, None) == L.MA_EINVAL
    assert lib.ma_set_flags(None, 0) == L.MA_EINVAL
    assert lib.ma_read_state(None, 0, 0, 0, None) == L.MA_EINVAL
    assert lib.ma_export_state(None, None, None, None, None) == L.MA_EINVAL
    assert lib.ma_import_state(None, None, None, None, 0) == L.MA_EINVAL
    assert lib.ma_kernel_times(None, None, None, 0) == L.MA_EINVAL
    assert lib.ma_set_pipeline(None, 4) == L.MA_EINVAL
    assert lib.ma_debug_residual(None, None, None, 0, None, None) == L.MA_EINVAL
    assert lib.ma_debug_moments(None, None, 0, None, None, None) == L.MA_EINVAL
    assert lib.ma_get_pipeline(None) == -1


def test_adamw_argument_checks_without_gpu():
    lib = L.lib()
    assert lib.ma_adamw_step(-1, 1, 0.9, 0.999, 1e-8, 1e-3, 0.0, None, None, None, None, None) == L.MA_EINVAL
    assert lib.ma_adamw_step(10, 0, 0.9, 0.999, 1e-8, 1e-3, 0.0, None, None, None, None, None) == L.MA_EINVAL
    assert lib.ma_adamw_step(0, 1, 0.9, 0.999, 1e-8, 1e-3, 0.0, None, None, None, None, None) == L.MA_OK
    assert lib.ma_adamw_step(10, 1, 0.9, 0.999, 1e-8, 1e-3, 0.0, None, None, None, None, None) == L.MA_EINVAL


def test_adamw8_argument_checks_without_gpu():
    lib = L.lib()
    args = (0.9, 0.999, 1e-8, 1e-3, 0.0)
    assert lib.ma_adamw8_step(-1, 1, *args, None, None, None, None, None, None, None) == L.MA_EINVAL
    assert lib.ma_adamw8_step(0, 1, *args, None, None, None, None, None, None, None) == L.MA_OK
    assert lib.ma_adamw8_step(5, 1, *args, None, None, None, None, None, None, None) == L.MA_EINVAL
