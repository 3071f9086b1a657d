"""Synthetic workloads: model-shaped flat parameter sets and seeded gradients.

The MicroAdam page's experiments fine-tune BERT, OPT and LLaMA-2 models; no
datasets or weights are used here.  Each workload is a flat fp32 parameter
vector with the tensor list of the named model (per layer q, k, v, o, then the
feed-forward matrices, then the embedding and, for LLaMA-2, the head; rows
concatenated in that order) and bf16 gradients drawn per step:

  tiny        one tensor of 2^20;  N(0, 1e-3), each entry x50 with prob. 0.01
  bert_base   12 x [4 x 768^2, 768x3072, 3072x768] + 30522x768;
              1e-3 * Student-t(3)
  opt_1_3b    24 x [4 x 2048^2, 2048x8192, 8192x2048] + 50272x2048;
              N(0, s_T), s_T = 10^U(-5,-2) once per tensor
  llama2_7b   32 x [4 x 4096^2, 3 x 4096x11008] + 2 x 32000x4096;
              s_T * Student-t(3), s_T = 10^U(-4,-2) once per tensor
  llama2_13b  40 x [4 x 5120^2, 3 x 5120x13824] + 2 x 32000x5120; as llama2_7b

Parameters ~ N(0, 0.02) with seed 1; gradients of step t use seed 1000 with t
as a counter word; per-tensor scales come from numpy's PCG64 seeded 2024.
All values are produced on the GPU by libmasynth (Philox4x32-10 + Box-Muller).
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmasynth.so")

PARAM_SEED = 1
GRAD_SEED = 1000
SCALE_SEED = 2024
KIND_GAUSS, KIND_STUDENT_T = 0, 1


@dataclass(frozen=True)
class Workload:
    name: str
    tensors: tuple          # ((name, numel), ...)
    kind: int
    scale_lo: float         # log10 range of the per-tensor scale (lo == hi: fixed)
    scale_hi: float
    p_outlier: float
    outlier_mult: float
    m: int
    steps: int
    block: int = 16384

    @property
    def d(self) -> int:
        return sum(n for _, n in self.tensors)

    @property
    def k(self) -> int:
        return self.d // 100

    def segments(self):
        ends = np.cumsum([n for _, n in self.tensors]).astype(np.int64)
        if self.scale_lo == self.scale_hi:
            scales = np.full(len(self.tensors), 10.0 ** self.scale_lo, np.float32)
        else:
            rng = np.random.default_rng(SCALE_SEED)
            scales = (10.0 ** rng.uniform(self.scale_lo, self.scale_hi, len(self.tensors))).astype(np.float32)
        return ends, scales


def _layers(n_layers, h, ff, swiglu):
    out = []
    for layer in range(n_layers):
        for nm in ("q", "k", "v", "o"):
            out.append((f"l{layer}.{nm}", h * h))
        if swiglu:
            out += [(f"l{layer}.gate", h * ff), (f"l{layer}.up", h * ff), (f"l{layer}.down", ff * h)]
        else:
            out += [(f"l{layer}.up", h * ff), (f"l{layer}.down", ff * h)]
    return out


WORKLOADS = {
    "tiny": Workload("tiny", (("flat", 2 ** 20),), KIND_GAUSS, -3.0, -3.0, 0.01, 50.0, 10, 20),
    "bert_base": Workload("bert_base", tuple(_layers(12, 768, 3072, False) + [("embed", 30522 * 768)]),
                          KIND_STUDENT_T, -3.0, -3.0, 0.0, 1.0, 10, 50),
    "opt_1_3b": Workload("opt_1_3b", tuple(_layers(24, 2048, 8192, False) + [("embed", 50272 * 2048)]),
                         KIND_GAUSS, -5.0, -2.0, 0.0, 1.0, 10, 20),
    "llama2_7b": Workload("llama2_7b", tuple(_layers(32, 4096, 11008, True) +
                                             [("embed", 32000 * 4096), ("head", 32000 * 4096)]),
                          KIND_STUDENT_T, -4.0, -2.0, 0.0, 1.0, 10, 10),
    "llama2_13b": Workload("llama2_13b", tuple(_layers(40, 5120, 13824, True) +
                                               [("embed", 32000 * 5120), ("head", 32000 * 5120)]),
                           KIND_STUDENT_T, -4.0, -2.0, 0.0, 1.0, 10, 5),
}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m memory_compressed_adaptive_amd.build`")
        L = C.CDLL(LIB_PATH)
        p, i64, u64, f32 = C.c_void_p, C.c_int64, C.c_uint64, C.c_float
        L.masyn_normal_f32.restype = C.c_int
        L.masyn_normal_f32.argtypes = [p, i64, u64, f32, f32, p]
        L.masyn_grads_bf16.restype = C.c_int
        L.masyn_grads_bf16.argtypes = [p, i64, u64, i64, C.c_int, p, p, C.c_int, f32, f32, p]
        L.masyn_copy_f32.restype = C.c_int
        L.masyn_copy_f32.argtypes = [p, p, i64, p]
        _lib = L
    return _lib


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(int(s.cuda_stream))


def fill_params(theta, seed: int = PARAM_SEED, mean: float = 0.0, std: float = 0.02, stream=None):
    rc = lib().masyn_normal_f32(C.c_void_p(theta.data_ptr()), theta.numel(), seed, mean, std, _stream(stream))
    if rc:
        raise RuntimeError(f"masyn_normal_f32 failed ({rc})")


class GradSource:
    """Device-side gradient generator for one workload (segment table on the GPU)."""

    def __init__(self, w: Workload, seed: int = GRAD_SEED):
        import torch
        ends, scales = w.segments()
        self.w = w
        self.seed = seed
        self.ends = torch.from_numpy(ends).cuda()
        self.scales = torch.from_numpy(scales).cuda()

    def fill(self, g, step: int, stream=None):
        w = self.w
        rc = lib().masyn_grads_bf16(C.c_void_p(g.data_ptr()), g.numel(), self.seed, int(step), w.kind,
                                    C.c_void_p(self.ends.data_ptr()), C.c_void_p(self.scales.data_ptr()),
                                    int(self.ends.numel()), w.p_outlier, w.outlier_mult, _stream(stream))
        if rc:
            raise RuntimeError(f"masyn_grads_bf16 failed ({rc})")


def copy_f32(dst, src, stream=None):
    rc = lib().masyn_copy_f32(C.c_void_p(dst.data_ptr()), C.c_void_p(src.data_ptr()), src.numel(), _stream(stream))
    if rc:
        raise RuntimeError(f"masyn_copy_f32 failed ({rc})")


def sample_blocks(n_b: int, every: int = 397):
    """Deterministic block sample: every `every`-th block plus the first and last."""
    js = set(range(0, n_b, every)) | {0, n_b - 1}
    return np.array(sorted(js), np.int64)
