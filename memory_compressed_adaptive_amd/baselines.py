"""The page's comparison optimizers on the same device path (second paragraph
of the MicroAdam page): fp32 AdamW (8 bytes of state per parameter, one call
of ma_adamw_step) and 8-bit block-quantized AdamW (2 bytes plus 8 per 256
parameters, ma_adamw8_step)."""
from __future__ import annotations

import ctypes as C

from . import _lib as _L


def adamw_step(theta, grads, m, v, t: int, beta1=0.9, beta2=0.999, eps=1e-8, lr=1e-4, wd=0.0, stream=None):
    """theta, m, v: contiguous fp32 CUDA tensors of n elements (in place);
    grads: bf16 (or int16 bit pattern) CUDA tensor of n elements; t >= 1."""
    import torch
    n = theta.numel()
    for x in (theta, m, v):
        _L.require(x.is_cuda and x.is_contiguous() and x.numel() == n and x.element_size() == 4,
                   "theta, m and v must be contiguous fp32 CUDA tensors of one length")
    _L.require(grads.is_cuda and grads.is_contiguous() and grads.numel() == n and grads.element_size() == 2,
               "grads must be a contiguous bf16 CUDA tensor of theta's length")
    s = stream if stream is not None else torch.cuda.current_stream()
    _L.check(_L.lib().ma_adamw_step(n, int(t), beta1, beta2, eps, lr, wd, C.c_void_p(theta.data_ptr()),
                                    C.c_void_p(grads.data_ptr()), C.c_void_p(m.data_ptr()),
                                    C.c_void_p(v.data_ptr()), C.c_void_p(int(s.cuda_stream))))


Q8_BLOCK = 256


def adamw8_step(theta, grads, cm, cv, sm, sr, t: int, beta1=0.9, beta2=0.999, eps=1e-8, lr=1e-4, wd=0.0,
                stream=None):
    """theta fp32, grads bf16/int16, cm int8, cv uint8 (n elements each), sm and
    sr fp32 (ceil(n/256) each), all contiguous CUDA tensors; t >= 1."""
    import torch
    n = theta.numel()
    nq = -(-n // Q8_BLOCK)
    ts = (theta, grads, cm, cv, sm, sr)
    _L.require(all(x.is_cuda and x.is_contiguous() for x in ts), "every tensor must be a contiguous CUDA tensor")
    _L.require(theta.element_size() == 4, "theta must be fp32")
    _L.require(grads.numel() == n and grads.element_size() == 2, "grads must be bf16 of theta's length")
    _L.require(cm.numel() == n and cv.numel() == n and cm.element_size() == 1 and cv.element_size() == 1,
               "cm and cv must be 8-bit codes of theta's length")
    _L.require(sm.numel() == nq and sr.numel() == nq and sm.element_size() == 4 and sr.element_size() == 4,
               f"sm and sr must be fp32 scales, one per {Q8_BLOCK} parameters")
    s = stream if stream is not None else torch.cuda.current_stream()
    _L.check(_L.lib().ma_adamw8_step(n, int(t), beta1, beta2, eps, lr, wd, C.c_void_p(theta.data_ptr()),
                                     C.c_void_p(grads.data_ptr()), C.c_void_p(cm.data_ptr()),
                                     C.c_void_p(cv.data_ptr()), C.c_void_p(sm.data_ptr()),
                                     C.c_void_p(sr.data_ptr()), C.c_void_p(int(s.cuda_stream))))
