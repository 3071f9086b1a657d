"""The page's comparison optimizer on the same device path: fp32 AdamW (8 bytes
of state per parameter, second paragraph of the MicroAdam page), one step per
call of ma_adamw_step in libmicroadam."""
from __future__ import annotations

import ctypes as C

from . import _lib as _L


def adamw_step(theta, grads, m, v, t: int, beta1=0.9, beta2=0.999, eps=1e-8, lr=1e-4, wd=0.0, stream=None):
    """theta, m, v: contiguous fp32 CUDA tensors of n elements (in place);
    grads: bf16 (or int16 bit pattern) CUDA tensor of n elements; t >= 1."""
    import torch
    n = theta.numel()
    for x in (theta, m, v):
        assert x.is_cuda and x.is_contiguous() and x.numel() == n and x.element_size() == 4
    assert grads.is_cuda and grads.is_contiguous() and grads.numel() == n and grads.element_size() == 2
    s = stream if stream is not None else torch.cuda.current_stream()
    _L.check(_L.lib().ma_adamw_step(n, int(t), beta1, beta2, eps, lr, wd, C.c_void_p(theta.data_ptr()),
                                    C.c_void_p(grads.data_ptr()), C.c_void_p(m.data_ptr()),
                                    C.c_void_p(v.data_ptr()), C.c_void_p(int(s.cuda_stream))))
