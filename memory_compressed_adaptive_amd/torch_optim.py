"""torch.optim front end: MicroAdam over ordinary parameter groups.

Each parameter group is packed into one flat device buffer (fp32, or bfloat16
when the group's parameters are bfloat16), and every parameter's storage is
replaced by a view of that buffer, so the model and the optimizer share the
memory.  At each step the group's gradients are gathered into a flat bfloat16
buffer (torch's round-to-nearest-even conversion) and one libmicroadam handle
runs the whole MicroAdam step on it (page "MicroAdam (Sparse-Gradient Adaptive
Optimization with Quantized Error Feedback)", first paragraph).  The flat order
is the order of the group's parameter list; blocks of B_d ignore tensor
boundaries.  A parameter without a gradient contributes zeros.
"""
from __future__ import annotations

import torch

from .optimizer import MicroAdam as _Handle


class MicroAdamW(torch.optim.Optimizer):
    """MicroAdam with decoupled weight decay.

    density: Top-k fraction (k = floor(density * d), the page's k = d/100 by
    default); m: window rows; block: B_d.  Hyperparameters are per group; lr
    may be changed between steps (param_groups[i]["lr"]).
    """

    def __init__(self, params, lr=1e-4, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0,
                 density=0.01, m=10, block=16384, seed=42):
        defaults = dict(lr=lr, betas=betas, eps=eps, weight_decay=weight_decay, density=density,
                        m=m, block=block, seed=seed)
        super().__init__(params, defaults)
        for gi, group in enumerate(self.param_groups):
            ps = group["params"]
            if not ps:
                continue
            dev = ps[0].device
            dt = ps[0].dtype
            if dev.type != "cuda":
                raise ValueError("MicroAdamW needs CUDA (HIP) parameters")
            if any(p.device != dev or p.dtype != dt for p in ps):
                raise ValueError("the parameters of one group must share device and dtype")
            if dt not in (torch.float32, torch.bfloat16):
                raise ValueError("parameters must be float32 or bfloat16")
            d = sum(p.numel() for p in ps)
            flat = torch.empty(d, dtype=dt, device=dev)
            off = 0
            for p in ps:
                n = p.numel()
                flat[off:off + n].copy_(p.detach().reshape(-1))
                p.data = flat[off:off + n].view_as(p)
                off += n
            k = int(d * group["density"])
            b1, b2 = group["betas"]
            h = _Handle(d, block=group["block"], k=k, m=group["m"], beta1=b1, beta2=b2, eps=group["eps"],
                        lr=group["lr"], wd=group["weight_decay"], seed=group["seed"] + gi)
            group["_flat"] = flat
            group["_gflat"] = torch.empty(d, dtype=torch.bfloat16, device=dev)
            group["_handle"] = h
            group["_lr_set"] = group["lr"]

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        for group in self.param_groups:
            if "_handle" not in group:
                continue
            h = group["_handle"]
            if group["lr"] != group["_lr_set"]:
                h.set_lr(group["lr"])
                group["_lr_set"] = group["lr"]
            gflat = group["_gflat"]
            off = 0
            for p in group["params"]:
                n = p.numel()
                if p.grad is None:
                    gflat[off:off + n].zero_()
                else:
                    gflat[off:off + n].copy_(p.grad.reshape(-1))
                off += n
            flat = group["_flat"]
            h.step(flat if flat.dtype == torch.float32 else flat.view(torch.int16), gflat.view(torch.int16))
        return loss

    def state_dict(self):
        sd = super().state_dict()
        sd["microadam"] = [g["_handle"].export_state() if "_handle" in g else None for g in self.param_groups]
        for g in sd["param_groups"]:
            for key in ("_flat", "_gflat", "_handle", "_lr_set"):
                g.pop(key, None)
        return sd

    def load_state_dict(self, state_dict):
        saved = state_dict.get("microadam", [])
        groups = [dict(g) for g in state_dict["param_groups"]]
        keep = [{k: g[k] for k in ("_flat", "_gflat", "_handle", "_lr_set") if k in g} for g in self.param_groups]
        super().load_state_dict({"state": state_dict["state"], "param_groups": groups})
        for g, extra, st in zip(self.param_groups, keep, saved):
            g.update(extra)
            if st is not None:
                g["_handle"].import_state(st)
